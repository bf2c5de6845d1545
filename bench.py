#!/usr/bin/env python3
"""Benchmark: 16-layer hybrid backbone forward on one MI355X.

Workload: 160 users of 1000..2000 tokens (70 % H, 20 % R, 10 % T), d_model
512, 8 query / 2 KV heads, head_dim 64, bf16 storage with fp32 accumulation,
4 blocks of (1 full-attention + 3 target-attention) layers; seeded synthetic
inputs (the pages' production logs are private).  One step = building the
mask metadata for the batch + the whole 16-layer forward, in place on X (each
step consumes the previous step's output; every step does the full work).

Prints ONE JSON line on stdout: user-samples/s, the full-attention kernel's
achieved masked TFLOP/s against the bf16 MFMA peak (its duration measured with
HIP events on its own launch stream inside the timed region), a per-kernel
breakdown from a second, separately timed pass, and the CPU oracle timed on a
bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(n_rows_meta, lens, split):
    """Sum of n_i over full-layer rows and over T rows (from the device metadata)."""
    import numpy as np
    n = n_rows_meta
    off = np.concatenate([[0], np.cumsum(lens[:, 0] + lens[:, 1] + split * lens[:, 2])])
    lc = lens[:, 0] + lens[:, 1]
    t_sum = sum(int(n[off[u] + lc[u]:off[u + 1]].sum()) for u in range(len(lens)))
    return int(n.sum()), t_sum


def computed_pairs(tiles, p, n, gperm=None):
    """(query, key) pairs per head that the bf16 attention kernel computes over one layer's tile
    list, and the visible pairs sum(n_i) of the same rows.

    Follows the kernel's own walk: per 32-row slice of a tile, the key tiles of 64 from the user's
    aligned first row up to the slice's largest visible prefix; tiles below its smallest prefix run
    both 32-key blocks, the others skip a block no row of the slice sees; every block computes 32
    rows x 32 keys (rows past the tile's end included); a T row's own key is one more pair.
    """
    import numpy as np
    comp = vis = 0
    for u, row0, nr, _fe, _end, grow0, qrow0, urow0 in tiles.tolist():
        for s in (0, 1):
            m = min(32, nr - 32 * s)
            if m <= 0:
                continue
            q0 = qrow0 + 32 * s
            gi = gperm[q0:q0 + m] if gperm is not None else np.arange(grow0 + 32 * s, grow0 + 32 * s + m)
            pl, nl = p[gi], n[gi]
            vis += int(nl.sum())
            comp += int((nl - pl).sum())
            pmax, pmin = int(pl.max()), int(pl.min())
            if pmax <= 0:
                continue
            t0, kz, kf = urow0 & ~63, urow0 + pmax, urow0 + pmin
            n_main = (kz - t0 + 63) >> 6
            n_un = n_main if kf >= kz else min(n_main, max(kf - t0, 0) >> 6)
            blocks = 2 * n_un
            for it in range(n_un, n_main):
                ts = t0 + 64 * it
                lo, lim_hi = max(urow0 - ts, 0), kz - ts
                blocks += sum(1 for b0 in (0, 32) if not (lo >= b0 + 32 or lim_hi <= b0))
            comp += 32 * 32 * blocks
    return comp, vis


def recorded_traffic():
    """HBM bytes per launch of the full-layer attention kernel from the committed PMC summary.

    The summary records the hash of the kernel source it was measured on; a
    different source means the figure no longer applies (None).
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_full_cfg3_hbm_traffic.md")
    try:
        fields = dict(l.split(": ", 1) for l in open(path).read().splitlines() if ": " in l and not l.startswith("|"))
        src = open(os.path.join(ROOT, fields["kernel_source"].strip()), "rb").read()
        if hashlib.sha256(src).hexdigest() != fields["kernel_source_sha256"].strip():
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(wl, seconds: float):
    """Oracle backbone (float64 numpy) on users of the batch until `seconds` pass."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import model as om
    r = om.bf16_round
    full = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl.full]
    tgt = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl.target]
    t0 = time.perf_counter()
    done = 0
    while True:
        om.backbone(wl.batch, wl.x, full, tgt, wl.dims, wl.n_blocks, wl.k_target, boundary=r, users=[done])
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= wl.batch.n_users:
            break
    threads = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = int(max(threads)) if threads else 1
    return {"value": done / el, "unit": "user-samples/s", "cores": cores, "kind": "oracle",
            "sample": f"first {done} of {wl.batch.n_users} users, 16-layer backbone forward, float64 numpy, "
                      f"{el:.1f} s", "cpu": cpu_model()}


def oracle_rate(fn, n_users: int, seconds: float, what: str):
    """Time fn(u) (the oracle on user u) on users 0, 1, ... until `seconds` pass."""
    t0 = time.perf_counter()
    done = 0
    while True:
        fn(done)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= n_users:
            break
    return {"value": done / el, "unit": "user-samples/s", "kind": "oracle",
            "sample": f"first {done} of {n_users} users, {what}, float64 numpy, {el:.1f} s"}


def blas_threads():
    from threadpoolctl import threadpool_info
    threads = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return int(max(threads)) if threads else 1
def time_launches(fn, n, torch):
    """Mean milliseconds of fn() over n back-to-back calls on the current stream (events around them)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def config_sections(args, B, torch, synth, np):
    """Configs 1, 2 (split 1 and 4) and 4 in their own launch shapes, each with the oracle timed beside it."""
    from hybrid_masked_attention_amd.tensors import DeviceWorkload, to_device
    from oracle import grad as og
    from oracle import model as om
    n = args.config_steps
    out = {}
    r = om.bf16_round

    def rw(w):
        return {k: (v if k.startswith("ln") else r(v)) for k, v in w.items()}

    def flops_bytes(wl, lay, meta, kind):
        views = B.meta_views(meta, lay, wl.batch.n_users)
        nn = views["n"].cpu().numpy().astype(np.int64)
        pf, pt = visible_pairs(nn, wl.batch.lens.astype(np.int64), wl.batch.split)
        d = wl.dims
        hd, gd, D = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim, d.d_model
        R, T = lay.n_rows, lay.n_t_rows
        if kind == "full":
            return 4.0 * d.head_dim * d.n_q_heads * pf, 2.0 * R * D * (2 * hd + 2 * gd) + 2.0 * R * hd * D, None
        attn = 4.0 * d.head_dim * d.n_q_heads * pt
        proj = 2.0 * R * D * 2 * gd + 2.0 * T * D * 2 * hd + 2.0 * T * hd * D
        return attn, proj, 2.0 * (R * 2 * gd + 2 * T * hd)

    def layer_case(wl, kind, label):
        dw = DeviceWorkload(wl)
        lay = B.meta_layout(dw.batch)
        meta = B.mask_build(dw.batch)
        op = B.OP_FULL if kind == "full" else B.OP_TARGET
        ws = B.workspace(dw.batch, dw.dims, op)
        x_out = torch.empty_like(dw.x)
        fn = B.attn_full if kind == "full" else B.attn_target
        w = dw.full[0] if kind == "full" else dw.target[0]
        run = lambda: fn(dw.batch, dw.dims, meta, w, dw.x, x_out, ws)
        for _ in range(3):
            run()
        layer_ms = time_launches(run, n, torch)
        kc = B.K_ATTN_FULL if kind == "full" else B.K_ATTN_TARGET
        B.timing_enable([kc])
        B.timing_read(kc)
        for _ in range(n):
            run()
        torch.cuda.synchronize()
        B.timing_enable([])
        cnt, ms = B.timing_read(kc)
        attn_ms = ms / max(1, cnt)
        attn, proj, abytes = flops_bytes(wl, lay, meta, kind)
        res = {"rows": int(lay.n_rows), "t_rows": int(lay.n_t_rows), "launches": n,
               "layer_us": 1000.0 * layer_ms, "attn_us": 1000.0 * attn_ms,
               "layer_masked_TFLOPs": (attn + proj) / (layer_ms * 1e-3) / 1e12,
               "attn_TFLOPs": attn / (attn_ms * 1e-3) / 1e12}
        res["layer_mfma_frac"] = res["layer_masked_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
        if abytes is not None:
            res["attn_GBs"] = abytes / (attn_ms * 1e-3) / 1e9
            res["attn_hbm_frac"] = res["attn_GBs"] / HBM_PEAK_GBS
            res["attn_bytes"] = abytes
        if not args.no_cpu_baseline:
            xr = r(wl.x)
            wr = rw(wl.full[0] if kind == "full" else wl.target[0])
            ofn = om.full_layer if kind == "full" else om.target_layer

            def one(u):
                rows = wl.batch.rows_of([u])
                ofn(wl.batch.subset([u]), xr[rows], wr, wl.dims)
            rate = oracle_rate(one, wl.batch.n_users, 4.0, f"one {kind} layer (oracle.model)")
            rate["ms_per_layer_batch"] = 1000.0 * wl.batch.n_users / rate["value"]
            rate["cores"] = blas_threads()
            res["cpu_oracle"] = rate
            if label == "config1":
                from threadpoolctl import threadpool_limits
                with threadpool_limits(1):
                    one1 = oracle_rate(one, wl.batch.n_users, 4.0, f"one {kind} layer (oracle.model), 1 thread")
                one1["ms_per_layer_batch"] = 1000.0 * wl.batch.n_users / one1["value"]
                one1["cores"] = 1
                res["cpu_oracle_1core"] = one1
        log(f"{label}: " + json.dumps({k: v for k, v in res.items() if not isinstance(v, dict)}))
        return res

    out["config1"] = layer_case(synth.config1(), "full", "config1")
    for s in (1, 4):
        out[f"config2_s{s}"] = layer_case(synth.config2(s), "target", f"config2_s{s}")

    # config 4: forward and backward of one full and one target layer, 64 users of 5632 rows, d 1024
    wl = synth.config4()
    dw = DeviceWorkload(wl)
    meta = B.mask_build(dw.batch)
    dy = to_device(wl.dy, "bf16")
    ws_f = B.workspace(dw.batch, dw.dims, B.OP_FULL)
    ws_t = B.workspace(dw.batch, dw.dims, B.OP_TARGET)
    ws_fb = B.workspace(dw.batch, dw.dims, B.OP_FULL_BWD)
    ws_tb = B.workspace(dw.batch, dw.dims, B.OP_TARGET_BWD)
    x1, x2 = torch.empty_like(dw.x), torch.empty_like(dw.x)
    dx1, dx2 = torch.empty_like(dw.x), torch.empty_like(dw.x)
    fg = {k: torch.empty(tuple(dw.full[0][k].shape), dtype=torch.float32, device="cuda") for k in B.FULL_GRAD_KEYS}
    tg = {k: torch.empty(tuple(dw.target[0][k].shape), dtype=torch.float32, device="cuda")
          for k in B.TARGET_GRAD_KEYS}

    def fwd():
        B.attn_full(dw.batch, dw.dims, meta, dw.full[0], dw.x, x1, ws_f)
        B.attn_target(dw.batch, dw.dims, meta, dw.target[0], x1, x2, ws_t)

    def bwd():
        B.attn_target_bwd(dw.batch, dw.dims, meta, dw.target[0], x1, dy, dx2, tg, ws_tb)
        B.attn_full_bwd(dw.batch, dw.dims, meta, dw.full[0], dw.x, dx2, dx1, fg, ws_fb)

    fwd(); bwd()
    k4 = max(2, n // 4)
    fwd_ms = time_launches(fwd, k4, torch)
    bwd_ms = time_launches(bwd, k4, torch)
    c4 = {"users": wl.batch.n_users, "rows": int(wl.batch.total_rows), "steps": k4,
          "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "fwd_bwd_ms": fwd_ms + bwd_ms,
          "what": "forward of one full + one target layer, then both layers' backward (dX and every weight / "
                  "GLN gradient), d 1024, 16Q/4KV, split 4"}
    if not args.no_cpu_baseline:
        xr = r(wl.x)
        wf, wt = rw(wl.full[0]), rw(wl.target[0])

        def one(u):
            rows = wl.batch.rows_of([u])
            sub = wl.batch.subset([u])
            x_1 = om.full_layer(sub, xr[rows], wf, wl.dims)
            g = og.target_layer_bwd(sub, r(x_1), wt, wl.dims, wl.dy[rows])
            og.full_layer_bwd(sub, xr[rows], wf, wl.dims, r(g["x"]))
        rate = oracle_rate(one, wl.batch.n_users, 1.0, "forward of the full layer, backward of both layers, "
                                                         "one user")
        rate["ms_per_batch"] = 1000.0 * wl.batch.n_users / rate["value"]
        rate["cores"] = blas_threads()
        c4["cpu_oracle"] = rate
    log("config4: " + json.dumps({k: v for k, v in c4.items() if not isinstance(v, dict)}))
    out["config4"] = c4
    del dw, ws_f, ws_t, ws_fb, ws_tb, x1, x2, dx1, dx2, fg, tg, dy
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed forward steps (0: skip the forward timing, for profiling the other parts alone)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--serve-steps", type=int, default=10,
                    help="also time request-level serving: one context pass filling the K/V cache, then this many "
                         "candidate passes over the cached context (0 skips)")
    ap.add_argument("--v2-steps", type=int, default=5,
                    help="also time the V2 target side on config 3's users (AutoSplit into 4 sub-tokens, the "
                         "16-layer stack with a per-sub-token SwiGLU FFN and token mixing after every target "
                         "layer, mean pooling); 0 skips")
    ap.add_argument("--sparse-steps", type=int, default=5,
                    help="timed forward steps with 2:4 structured-sparse projections (0 skips)")
    ap.add_argument("--train-steps", type=int, default=3,
                    help="also time this many training gradient passes (mtfm_backbone_bwd: forward keeping the "
                         "layer inputs, then every layer's backward); 0 skips")
    ap.add_argument("--config-steps", type=int, default=10,
                    help="also time config 1 (one full layer, 32 users), config 2 (one target layer, split 1 and 4) "
                         "and config 4 (forward + backward of one full and one target layer, 64 long users) in their "
                         "own shapes, this many launches each, with the oracle beside each; 0 skips")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB first (calibrates PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    log("generating config-3 workload ...")
    wl = synth.config3()
    dw = DeviceWorkload(wl)
    batch, dims = dw.batch, dw.dims
    lay = B.meta_layout(batch)
    meta = torch.empty(lay.total_bytes, dtype=torch.uint8, device="cuda")
    ws = B.workspace(batch, dims, B.OP_BACKBONE, k_target=wl.k_target)
    x = dw.x
    stream = torch.cuda.current_stream()

    def step():
        B.mask_build(batch, meta)
        B.backbone_fwd(batch, dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, x, ws)

    log(f"rows={lay.n_rows} t_rows={lay.n_t_rows} full_tiles={lay.n_full_tiles} target_tiles={lay.n_target_tiles}")
    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mb} MiB read + {args.copy_probe_mb} MiB written")
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    # counters for the FLOP / byte model (from the device metadata of this batch)
    B.mask_build(batch, meta)
    views = B.meta_views(meta, lay, wl.batch.n_users)
    n_host = views["n"].cpu().numpy().astype(np.int64)
    pairs_full, pairs_t = visible_pairs(n_host, wl.batch.lens.astype(np.int64), wl.batch.split)
    # tile-padding waste: pairs the kernel computes per head over visible pairs
    p_host = views["p"].cpu().numpy().astype(np.int64)
    comp_f, vis_f = computed_pairs(views["full_tiles"].cpu().numpy(), p_host, n_host)
    comp_t, vis_t = computed_pairs(views["target_tiles_sorted"].cpu().numpy(), p_host, n_host,
                                   gperm=views["tsort_g"].cpu().numpy().astype(np.int64))
    assert vis_f == pairs_full and vis_t == pairs_t, "tile walk and row metadata disagree on the visible pairs"
    tile_padding = {"what": "(query, key) pairs the attention kernel computes per head (32 x 32 MFMA blocks "
                            "it runs plus each T row's self term) over the visible pairs sum(n_i)",
                    "full_layer": comp_f / vis_f if vis_f else None,
                    "target_layer": comp_t / vis_t if vis_t else None}
    log("tile padding: " + json.dumps(tile_padding))
    d = wl.dims
    H, G, dh, D = d.n_q_heads, d.n_kv_heads, d.head_dim, d.d_model
    hd, gd = H * dh, G * dh
    R, T, C = lay.n_rows, lay.n_t_rows, lay.n_ctx_rows
    attn_full_flops = 4.0 * dh * H * pairs_full
    attn_t_flops = 4.0 * dh * H * pairs_t
    proj_full_flops = 2.0 * R * D * (2 * hd + 2 * gd) + 2.0 * R * hd * D
    proj_t_flops = 2.0 * R * D * 2 * gd + 2.0 * T * D * 2 * hd + 2.0 * T * hd * D
    layers_full, layers_t = wl.n_blocks, wl.n_blocks * wl.k_target
    step_flops = layers_full * (attn_full_flops + proj_full_flops) + layers_t * (attn_t_flops + proj_t_flops)
    # bytes the target-attention kernel must move: K and V of every packed row once (context rows as key
    # tiles, each T row's own for its self term), Q of the T rows in, A of the T rows out
    attn_t_bytes = 2.0 * (R * 2 * gd + 2 * T * hd)

    # ---- timed region: full-attention kernel bracketed by events on its stream
    # (--steps 0 skips it: a profiling run of the training / serving / V2 parts alone)
    ms_step = samples_s = attn_ms = attn_tflops = None
    if args.steps > 0:
        B.timing_enable([B.K_ATTN_FULL])
        B.timing_read(B.K_ATTN_FULL)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        B.timing_enable([])
        n_attn, ms_attn = B.timing_read(B.K_ATTN_FULL)
        elapsed = t1 - t0
        ms_step = 1000.0 * elapsed / args.steps
        samples_s = wl.batch.n_users * args.steps / elapsed
        attn_ms = ms_attn / max(1, n_attn)
        attn_tflops = attn_full_flops / (attn_ms * 1e-3) / 1e12
        log(f"timed {args.steps} steps: {ms_step:.3f} ms/step, {samples_s:.1f} user-samples/s; "
            f"full attention {attn_ms:.3f} ms/launch -> {attn_tflops:.1f} TFLOP/s")

    breakdown = None
    if not args.no_breakdown and args.steps > 0:
        # full layers: pre-norm, U|Q|K|V projection, attention (gated GLN fused), output projection;
        # target layers: context and T-row normalisations, K|V and T-row projections, attention,
        # T-row output projection
        classes = [B.K_MASK, B.K_GLN, B.K_GEMM_UQKV, B.K_ATTN_FULL, B.K_GEMM_OUT, B.K_GLN_T, B.K_GEMM_KV,
                   B.K_GEMM_T, B.K_ATTN_TARGET, B.K_GEMM_OUT_T]
        names = ["mask", "gln_full", "gemm_uqkv", "attn_full", "gemm_out_full", "gln_target", "gemm_kv",
                 "gemm_t", "attn_target", "gemm_out_t"]
        B.timing_enable(classes)
        for k in classes:
            B.timing_read(k)
        kb = max(2, args.steps // 4)
        for _ in range(kb):
            step()
        torch.cuda.synchronize()
        B.timing_enable([])
        breakdown = {}
        for k, nm in zip(classes, names):
            n, ms = B.timing_read(k)
            breakdown[nm] = {"launches_per_step": n / kb, "ms_per_step": ms / kb,
                             "ms_per_launch": ms / max(1, n)}
        tat = breakdown["attn_target"]["ms_per_launch"]
        breakdown["attn_target"]["achieved_GBs"] = attn_t_bytes / (tat * 1e-3) / 1e9 if tat > 0 else None
        breakdown["attn_target"]["hbm_frac"] = (breakdown["attn_target"]["achieved_GBs"] or 0) / HBM_PEAK_GBS
        breakdown["attn_target"]["achieved_TFLOPs"] = attn_t_flops / (tat * 1e-3) / 1e12 if tat > 0 else None
        full_ms = sum(breakdown[k]["ms_per_step"] for k in ("gln_full", "gemm_uqkv", "attn_full", "gemm_out_full"))
        breakdown["full_layers_ms_per_step"] = full_ms
        breakdown["full_layers_masked_TFLOPs"] = layers_full * (attn_full_flops + proj_full_flops) / (full_ms * 1e-3) / 1e12
        breakdown["full_layers_mfma_frac"] = breakdown["full_layers_masked_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
        breakdown["sum_ms_per_step"] = sum(v["ms_per_step"] for v in breakdown.values() if isinstance(v, dict))
        breakdown["note"] = ("per-class times are HIP-event spans around each launch; the events themselves add a "
                             "few microseconds between launches, so the sum slightly exceeds ms_per_step")
        log("breakdown: " + json.dumps(breakdown))

    train = None
    if args.train_steps > 0:
        # training gradient pass of the same batch: dL/dX and every layer's weight / GLN gradients
        nb = B.backbone_bwd_workspace_bytes(batch, dims, wl.n_blocks, wl.k_target)
        ws_b = torch.empty(nb, dtype=torch.uint8, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(33)
        dy = torch.randn(x.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        dx = torch.empty_like(x)
        fg = [{k: torch.empty(tuple(w[k].shape), dtype=torch.float32, device="cuda") for k in B.FULL_GRAD_KEYS}
              for w in dw.full]
        tg = [{k: torch.empty(tuple(w[k].shape), dtype=torch.float32, device="cuda") for k in B.TARGET_GRAD_KEYS}
              for w in dw.target]

        def train_step():
            B.mask_build(batch, meta)
            B.backbone_bwd(batch, dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, x, dy, dx, fg, tg, ws_b)

        train_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.train_steps):
            train_step()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        train = {"what": "mtfm_backbone_bwd with the full workspace: forward keeping 15 layers' inputs and "
                         "intermediates + backward of all 16 layers (dX and every weight / GLN gradient), "
                         "incl. mask build",
                 "steps": args.train_steps, "ms_per_step": 1000.0 * el / args.train_steps,
                 "user_samples_per_s": wl.batch.n_users * args.train_steps / el,
                 "workspace_GiB": nb / 2 ** 30}
        log(f"training gradient pass: {train['ms_per_step']:.2f} ms/step, {train['user_samples_per_s']:.1f} "
            f"user-samples/s")
        del ws_b, dy, dx, fg, tg
        if not args.no_cpu_baseline:
            # the oracle's gradient pass on single users of the same batch
            from oracle import grad as og
            from oracle import model as om
            r = om.bf16_round
            full_r = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl.full]
            tgt_r = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl.target]
            dy_h = np.random.default_rng(33).standard_normal((wl.batch.total_rows, wl.dims.d_model))

            def train_user(u):
                rows = wl.batch.rows_of([u])
                og.backbone_bwd(wl.batch.subset([u]), wl.x[rows], full_r, tgt_r, wl.dims, wl.n_blocks,
                                wl.k_target, dy_h[rows], boundary=r)

            train["cpu_oracle"] = oracle_rate(train_user, wl.batch.n_users, min(args.cpu_seconds, 10.0),
                                              "16-layer forward + backward (oracle.grad.backbone_bwd)")
            log(f"training oracle: {train['cpu_oracle']}")

    serve = None
    if args.serve_steps > 0:
        # the same users' context once into the K/V cache, then the batch's candidates (T rows) against it
        lens_c = wl.batch.lens.copy()
        lens_c[:, 2] = 0
        cb = B.DeviceBatch(lens_c, wl.batch.split, wl.batch.ts_r, np.zeros(0, np.int32))
        meta_c = B.mask_build(cb)
        off = wl.batch.row_off
        ctx_idx, t_idx = [], []
        for u in range(wl.batch.n_users):
            lh, lr, lt = (int(v) for v in wl.batch.lens[u])
            ctx_idx.append(np.arange(off[u], off[u] + lh + lr))
            t_idx.append(np.arange(off[u] + lh + lr, off[u + 1]))
        ctx_idx = torch.as_tensor(np.concatenate(ctx_idx), device="cuda")
        t_idx = torch.as_tensor(np.concatenate(t_idx), device="cuda")
        cache = torch.empty(B.kv_cache_bytes(cb, dims, wl.n_blocks, wl.k_target), dtype=torch.uint8, device="cuda")
        ws_c = torch.empty(B.serve_workspace_bytes(cb, dims, wl.k_target, B.SERVE_CONTEXT), dtype=torch.uint8,
                           device="cuda")
        ws_t = torch.empty(B.serve_workspace_bytes(batch, dims, wl.k_target, B.SERVE_TARGETS), dtype=torch.uint8,
                           device="cuda")
        x_c0, x_t0 = dw.x[ctx_idx].contiguous(), dw.x[t_idx].contiguous()
        x_c, x_t = x_c0.clone(), x_t0.clone()

        def ctx_pass():
            x_c.copy_(x_c0)
            B.mask_build(cb, meta_c)
            B.serve_context(cb, dims, wl.n_blocks, wl.k_target, meta_c, dw.full, dw.target, x_c, cache, ws_c)

        def cand_pass():
            x_t.copy_(x_t0)
            B.mask_build(batch, meta)
            B.serve_targets(batch, dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, cache, x_t, ws_t)

        ctx_pass()
        cand_pass()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx_pass()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.serve_steps):
            cand_pass()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        cand_ms = 1000.0 * (t2 - t1) / args.serve_steps
        serve = {"what": "context pass (160 users' H/R rows through 16 layers, every layer's K/V^T cached) once; "
                         "candidate pass (the batch's T rows through 16 layers against the cache) timed",
                 "context_ms": 1000.0 * (t1 - t0), "candidate_pass_ms": cand_ms,
                 "candidates_per_s": float(wl.batch.lens[:, 2].sum()) / (cand_ms * 1e-3),
                 "t_rows": int(T), "kv_cache_GiB": cache.numel() / 2 ** 30,
                 "vs_full_forward": ms_step / cand_ms if ms_step else None}
        log(f"serving: context {serve['context_ms']:.2f} ms once, candidates {cand_ms:.3f} ms/pass "
            f"({serve['candidates_per_s']:.0f} candidates/s, {serve['vs_full_forward'] or 0:.1f}x the full forward)")
        del cache, ws_c, ws_t, x_c, x_t, x_c0, x_t0

        # one request: a single user's long history cached, a list of candidates against it (the
        # target attention then splits each slice's keys over several workgroups)
        b1 = synth.make_batch(np.random.default_rng(31), np.array([[6000, 2000, 512]], np.int32), 1)
        db1 = B.DeviceBatch(b1.lens, 1, b1.ts_r, b1.ts_t)
        lens1c = b1.lens.copy()
        lens1c[:, 2] = 0
        cb1 = B.DeviceBatch(lens1c, 1, b1.ts_r, np.zeros(0, np.int32))
        meta1c, meta1 = B.mask_build(cb1), B.mask_build(db1)
        cache1 = torch.empty(B.kv_cache_bytes(cb1, dims, wl.n_blocks, wl.k_target), dtype=torch.uint8, device="cuda")
        ws1c = torch.empty(B.serve_workspace_bytes(cb1, dims, wl.k_target, B.SERVE_CONTEXT), dtype=torch.uint8,
                           device="cuda")
        ws1t = torch.empty(B.serve_workspace_bytes(db1, dims, wl.k_target, B.SERVE_TARGETS), dtype=torch.uint8,
                           device="cuda")
        gen = torch.Generator().manual_seed(32)
        xc1 = torch.randn(8000, dims.d_model, generator=gen).to(device="cuda", dtype=torch.bfloat16)
        xt1_0 = torch.randn(512, dims.d_model, generator=gen).to(device="cuda", dtype=torch.bfloat16)
        xt1 = xt1_0.clone()
        B.serve_context(cb1, dims, wl.n_blocks, wl.k_target, meta1c, dw.full, dw.target, xc1, cache1, ws1c)

        def one_pass():
            xt1.copy_(xt1_0)
            B.mask_build(db1, meta1)
            B.serve_targets(db1, dims, wl.n_blocks, wl.k_target, meta1, dw.full, dw.target, cache1, xt1, ws1t)

        one_pass()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.serve_steps):
            one_pass()
        torch.cuda.synchronize()
        one_ms = 1000.0 * (time.perf_counter() - t0) / args.serve_steps
        serve["one_user"] = {"what": "one user's 6000 H + 2000 R rows cached (16 layers), 512 candidates through "
                                     "the 16 layers against it; metadata build included",
                             "candidate_pass_ms": one_ms, "candidates_per_s": 512 / (one_ms * 1e-3)}
        log(f"serving one user (8000 context rows, 512 candidates): {one_ms:.3f} ms/pass")
        del cache1, ws1c, ws1t, xc1, xt1, xt1_0

    v2 = None
    if args.v2_steps > 0:
        from hybrid_masked_attention_amd.tensors import to_device, weights_to_device
        wl2, feats, w_split, ffn = synth.config3_v2()
        dw2 = DeviceWorkload(wl2)
        meta2 = B.mask_build(dw2.batch)
        d_ff = ffn[0]["w_gate"].shape[1]
        ws2 = torch.empty(B.backbone_v2_workspace_bytes(dw2.batch, dw2.dims, wl2.k_target, d_ff), dtype=torch.uint8,
                          device="cuda")
        fd, wd = to_device(feats, "bf16"), to_device(w_split, "bf16")
        ffd = [weights_to_device(w, "bf16") for w in ffn]
        n_par = feats.shape[0]
        pooled = torch.empty((n_par, wl2.dims.d_model), dtype=torch.bfloat16, device="cuda")
        x2 = dw2.x.clone()

        def v2_step():
            B.mask_build(dw2.batch, meta2)
            B.autosplit(dw2.batch, dw2.dims, feats.shape[1], meta2, fd, wd, x2)
            B.backbone_v2_fwd(dw2.batch, dw2.dims, wl2.n_blocks, wl2.k_target, d_ff, meta2, dw2.full, dw2.target,
                              ffd, x2, ws2)
            B.token_pool(dw2.batch, dw2.dims, meta2, x2, pooled)

        v2_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.v2_steps):
            v2_step()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        v2 = {"what": "V2 target side on config 3's 160 users: AutoSplit (feature width 512 -> 4 sub-tokens), "
                      "16 layers with a per-sub-token SwiGLU FFN (hidden 1024) and token mixing after each target "
                      "layer, mean pooling; metadata build included",
              "rows": int(wl2.batch.total_rows), "t_rows": int(wl2.batch.total_t_rows), "steps": args.v2_steps,
              "ms_per_step": 1000.0 * el / args.v2_steps,
              "user_samples_per_s": wl2.batch.n_users * args.v2_steps / el}
        log(f"V2 target side: {v2['ms_per_step']:.2f} ms/step, {v2['user_samples_per_s']:.1f} user-samples/s")
        del dw2, ws2, x2, pooled, ffd
        if not args.no_cpu_baseline:
            from oracle import model as om
            from oracle import v2 as ov2
            r = om.bf16_round
            f2 = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl2.full]
            t2 = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl2.target]
            v2["cpu_oracle"] = oracle_rate(
                lambda u: ov2.backbone_v2(wl2.batch, wl2.x, f2, t2, ffn, wl2.dims, wl2.n_blocks, wl2.k_target,
                                          boundary=r, users=[u]),
                wl2.batch.n_users, min(args.cpu_seconds, 10.0), "V2 16-layer stack with token FFNs (oracle.v2)")
            log(f"V2 oracle: {v2['cpu_oracle']}")

    sparse = None
    if args.sparse_steps > 0:
        # the same forward with every projection 2:4-pruned and packed (inference weights)
        t0 = time.perf_counter()
        full_s = [dict(w, **B.pack_full_s24(w)) for w in dw.full]
        tgt_s = [dict(w, **B.pack_target_s24(w, wl.batch.split)) for w in dw.target]
        torch.cuda.synchronize()
        pack_ms = 1000.0 * (time.perf_counter() - t0)

        def sparse_step():
            B.mask_build(batch, meta)
            B.backbone_fwd(batch, dims, wl.n_blocks, wl.k_target, meta, full_s, tgt_s, x, ws)

        for _ in range(2):
            sparse_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.sparse_steps):
            sparse_step()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        proj = [B.K_GEMM_UQKV, B.K_GEMM_OUT, B.K_GEMM_KV, B.K_GEMM_T, B.K_GEMM_OUT_T]
        B.timing_enable(proj)
        for k in proj:
            B.timing_read(k)
        for _ in range(2):
            sparse_step()
        torch.cuda.synchronize()
        B.timing_enable([])
        proj_ms = sum(B.timing_read(k)[1] for k in proj) / 2
        proj_flops = layers_full * proj_full_flops + layers_t * proj_t_flops
        sparse = {"what": "the config-3 forward with every projection (U|Q|K|V, K|V, T rows, output) 2:4-pruned "
                          "and run on the sparse MFMA (mtfm_s24_pack'ed weights); metadata build included",
                  "steps": args.sparse_steps, "ms_per_step": 1000.0 * el / args.sparse_steps,
                  "user_samples_per_s": wl.batch.n_users * args.sparse_steps / el,
                  "pack_ms_all_layers": pack_ms,
                  "projection_ms_per_step": proj_ms,
                  "projection_dense_equiv_TFLOPs": proj_flops / (proj_ms * 1e-3) / 1e12 if proj_ms > 0 else None}
        if breakdown:
            dense_proj = sum(breakdown[k]["ms_per_step"]
                             for k in ("gemm_uqkv", "gemm_out_full", "gemm_kv", "gemm_t", "gemm_out_t"))
            sparse["projection_dense_ms_per_step"] = dense_proj
            sparse["projection_speedup"] = dense_proj / proj_ms if proj_ms > 0 else None
        if ms_step:
            sparse["vs_dense_forward"] = ms_step / sparse["ms_per_step"]
        log("sparse projections: " + json.dumps(sparse))
        del full_s, tgt_s

    configs = None
    if args.config_steps > 0:
        configs = config_sections(args, B, torch, synth, np)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s ...")
        cpu = cpu_baseline(wl, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")

    out = {
        "metric": "user-samples/s, 16-layer hybrid attn fwd; masked TFLOP/s vs MFMA peak",
        "value": samples_s,
        "unit": "user-samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "config 3: 16-layer hybrid backbone fwd (4 x (1 full + 3 target)), 160 users, "
                               "N~U[1000,2000] 70/20/10 H/R/T, d 512, 8Q/2KV, dh 64",
                   "users": wl.batch.n_users, "rows": int(R), "t_rows": int(T), "parallelism": "single-gpu"},
        "step_algorithmic_TFLOP": step_flops / 1e12,
        "step_TFLOPs": step_flops / (ms_step * 1e-3) / 1e12 if ms_step else None,
        "roofline": {"kernel": "attn_bf16_kernel (full layer)", "bound": "mfma", "achieved": attn_tflops,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS if attn_tflops else None,
                     "traffic": recorded_traffic(), "flops_per_launch": attn_full_flops,
                     "ms_per_launch": attn_ms} if args.steps > 0 else None,
        "tile_padding": tile_padding,
        "breakdown": breakdown,
        "train": train,
        "serve": serve,
        "v2": v2,
        "sparse": sparse,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
