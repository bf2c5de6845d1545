"""GPU parity of the 2:4 structured-sparse projections ([explainer] §5.2.1).

mtfm_s24_pack is index work: its packed matrix, decoded with the layout that
include/mtfm.h states, must equal the oracle's pruning bit for bit -- the
kept values and their positions.  Layers, the backbone and the serving path
whose weight structs carry the packed projections must reproduce the
oracle's model run on the pruned weights to the bar of the dense bf16 path
(max|gpu - ref| <= 1e-2 * max|ref| per tensor): the sparse instruction only
skips the zeros, so the sums are the dense ones on the pruned weights up to
rounding order.  The backward entry points ignore the packed fields.
"""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import sparse as osp
from tests._parity import TOL_BF16, Report, rounded_inputs, say, to_np, ws_tensor

pytestmark = pytest.mark.gpu


def decode_s24(buf, rows, k):
    """Dense [rows][k] matrix and kept-position mask from a packed buffer (layout of include/mtfm.h)."""
    nks = k // 32
    raw = np.asarray(buf, np.uint8)
    bits = raw[:rows * k].view(np.uint16).reshape(nks, rows, 2, 8)
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    idx = raw[rows * k:rows * k + rows * k // 8].view(np.uint16).reshape(nks, rows, 2).astype(np.int64)
    dense = np.zeros((rows, k))
    keep = np.zeros((rows, k), bool)
    r = np.arange(rows)
    for ks in range(nks):
        for h in range(2):
            for j in range(4):
                q = 2 * h + j + (2 if j >= 2 else 0)          # group of the K step
                p0 = (idx[ks, :, h] >> (4 * j)) & 3
                p1 = (idx[ks, :, h] >> (4 * j + 2)) & 3
                assert np.all(p0 != p1), "a group's two kept entries share a position"
                for e, p in ((0, p0), (1, p1)):
                    col = ks * 32 + 4 * q + p
                    dense[r, col] = vals[ks, :, h, 2 * j + e]
                    keep[r, col] = True
    return dense, keep


def _bf16_matrix(rng, rows, k):
    """Normal values, plus rows of small integers (many ties) and of zeros of both signs."""
    w = rng.standard_normal((rows, k))
    w[1::5] = rng.integers(-2, 3, size=w[1::5].shape)
    w[3::7] = 0.0
    w[4::7, ::3] = -0.0
    return om.bf16_round(w)


def test_pack_matches_oracle_pruning():
    import torch
    from hybrid_masked_attention_amd import binding as B
    rng = np.random.default_rng(31)
    k = 160
    segs = [_bf16_matrix(rng, r, k) for r in (48, 0, 16, 200)]     # an empty segment is skipped
    say(f"s24 pack: segments {[s.shape for s in segs]}")
    dev = [torch.as_tensor(s, dtype=torch.float32).to(torch.bfloat16).cuda() for s in segs]
    packed = B.s24_pack(dev)
    torch.cuda.synchronize()
    rows = sum(s.shape[0] for s in segs)
    assert packed.numel() == B.s24_pack_bytes(rows, k) == rows * k * 9 // 8
    dense, keep = decode_s24(packed.cpu().numpy(), rows, k)
    w = np.concatenate(segs)
    np.testing.assert_array_equal(keep, osp.keep_mask_24(w))
    np.testing.assert_array_equal(dense, osp.prune_24(w))
    # -0.0 kept as -0.0 (the bits move unchanged)
    assert np.array_equal(np.signbit(dense[keep]), np.signbit(w[keep]))


def _run_layer(wl, kind):
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    say(f"sparse layer parity: {wl.name} {kind} rows={wl.batch.total_rows} users={wl.batch.n_users}")
    dw = DeviceWorkload(wl).pack_s24()
    meta = B.mask_build(dw.batch)
    op = B.OP_FULL if kind == "full" else B.OP_TARGET
    ws = B.workspace(dw.batch, dw.dims, op)
    out = torch.empty_like(dw.x)
    if kind == "full":
        B.attn_full(dw.batch, dw.dims, meta, dw.full[0], dw.x, out, ws)
    else:
        B.attn_target(dw.batch, dw.dims, meta, dw.target[0], dw.x, out, ws)
    torch.cuda.synchronize()
    off_a, off_y = B.workspace_probe(dw.batch, dw.dims, op)
    hd = wl.dims.n_q_heads * wl.dims.head_dim
    rows = wl.batch.total_rows if kind == "full" else wl.batch.total_t_rows
    y = to_np(ws_tensor(ws, off_y, rows, hd, wl.dtype))
    return to_np(dw.x), to_np(out), y


def _check_layer(wl, kind):
    x_dev, out_dev, y_dev = _run_layer(wl, kind)
    x, full, tgt = rounded_inputs(wl)
    np.testing.assert_array_equal(x_dev, x)
    if kind == "full":
        out, parts = om.full_layer(wl.batch, x, osp.prune_full_weights(full[0]), wl.dims, return_parts=True)
    else:
        out, parts = om.target_layer(wl.batch, x, osp.prune_target_weights(tgt[0]), wl.dims, return_parts=True)
    r = Report(TOL_BF16)
    r.close("X'", out_dev, out)
    r.branch("dX", out_dev, out, x, wl.dtype)
    r.close("Y", y_dev, parts["y"])
    # the pruning matters at this scale: the dense layer is measurably different
    if kind == "full":
        dense = om.full_layer(wl.batch, x, full[0], wl.dims)
    else:
        dense = om.target_layer(wl.batch, x, tgt[0], wl.dims)
    d = float(np.max(np.abs(dense - out))) / float(np.max(np.abs(out - x)))
    say(f"  pruned vs dense branch difference: {d:.3e}")
    assert d > 10 * TOL_BF16
    r.check()


def test_config1_full_layer_sparse():
    _check_layer(synth.config1(), "full")


@pytest.mark.parametrize("split", [1, 4])
def test_config2_target_layer_sparse(split):
    _check_layer(synth.config2(split), "target")


EDGE_LENS = [[0, 0, 0], [64, 0, 0], [0, 64, 0], [0, 0, 3], [130, 64, 17], [1, 0, 1], [63, 1, 0],
             [65, 63, 33], [5, 200, 2]]


@pytest.mark.parametrize("split", [1, 4])
@pytest.mark.parametrize("kind", ["full", "target"])
def test_edge_users_sparse(kind, split):
    rng = np.random.default_rng(300 + split)
    batch = synth.make_batch(rng, np.asarray(EDGE_LENS, np.int32), split)
    dims = synth.Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    wl = synth.Workload(f"edge_s24_{split}", batch, dims, "bf16", x,
                        full=[synth.full_weights(rng, dims, 0.05, 0.05)],
                        target=[synth.target_weights(rng, dims, split, 0.05, 0.05)])
    _check_layer(wl, kind)


@pytest.mark.parametrize("shape", [(512, 8, 8), (256, 4, 1), (1024, 16, 4)])
def test_other_widths_sparse(shape):
    """Other model widths and GQA ratios: K = 256 .. 1024 (8 .. 32 sparse K steps, a multiple of
    the three-stage ring or not) and projection stacks of 640 .. 2560 rows."""
    d, h, g = shape
    rng = np.random.default_rng(400 + d + g)
    batch = synth.make_batch(rng, np.asarray(EDGE_LENS[4:], np.int32), 1)
    dims = synth.Dims(d, h, g, 64)
    x = rng.standard_normal((batch.total_rows, d)).astype(np.float32)
    wl = synth.Workload(f"widths_s24_{d}_{h}_{g}", batch, dims, "bf16", x,
                        full=[synth.full_weights(rng, dims, 0.05, 0.05)],
                        target=[synth.target_weights(rng, dims, 1, 0.05, 0.05)])
    _check_layer(wl, "full")
    _check_layer(wl, "target")


def _pruned(ws, prune):
    return [prune(w) for w in ws]


def test_config3_backbone_sparse_sampled_users():
    """The 160-user, 16-layer bf16 batch with every projection packed (the benchmarked sparse
    launch); oracle on sampled users with the pruned weights."""
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    wl = synth.config3()
    say(f"sparse backbone parity: {wl.batch.n_users} users, {wl.batch.total_rows} rows")
    dw = DeviceWorkload(wl).pack_s24()
    meta = B.mask_build(dw.batch)
    ws = B.workspace(dw.batch, dw.dims, B.OP_BACKBONE, k_target=wl.k_target)
    x = dw.x.clone()
    B.backbone_fwd(dw.batch, dw.dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, x, ws)
    torch.cuda.synchronize()
    got = to_np(x)
    xr, full, tgt = rounded_inputs(wl)
    users = [0, 77, 159]
    ref = om.backbone(wl.batch, xr, _pruned(full, osp.prune_full_weights), _pruned(tgt, osp.prune_target_weights),
                      wl.dims, wl.n_blocks, wl.k_target, boundary=om.bf16_round, users=users)
    rows = wl.batch.rows_of(users)
    assert np.all(np.isfinite(got))
    r = Report(TOL_BF16)
    r.close("X' (3 users)", got[rows], ref)
    r.branch("dX (3 users, 16 roundings allowed)", got[rows], ref, xr[rows], "bf16", roundings=16)
    r.check()


@pytest.mark.parametrize("split", [1, 4])
def test_serving_sparse_matches_oracle(split):
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    from tests.test_gpu_serve import _rows, _serve_context, _serve_targets, _small
    wl = _small(split, 520 + split)
    say(f"sparse serving: {wl.batch.n_users} users, {wl.batch.total_rows} rows, split {split}")
    dw = DeviceWorkload(wl).pack_s24()
    ctx_rows, t_rows = _rows(wl.batch)
    x_ctx, cache = _serve_context(wl, dw, B, torch)
    x_t = dw.x[torch.as_tensor(t_rows, device="cuda")].contiguous()
    _serve_targets(wl, dw, B, torch, cache, x_t)
    torch.cuda.synchronize()
    xr, full, tgt = rounded_inputs(wl)
    o = om.backbone(wl.batch, xr, _pruned(full, osp.prune_full_weights), _pruned(tgt, osp.prune_target_weights),
                    wl.dims, wl.n_blocks, wl.k_target, boundary=om.bf16_round)
    r = Report(TOL_BF16)
    r.branch("context rows", to_np(x_ctx), o[ctx_rows], xr[ctx_rows], "bf16", roundings=16)
    r.branch("T rows", to_np(x_t), o[t_rows], xr[t_rows], "bf16", roundings=16)
    r.check()


def test_backward_ignores_packed_weights():
    """mtfm_backbone_bwd with the packed fields set computes the dense-weight gradients bit for bit."""
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload, to_device
    rng = np.random.default_rng(77)
    lens = [[130, 64, 17], [1, 0, 1], [63, 1, 0], [65, 63, 33], [5, 70, 2]]
    batch = synth.make_batch(rng, np.asarray(lens, np.int32), 1)
    dims = synth.Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, 512)).astype(np.float32)
    wl = synth.Workload("bwd_s24", batch, dims, "bf16", x, full=[synth.full_weights(rng, dims, 0.05, 0.05)],
                        target=[synth.target_weights(rng, dims, 1, 0.05, 0.05)], n_blocks=1, k_target=1)
    dy = to_device(rng.standard_normal((batch.total_rows, 512)).astype(np.float32), "bf16")

    def run(packed):
        dw = DeviceWorkload(wl)
        if packed:
            dw.pack_s24()
        meta = B.mask_build(dw.batch)
        ws = torch.empty(B.backbone_bwd_workspace_bytes(dw.batch, dw.dims, 1, 1), dtype=torch.uint8, device="cuda")
        dx = torch.empty_like(dw.x)
        fg = [{k: torch.empty(tuple(w[k].shape), dtype=torch.float32, device="cuda") for k in B.FULL_GRAD_KEYS}
              for w in dw.full]
        tg = [{k: torch.empty(tuple(w[k].shape), dtype=torch.float32, device="cuda") for k in B.TARGET_GRAD_KEYS}
              for w in dw.target]
        B.backbone_bwd(dw.batch, dw.dims, 1, 1, meta, dw.full, dw.target, dw.x, dy, dx, fg, tg, ws)
        torch.cuda.synchronize()
        return [to_np(dx)] + [to_np(v) for g in fg + tg for v in g.values()]

    for a, b in zip(run(False), run(True)):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("split", [1, 4])
def test_v2_stack_sparse(split):
    """The V2 stack (token FFNs after every target layer) with every projection packed: the
    projections use the pruned weights, the FFNs stay dense ([explainer] §5.2.1 names the U, V, Q,
    K and output projections)."""
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    from oracle import v2 as ov
    from tests.test_gpu_v2 import _ffn_dev, _round_ffn, _small_v2
    wl, ffn = _small_v2(split, 640 + split)
    say(f"sparse V2 stack: {wl.batch.n_users} users, {wl.batch.total_rows} rows, split {split}")
    dw = DeviceWorkload(wl).pack_s24()
    meta = B.mask_build(dw.batch)
    ws = torch.empty(B.backbone_v2_workspace_bytes(dw.batch, dw.dims, wl.k_target, 256), dtype=torch.uint8,
                     device="cuda")
    x = dw.x.clone()
    B.backbone_v2_fwd(dw.batch, dw.dims, wl.n_blocks, wl.k_target, 256, meta, dw.full, dw.target,
                      [_ffn_dev(w) for w in ffn], x, ws)
    torch.cuda.synchronize()
    got = to_np(x)
    xr, full, tgt = rounded_inputs(wl)
    ref = ov.backbone_v2(wl.batch, xr, _pruned(full, osp.prune_full_weights), _pruned(tgt, osp.prune_target_weights),
                         [_round_ffn(w) for w in ffn], wl.dims, 2, 3, boundary=om.bf16_round)
    tr = ov.t_rows(wl.batch)
    ctx = np.setdiff1d(np.arange(wl.batch.total_rows), tr)
    r = Report(TOL_BF16)
    r.branch("context rows", got[ctx], ref[ctx], xr[ctx], "bf16", roundings=8)
    r.branch("T rows", got[tr], ref[tr], xr[tr], "bf16", roundings=14)
    r.check()


def test_sparse_layers_are_deterministic():
    """Two runs of the sparse-projection layers on the same inputs are bit-identical."""
    rng = np.random.default_rng(700)
    batch = synth.make_batch(rng, np.asarray(EDGE_LENS, np.int32), 4)
    dims = synth.Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    wl = synth.Workload("det_s24", batch, dims, "bf16", x, full=[synth.full_weights(rng, dims, 0.05, 0.05)],
                        target=[synth.target_weights(rng, dims, 4, 0.05, 0.05)])
    for kind in ("full", "target"):
        a, b = _run_layer(wl, kind), _run_layer(wl, kind)
        for u, v in zip(a, b):
            np.testing.assert_array_equal(u, v)
