"""GPU parity of the V2 target side (AutoSplit, per-sub-token SwiGLU FFN with token mixing, mean
pooling, and the V2 stack) against oracle/v2.py on the same bf16-rounded inputs.  Bars as for the
layers: 1e-2 * max|ref| for activations, the residual-branch bar with one bf16 rounding allowed per
stored layer output for stacks; rows a call must not touch are compared bit for bit."""
import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import v2 as ov
from tests._parity import TOL_BF16, Report, rounded_inputs, say, to_np

pytestmark = pytest.mark.gpu
LENS = [[130, 64, 17], [1, 0, 1], [63, 1, 0], [0, 0, 3], [65, 63, 33], [5, 70, 2], [0, 0, 0], [90, 30, 9]]


def _dev(a, dtype="bf16"):
    from hybrid_masked_attention_amd.tensors import to_device
    return to_device(a, dtype)


def _ffn_dev(w):
    from hybrid_masked_attention_amd.tensors import weights_to_device
    return weights_to_device(w, "bf16")


def _round_ffn(w):
    r = om.bf16_round
    return {k: (v.astype(np.float64) if k.startswith("ln") else r(v)) for k, v in w.items()}


def _setup(split, seed, d_ff=256):
    rng = np.random.default_rng(seed)
    batch = synth.make_batch(rng, np.asarray(LENS, np.int32), split)
    dims = synth.Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, 512)).astype(np.float32)
    return rng, batch, dims, x


def test_autosplit():
    import torch
    from hybrid_masked_attention_amd import binding as B
    rng, batch, dims, x = _setup(4, 200)
    P = int(batch.lens[:, 2].sum())
    feats = rng.standard_normal((P, 96)).astype(np.float32)
    w = (rng.standard_normal((4 * 512, 96)) / 10).astype(np.float32)
    db = B.DeviceBatch.from_synth(batch)
    meta = B.mask_build(db)
    xd = _dev(x)
    B.autosplit(db, B.make_dims(512, 8, 2, 64), 96, meta, _dev(feats), _dev(w), xd)
    torch.cuda.synchronize()
    got = to_np(xd)
    tr = ov.t_rows(batch)
    ref = ov.autosplit(om.bf16_round(feats), om.bf16_round(w), 4)
    r = Report(TOL_BF16)
    r.close("AutoSplit T rows", got[tr], ref)
    r.check()
    other = np.setdiff1d(np.arange(batch.total_rows), tr)
    np.testing.assert_array_equal(got[other], om.bf16_round(x)[other])


@pytest.mark.parametrize("split", [1, 4])
def test_token_ffn_and_mixing(split):
    import torch
    from hybrid_masked_attention_amd import binding as B
    rng, batch, dims, x = _setup(split, 210 + split)
    w = synth.ffn_weights(rng, dims, split, 256, 0.05, 0.05)
    db = B.DeviceBatch.from_synth(batch)
    cd = B.make_dims(512, 8, 2, 64)
    meta = B.mask_build(db)
    ws = torch.empty(max(1, B.token_ffn_workspace_bytes(db, cd, 256)), dtype=torch.uint8, device="cuda")
    xd = _dev(x)
    B.token_ffn(db, cd, 256, meta, _ffn_dev(w), xd, ws)
    torch.cuda.synchronize()
    got = to_np(xd)
    xr = om.bf16_round(x)
    tr = ov.t_rows(batch)
    ref = ov.token_mix(ov.token_ffn(xr[tr], _round_ffn(w), split, 1e-5), split)
    r = Report(TOL_BF16)
    r.branch("T rows", got[tr], ref, ov.token_mix(xr[tr], split), "bf16", roundings=1)
    r.close("T rows (whole values)", got[tr], ref)
    r.check()
    other = np.setdiff1d(np.arange(batch.total_rows), tr)
    np.testing.assert_array_equal(got[other], xr[other])


def test_token_pool():
    import torch
    from hybrid_masked_attention_amd import binding as B
    rng, batch, dims, x = _setup(4, 220)
    db = B.DeviceBatch.from_synth(batch)
    meta = B.mask_build(db)
    P = int(batch.lens[:, 2].sum())
    out = torch.empty((P, 512), dtype=torch.bfloat16, device="cuda")
    B.token_pool(db, B.make_dims(512, 8, 2, 64), meta, _dev(x), out)
    torch.cuda.synchronize()
    ref = ov.mean_pool(om.bf16_round(x)[ov.t_rows(batch)], 4)
    # fp32 sum of four bf16 values, scaled by 1/4 exactly, one final bf16 rounding: within half an ulp
    got = to_np(out)
    assert np.all(np.abs(got - ref) <= np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8) + 1e-30)


def _small_v2(split, seed, d_ff=256):
    rng, batch, dims, x = _setup(split, seed)
    full = [synth.full_weights(rng, dims, 0.02, 0.02) for _ in range(2)]
    tgt = [synth.target_weights(rng, dims, split, 0.02, 0.02) for _ in range(6)]
    ffn = [synth.ffn_weights(rng, dims, split, d_ff, 0.02, 0.02) for _ in range(6)]
    wl = synth.Workload(f"v2_small_s{split}", batch, dims, "bf16", x, full=full, target=tgt, n_blocks=2, k_target=3)
    return wl, ffn


def _v2_device(wl, ffn, d_ff):
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    dw = DeviceWorkload(wl)
    meta = B.mask_build(dw.batch)
    ws = torch.empty(B.backbone_v2_workspace_bytes(dw.batch, dw.dims, wl.k_target, d_ff), dtype=torch.uint8,
                     device="cuda")
    x = dw.x.clone()
    B.backbone_v2_fwd(dw.batch, dw.dims, wl.n_blocks, wl.k_target, d_ff, meta, dw.full, dw.target,
                      [_ffn_dev(w) for w in ffn], x, ws)
    torch.cuda.synchronize()
    return to_np(dw.x), to_np(x)


@pytest.mark.parametrize("split", [1, 4])
def test_v2_stack_small(split):
    """2 blocks x (1 full + 3 target layers, each followed by its token FFN and mixing)."""
    wl, ffn = _small_v2(split, 230 + split)
    say(f"V2 stack: {wl.batch.n_users} users, {wl.batch.total_rows} rows, split {split}")
    x0, got = _v2_device(wl, ffn, 256)
    xr, full, tgt = rounded_inputs(wl)
    np.testing.assert_array_equal(x0, xr)
    ref = ov.backbone_v2(wl.batch, xr, full, tgt, [_round_ffn(w) for w in ffn], wl.dims, 2, 3,
                         boundary=om.bf16_round)
    r = Report(TOL_BF16)
    tr = ov.t_rows(wl.batch)
    ctx = np.setdiff1d(np.arange(wl.batch.total_rows), tr)
    # one bf16 rounding allowed per stored layer output the rows pass through, as in the V1 backbone
    # tests: 8 for the context rows (2 full + 6 target layers), 14 for the T rows (plus the 6 FFNs).
    # Six mixings (an even number) are the identity permutation for S = 4, so the T rows' branch is
    # still measured against their own input.
    r.branch("context rows", got[ctx], ref[ctx], xr[ctx], "bf16", roundings=8)
    r.branch("T rows", got[tr], ref[tr], xr[tr], "bf16", roundings=14)
    r.check()


def test_config3_v2_sampled_user():
    """Config 3's 160 users with the V2 target side (AutoSplit, 16 layers with the token FFN after
    every target layer, pooling); one user against the oracle; deterministic."""
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    wl, feats, w_split, ffn = synth.config3_v2()
    say(f"V2 config 3: {wl.batch.total_rows} rows, {wl.batch.total_t_rows} T rows")
    dw = DeviceWorkload(wl)
    meta = B.mask_build(dw.batch)
    P = feats.shape[0]
    ws = torch.empty(B.backbone_v2_workspace_bytes(dw.batch, dw.dims, 3, 1024), dtype=torch.uint8, device="cuda")
    fd, wd = _dev(feats), _dev(w_split)
    ffd = [_ffn_dev(w) for w in ffn]

    def run():
        x = dw.x.clone()
        B.autosplit(dw.batch, dw.dims, feats.shape[1], meta, fd, wd, x)
        B.backbone_v2_fwd(dw.batch, dw.dims, 4, 3, 1024, meta, dw.full, dw.target, ffd, x, ws)
        out = torch.empty((P, 512), dtype=torch.bfloat16, device="cuda")
        B.token_pool(dw.batch, dw.dims, meta, x, out)
        torch.cuda.synchronize()
        return to_np(x), to_np(out)

    x1, pooled1 = run()
    x2, pooled2 = run()
    np.testing.assert_array_equal(x1, x2)
    np.testing.assert_array_equal(pooled1, pooled2)
    u = int(np.argmin(wl.batch.user_rows))
    xr, full, tgt = rounded_inputs(wl)
    tr_all = ov.t_rows(wl.batch)
    x_in = xr.copy()
    x_in[tr_all] = om.bf16_round(ov.autosplit(om.bf16_round(feats), om.bf16_round(w_split), 4))
    rows = wl.batch.rows_of([u])
    sub = wl.batch.subset([u])
    ref = ov.backbone_v2(sub, x_in[rows], full, tgt, [_round_ffn(w) for w in ffn], wl.dims, 4, 3,
                         boundary=om.bf16_round)
    r = Report(TOL_BF16)
    t_u = ov.t_rows(sub)
    c_u = np.setdiff1d(np.arange(len(rows)), t_u)
    got_u, xin_u = x1[rows], x_in[rows]
    # 16 stored outputs for context rows; 28 for T rows (16 layers + 12 FFNs); twelve mixings are the
    # identity permutation, so branches are measured against the rows' own inputs
    r.branch(f"user {u} context rows", got_u[c_u], ref[c_u], xin_u[c_u], "bf16", roundings=16)
    r.branch(f"user {u} T rows", got_u[t_u], ref[t_u], xin_u[t_u], "bf16", roundings=28)
    r.check()
    # pooling at full size: every parent's pooled row is the mean of the device's own sub-token rows:
    # an fp32 sum of 4 terms (rounding error at most 3 * 2^-24 * sum|x|), an exact 1/4, one bf16
    # rounding (half an ulp of the result); the rows themselves are pinned above
    subs = x1[tr_all].reshape(-1, 4, x1.shape[1])
    ref_pool = subs.mean(axis=1)
    big = np.maximum(np.abs(ref_pool), np.abs(pooled1))
    half = np.exp2(np.floor(np.log2(np.maximum(big, 1e-30))) - 8)
    fp32_sum = 3 * 2.0 ** -24 * np.abs(subs).sum(axis=1) / 4
    assert np.all(np.abs(pooled1 - ref_pool) <= half + fp32_sum + 1e-30)
