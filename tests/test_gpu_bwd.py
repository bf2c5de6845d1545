"""GPU parity of the backward pass against the oracle's hand-derived gradients.

The device runs bf16 storage with fp32 accumulation; the oracle runs float64
on the same bf16-rounded inputs and upstream gradient.  Every gradient tensor
(dX, each weight, each GLN parameter) must satisfy
max|gpu - ref| <= 1e-2 * max|ref|.
"""
import numpy as np
import pytest

import synth
from oracle import grad as og
from oracle import model as om
from tests._parity import TOL_BF16, Report, say, to_np

pytestmark = pytest.mark.gpu

FULL_KEYS = ("w_uqkv", "w_o", "ln1_g", "ln1_b", "ln2_g", "ln2_b")
TARGET_KEYS = ("w_u", "w_q", "w_kv", "w_o", "ln1_g", "ln1_b", "ln2_g", "ln2_b")


def _device_bwd(wl, kind, dy_np):
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload, to_device
    dw = DeviceWorkload(wl)
    meta = B.mask_build(dw.batch)
    op = B.OP_FULL_BWD if kind == "full" else B.OP_TARGET_BWD
    ws = B.workspace(dw.batch, dw.dims, op)
    dy = to_device(dy_np, "bf16")
    dx = torch.empty_like(dw.x)
    w = dw.full[0] if kind == "full" else dw.target[0]
    keys = FULL_KEYS if kind == "full" else TARGET_KEYS
    grads = {k: torch.full(tuple(w[k].shape), float("nan"), dtype=torch.float32, device="cuda") for k in keys}
    if kind == "full":
        B.attn_full_bwd(dw.batch, dw.dims, meta, w, dw.x, dy, dx, grads, ws)
    else:
        B.attn_target_bwd(dw.batch, dw.dims, meta, w, dw.x, dy, dx, grads, ws)
    torch.cuda.synchronize()
    return to_np(dx), {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}, to_np(dy), to_np(dw.x)


def _rounded(wl, kind):
    r = om.bf16_round
    w = wl.full[0] if kind == "full" else wl.target[0]
    return r(wl.x), {k: (v.astype(np.float64) if k.startswith("ln") else r(v)) for k, v in w.items()}


def _check(wl, kind, dy_np, users=None):
    say(f"backward parity: {wl.name} {kind} users={wl.batch.n_users} rows={wl.batch.total_rows}")
    dx, grads, dy_dev, x_dev = _device_bwd(wl, kind, dy_np)
    xr, wr = _rounded(wl, kind)
    np.testing.assert_array_equal(x_dev, xr)
    r = Report(TOL_BF16)
    if users is None:
        fn = og.full_layer_bwd if kind == "full" else og.target_layer_bwd
        ref = fn(wl.batch, xr, wr, wl.dims, dy_dev)
        r.close("dX", dx, ref["x"])
        for k in grads:
            r.close(f"d{k}", grads[k], ref[k])
    else:   # dX of a user depends on that user only: check sampled users one by one
        for u in users:
            sub = wl.batch.subset([u])
            rows = wl.batch.rows_of([u])
            fn = og.full_layer_bwd if kind == "full" else og.target_layer_bwd
            ref = fn(sub, xr[rows], wr, wl.dims, dy_dev[rows])
            r.close(f"dX user {u}", dx[rows], ref["x"])
        for k, v in grads.items():
            assert np.all(np.isfinite(v)), k
    r.check()
    return dx, grads


def _small(lens, split, seed, heads=(8, 2)):
    rng = np.random.default_rng(seed)
    batch = synth.make_batch(rng, np.asarray(lens, np.int32), split)
    dims = synth.Dims(512, heads[0], heads[1], 64)
    x = rng.standard_normal((batch.total_rows, 512)).astype(np.float32)
    wf = synth.full_weights(rng, dims, 0.05, 0.05)
    wt = synth.target_weights(rng, dims, split, 0.05, 0.05)
    dy = rng.standard_normal((batch.total_rows, 512)).astype(np.float32)
    return synth.Workload(f"bwd_small_{seed}", batch, dims, "bf16", x, full=[wf], target=[wt], dy=dy)


SMALL_LENS = [[130, 64, 17], [1, 0, 1], [63, 1, 0], [0, 0, 3], [65, 63, 33], [5, 70, 2], [0, 0, 0], [200, 30, 9]]


@pytest.mark.parametrize("split", [1, 4])
@pytest.mark.parametrize("kind", ["full", "target"])
def test_backward_small_ragged(kind, split):
    wl = _small(SMALL_LENS, split, 70 + split)
    _check(wl, kind, wl.dy)


@pytest.mark.parametrize("heads", [(8, 8), (8, 4), (8, 1)])
@pytest.mark.parametrize("kind", ["full", "target"])
def test_backward_other_gqa_ratios(kind, heads):
    """r = H/G of 1, 2 and 8 query heads per KV group: the dQ kernel's DMA split over r waves and
    the dK/dV kernel's head passes (one head per pass at r = 1, four passes at r = 8)."""
    wl = _small(SMALL_LENS, 4, 75 + heads[1], heads)
    _check(wl, kind, wl.dy)


@pytest.mark.parametrize("kind", ["full", "target"])
def test_weight_gradient_gemm_paths_agree(kind, monkeypatch):
    """The register-staged weight-gradient GEMM (used for operands past 2 GiB, forced here by
    MTFM_GEMM_TN_STAGED=1) and the DMA one accumulate the same rows in the same order: every
    gradient agrees bit for bit."""
    wl = _small(SMALL_LENS, 4, 79)
    dx1, g1 = _device_bwd(wl, kind, wl.dy)[:2]
    monkeypatch.setenv("MTFM_GEMM_TN_STAGED", "1")
    dx2, g2 = _device_bwd(wl, kind, wl.dy)[:2]
    np.testing.assert_array_equal(dx1, dx2)
    for k in g1:
        np.testing.assert_array_equal(g1[k], g2[k])


@pytest.mark.parametrize("kind", ["full", "target"])
def test_backward_config4_two_user_slice(kind):
    """Config 4's shapes (4096 H + 512 R + 256 x 4 T rows, d 1024, 16Q/4KV) on its first two users."""
    full = synth.config4()
    users = [0, 1]
    rows = full.batch.rows_of(users)
    wl = synth.Workload("cfg4_2users", full.batch.subset(users), full.dims, "bf16", full.x[rows],
                        full=full.full, target=full.target, dy=full.dy[rows])
    _check(wl, kind, wl.dy)


@pytest.mark.parametrize("kind", ["full", "target"])
def test_backward_config4_full_batch_sampled(kind):
    """All 64 users (the timed launch); dX of sampled users against the oracle; deterministic."""
    wl = synth.config4()
    dx1, g1 = _check(wl, kind, wl.dy, users=[5])
    dx2, g2 = _device_bwd(wl, kind, wl.dy)[:2]
    np.testing.assert_array_equal(dx1, dx2)
    for k in g1:
        np.testing.assert_array_equal(g1[k], g2[k])
