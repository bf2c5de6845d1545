"""The candidate pass without a workspace (mtfm_serve_targets_noalloc) on the GPU.

It must compute exactly what mtfm_serve_targets computes with a caller
workspace: the same kernels and shapes, only the scratch memory differs.
Checked bit for bit on two calls in a row over one context cache, the second
with fewer candidates (the static scratch keeps the first call's contents),
and once more in the first shape after the smaller one.
"""
import numpy as np
import pytest

import synth
from tests._parity import say, to_np
from tests.test_gpu_serve import _serve_context, _small

pytestmark = pytest.mark.gpu


def _candidates(wl, rng, n_t):
    """The same users and context with other candidates: n_t[u] parents, fresh exposure times."""
    lens = wl.batch.lens.copy()
    lens[:, 2] = n_t
    ts_t = rng.integers(0, synth.TS_HIGH, int(lens[:, 2].sum())).astype(np.int32)
    return synth.Batch(lens, wl.batch.split, wl.batch.ts_r, ts_t)


def test_serve_targets_noalloc_matches_workspace_entry_point():
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    wl = _small(4, 150)
    dw = DeviceWorkload(wl)
    _, cache = _serve_context(wl, dw, B, torch)
    rng = np.random.default_rng(151)
    big = rng.integers(3, 25, wl.batch.n_users)
    small = np.maximum(big // 3 - 1, 0)
    small[1] = 0
    for call, n_t in enumerate((big, small, big)):
        cb = _candidates(wl, rng, n_t)
        db = B.DeviceBatch.from_synth(cb)
        meta = B.mask_build(db)
        n_rows = cb.total_t_rows
        need = B.serve_workspace_bytes(db, dw.dims, wl.k_target, B.SERVE_TARGETS)
        say(f"noalloc call {call}: {n_rows} T rows, scratch {need} of {B.serve_targets_noalloc_max_bytes()} bytes")
        assert 0 < need <= B.serve_targets_noalloc_max_bytes()
        x0 = torch.as_tensor(rng.standard_normal((n_rows, wl.dims.d_model)).astype(np.float32),
                             device="cuda").to(torch.bfloat16)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = x0.clone()
        B.serve_targets(db, dw.dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, cache, ref, ws)
        got = x0.clone()
        B.serve_targets_noalloc(db, dw.dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, cache, got)
        torch.cuda.synchronize()
        a, b = to_np(got), to_np(ref)
        assert np.all(np.isfinite(a))
        assert not np.array_equal(a, to_np(x0)), "the pass changed nothing"
        np.testing.assert_array_equal(a, b)
