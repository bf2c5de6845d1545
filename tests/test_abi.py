"""Host-side checks of the C ABI (no GPU needed; nothing here launches a kernel).

The library must load, export every entry point declared in include/mtfm.h,
size its metadata from the host lengths, and reject bad arguments with the
documented status before enqueuing anything.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtfm.h")


@pytest.fixture(scope="module")
def B():
    from hybrid_masked_attention_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from hybrid_masked_attention_amd import build
        build.build()
    binding.lib()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtfm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_entry_points(B):
    assert declared_functions() == sorted(B.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(B):
    L = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(B):
    assert B.status_str(0) == "MTFM_OK"
    assert B.status_str(-4) == "MTFM_E_WORKSPACE"


def test_timing_classes_match_the_header(B):
    """The binding's kernel-class numbers are the header's, and the library refuses a class past the
    last one (host bookkeeping only: nothing is recorded while no class is enabled)."""
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "mtfm.h")).read()
    enum = dict((k, int(v)) for k, v in re.findall(r"MTFM_K_(\w+) = (\d+)", text))
    assert enum.pop("COUNT") == 12
    for name, value in enum.items():
        assert getattr(B, "K_" + name) == value, name
    B.timing_enable([])
    assert B.timing_read(B.K_GEMM_OUT_T) == (0, 0.0)
    with pytest.raises(B.MtfmError):
        B.timing_read(12)


def _host_batch(B, lens, split=1, ts_r=None, ts_t=None):
    lens = np.asarray(lens, np.int32).reshape(-1, 3)
    ts_r = np.zeros(max(0, int(lens[:, 1].sum())), np.int32) if ts_r is None else ts_r
    ts_t = np.zeros(max(0, int(lens[:, 2].sum())), np.int32) if ts_t is None else ts_t
    return B.DeviceBatch(lens, split, ts_r, ts_t, device=None)


def test_meta_layout_counts_match_lengths(B):
    for wl in (synth.config0(), synth.config1(), synth.config2(4)):
        b = B.DeviceBatch.from_synth(wl.batch, device=None)
        lay = B.meta_layout(b)
        rows = wl.batch.user_rows
        assert lay.n_rows == wl.batch.total_rows
        assert lay.n_t_rows == wl.batch.total_t_rows
        assert lay.n_full_tiles == int(np.sum((rows + 63) // 64))
        assert lay.n_target_tiles == int(np.sum((wl.batch.split * wl.batch.lens[:, 2] + 63) // 64))
        assert lay.n_ctx_rows == int(wl.batch.lens[:, :2].sum())
        offs = [lay.off_user, lay.off_p, lay.off_n, lay.off_type, lay.off_full_tiles, lay.off_target_tiles,
                lay.off_ctx_rows, lay.off_parent_row, lay.off_full_order, lay.off_target_order, lay.off_tsort_q,
                lay.off_tsort_g, lay.off_target_tiles_sorted, lay.total_bytes]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert B.meta_bytes(b) == lay.total_bytes


def test_empty_batch_is_valid(B):
    b = _host_batch(B, np.zeros((0, 3), np.int32))
    lay = B.meta_layout(b)
    assert lay.n_rows == 0 and lay.n_full_tiles == 0


def test_mask_build_rejects_bad_batches(B):
    L = B.lib()
    fake = ctypes.c_void_p(0x1000)
    bad_split = _host_batch(B, [[2, 1, 1]], split=3)
    assert L.mtfm_mask_build(ctypes.byref(bad_split.c), fake, 1 << 20, None) == B.E_DIMS
    neg = _host_batch(B, [[2, -1, 1]])
    assert L.mtfm_mask_build(ctypes.byref(neg.c), fake, 1 << 20, None) == B.E_DIMS
    ok = _host_batch(B, [[2, 1, 1]])
    assert L.mtfm_mask_build(ctypes.byref(ok.c), None, 1 << 20, None) == B.E_NULL
    # device lengths missing (host-only batch)
    assert L.mtfm_mask_build(ctypes.byref(ok.c), fake, 1 << 20, None) == B.E_NULL
    assert L.mtfm_mask_build(None, fake, 1 << 20, None) == B.E_NULL


def _with_fake_device(b):
    b.c.lens_d = 0x2000
    b.c.ts_r_d = 0x3000
    b.c.ts_t_d = 0x4000
    return b


def test_mask_build_rejects_small_meta_buffer(B):
    L = B.lib()
    b = _with_fake_device(_host_batch(B, [[5, 3, 2]]))
    need = B.meta_bytes(b)
    assert L.mtfm_mask_build(ctypes.byref(b.c), ctypes.c_void_p(0x1000), need - 1, None) == B.E_WORKSPACE


def test_layer_argument_checks(B):
    L = B.lib()
    b = _with_fake_device(_host_batch(B, [[5, 3, 2]]))
    fake = ctypes.c_void_p(0x1000)
    w = B.CFullW(*([0x5000] * 6))
    good = B.make_dims(512, 8, 2, 64, dtype=B.BF16)
    need = B.workspace_bytes(b, good, B.OP_FULL)
    assert need > 0

    def call(dims, ws_bytes=need, weights=w, meta=fake):
        return L.mtfm_attn_full(ctypes.byref(b.c), ctypes.byref(dims), meta, ctypes.byref(weights), fake, fake,
                                fake, ws_bytes, None)
    assert call(good, need - 1) == B.E_WORKSPACE
    assert call(B.make_dims(512, 8, 3, 64)) == B.E_UNSUPPORTED      # H % G != 0
    assert call(B.make_dims(512, 8, 2, 48)) == B.E_UNSUPPORTED      # head_dim
    assert call(B.make_dims(512, 8, 2, 32, dtype=B.BF16)) == B.E_UNSUPPORTED
    assert call(B.make_dims(500, 8, 2, 64)) == B.E_UNSUPPORTED      # d_model % 64
    for width in (192, 384, 768, 2048):                              # row kernels: 64 * 2^k up to 1024
        assert call(B.make_dims(width, 8, 2, 64)) == B.E_UNSUPPORTED, width
        assert call(B.make_dims(512, width // 64, 1, 64)) == B.E_UNSUPPORTED, width   # H * dh
    assert B.workspace_bytes(b, B.make_dims(512, 12, 4, 64), B.OP_FULL) == 0       # H * dh = 768
    assert B.workspace_bytes(b, B.make_dims(128, 8, 2, 64), B.OP_FULL_BWD) == 0    # backward: d_model >= 256
    assert call(B.make_dims(0, 8, 2, 64)) == B.E_DIMS
    assert call(B.make_dims(512, 8, 2, 64, ln_eps=0.0)) == B.E_DIMS
    assert call(B.make_dims(512, 8, 2, 64, dtype=7)) == B.E_UNSUPPORTED
    assert call(good, meta=None) == B.E_NULL
    w_missing = B.CFullW(0x5000, 0x5000, None, 0x5000, 0x5000, 0x5000)
    assert call(good, weights=w_missing) == B.E_NULL
    tw = B.CTargetW(*([0x5000] * 7 + [None]))
    assert L.mtfm_attn_target(ctypes.byref(b.c), ctypes.byref(good), fake, ctypes.byref(tw), fake, fake, fake,
                              1 << 30, None) == B.E_NULL
    # backbone: negative block counts
    fw = (B.CFullW * 1)(w)
    tws = (B.CTargetW * 1)(B.CTargetW(*([0x5000] * 8)))
    assert L.mtfm_backbone_fwd(ctypes.byref(b.c), ctypes.byref(good), -1, 3, fake, fw, tws, fake, fake, 1 << 30,
                               None) == B.E_DIMS


def test_workspace_sizes_grow_with_rows(B):
    d = B.make_dims(512, 8, 2, 64)
    small = _host_batch(B, [[10, 5, 2]])
    big = _host_batch(B, [[1000, 500, 200]])
    for op in (B.OP_FULL, B.OP_TARGET, B.OP_BACKBONE):
        assert 0 < B.workspace_bytes(small, d, op) < B.workspace_bytes(big, d, op)
    assert B.workspace_bytes(small, B.make_dims(500, 8, 2, 64), B.OP_FULL) == 0   # invalid dims -> 0


def test_s24_pack_sizes_and_argument_checks(B):
    """2:4 packing ([explainer] §5.2.1): 9/8 byte per weight (8 bf16 kept values and one 16-bit
    position word per 32 weights); argument errors are reported before anything is enqueued."""
    L = B.lib()
    assert B.s24_pack_bytes(1280, 512) == 1280 * 512 * 9 // 8
    assert B.s24_pack_bytes(512, 512) == 512 * 512 + 512 * 512 // 8
    assert B.s24_pack_bytes(16, 48) == 0 and B.s24_pack_bytes(0, 64) == 0 and B.s24_pack_bytes(8, -32) == 0
    segs = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    rows = (ctypes.c_int32 * 2)(64, 32)
    need = B.s24_pack_bytes(96, 64)

    def call(k=64, n=2, out=0x40000, nbytes=need, s=segs, r=rows):
        return L.mtfm_s24_pack(s, r, n, k, ctypes.c_void_p(out) if out else None, nbytes, None)
    assert call(k=48) == B.E_DIMS
    assert call(n=0) == B.E_DIMS and call(n=17) == B.E_DIMS
    assert call(out=0) == B.E_NULL
    assert call(s=None) == B.E_NULL
    assert call(nbytes=need - 1) == B.E_WORKSPACE
    assert call(out=0x40008) == B.E_UNSUPPORTED                          # 16-byte alignment
    assert call(s=(ctypes.c_void_p * 2)(0x10000, 0x20004)) == B.E_UNSUPPORTED
    assert call(r=(ctypes.c_int32 * 2)(64, -1)) == B.E_DIMS
    assert call(s=(ctypes.c_void_p * 2)(0x10000, None)) == B.E_NULL
    assert call(r=(ctypes.c_int32 * 2)(0, 0)) == B.OK                   # nothing to pack


def test_packed_weights_need_bf16_and_alignment(B):
    """A packed 2:4 projection in the weight structs is read by the bf16 forward only: fp32 dims or
    a misaligned pointer is rejected before anything is enqueued."""
    L = B.lib()
    b = _with_fake_device(_host_batch(B, [[5, 3, 2]]))
    fake = ctypes.c_void_p(0x1000)
    f32 = B.make_dims(512, 8, 2, 64, dtype=B.F32)
    bf = B.make_dims(512, 8, 2, 64, dtype=B.BF16)

    def full(dims, w):
        need = B.workspace_bytes(b, dims, B.OP_FULL)
        return L.mtfm_attn_full(ctypes.byref(b.c), ctypes.byref(dims), fake, ctypes.byref(w), fake, fake, fake,
                                need, None)

    def target(dims, w):
        need = B.workspace_bytes(b, dims, B.OP_TARGET)
        return L.mtfm_attn_target(ctypes.byref(b.c), ctypes.byref(dims), fake, ctypes.byref(w), fake, fake, fake,
                                  need, None)
    assert full(f32, B.CFullW(*([0x5000] * 6), 0x6000, None)) == B.E_UNSUPPORTED
    assert full(f32, B.CFullW(*([0x5000] * 6), None, 0x6000)) == B.E_UNSUPPORTED
    assert full(bf, B.CFullW(*([0x5000] * 6), 0x6008, None)) == B.E_UNSUPPORTED
    assert target(f32, B.CTargetW(*([0x5000] * 8), 0x6000, None, None)) == B.E_UNSUPPORTED
    assert target(bf, B.CTargetW(*([0x5000] * 8), None, 0x6004, None)) == B.E_UNSUPPORTED


def test_serve_targets_noalloc_rejects_batches_beyond_its_scratch(B):
    """The entry point without a workspace has a fixed per-GPU scratch array; a candidate batch that
    needs more is refused on the host (MTFM_E_WORKSPACE) before any device call."""
    L = B.lib()
    cap = B.serve_targets_noalloc_max_bytes()
    assert cap == 64 << 20
    d = B.make_dims(512, 8, 2, 64, dtype=B.BF16)
    fake = ctypes.c_void_p(0x1000)
    fw = (B.CFullW * 1)(B.CFullW(*([0x5000] * 6)))
    tws = (B.CTargetW * 1)(B.CTargetW(*([0x5000] * 8)))
    # 12,000 candidate rows at d 512 need ~66 MB of scratch; 2,000 need ~11 MB
    for n_t, fits in ((3000, False), (500, True)):
        b = _with_fake_device(_host_batch(B, [[100, 20, n_t]], split=4))
        need = B.serve_workspace_bytes(b, d, 1, B.SERVE_TARGETS)
        assert (need <= cap) == fits
        cache = B.kv_cache_bytes(b, d, 1, 1)
        if not fits:
            assert L.mtfm_serve_targets_noalloc(ctypes.byref(b.c), ctypes.byref(d), 1, 1, fake, fw, tws, fake,
                                                cache, fake, None) == B.E_WORKSPACE
        # no layers: every host check passes and nothing is enqueued (no device call either)
        assert L.mtfm_serve_targets_noalloc(ctypes.byref(b.c), ctypes.byref(d), 0, 1, fake, fw, tws, fake,
                                            B.kv_cache_bytes(b, d, 0, 1), fake, None) == (B.OK if fits else
                                                                                           B.E_WORKSPACE)
        assert L.mtfm_serve_targets_noalloc(ctypes.byref(b.c), ctypes.byref(d), 1, 1, fake, fw, tws, fake,
                                            cache - 1, fake, None) == B.E_WORKSPACE
