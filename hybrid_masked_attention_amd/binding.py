"""ctypes binding of libmtfm (argument marshalling only).

Every function here turns torch tensors into the plain pointers and sizes of
the C ABI declared in include/mtfm.h and calls it on the current torch
stream.  All computation happens in the HIP library; if libmtfm.so is missing
or fails to load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p, c_char_p
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MTFM_LIB selects another build of the library (the host-sanitizer build of
# the argument-checking tests); the default is the in-tree libmtfm.so.
LIB_PATH = os.environ.get("MTFM_LIB") or os.path.join(_HERE, "libmtfm.so")

OK, E_NULL, E_DIMS, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
OP_FULL, OP_TARGET, OP_BACKBONE, OP_FULL_BWD, OP_TARGET_BWD = 0, 1, 2, 3, 4
TILE = 64
UT_ROW, UT_ACT, UT_PARENT, UT_CTX, UT_FTILE, UT_TTILE, UT_TROW, UT_KTILE = range(8)
UT_COUNT = 8

# Names of the entry points declared in include/mtfm.h.
ENTRY_POINTS = [
    "mtfm_meta_bytes", "mtfm_meta_layout_of", "mtfm_mask_build", "mtfm_workspace_bytes",
    "mtfm_workspace_probe", "mtfm_attn_full", "mtfm_attn_target", "mtfm_backbone_fwd",
    "mtfm_attn_full_bwd", "mtfm_attn_target_bwd", "mtfm_timing_enable", "mtfm_timing_read",
    "mtfm_status_str", "mtfm_last_error", "mtfm_backbone_workspace_bytes",
    "mtfm_backbone_bwd_workspace_bytes", "mtfm_backbone_bwd_min_workspace_bytes", "mtfm_backbone_bwd",
    "mtfm_kv_cache_bytes", "mtfm_serve_workspace_bytes",
    "mtfm_serve_context", "mtfm_serve_targets", "mtfm_autosplit", "mtfm_token_ffn_workspace_bytes",
    "mtfm_token_ffn", "mtfm_token_pool", "mtfm_backbone_v2_workspace_bytes", "mtfm_backbone_v2_fwd",
    "mtfm_mask_dense", "mtfm_validate_batch", "mtfm_s24_pack_bytes", "mtfm_s24_pack",
    "mtfm_serve_targets_noalloc_max_bytes", "mtfm_serve_targets_noalloc",
]
BAD_ACTION_ORDER, BAD_LENGTHS = 1, 2
SERVE_CONTEXT, SERVE_TARGETS = 0, 1
(K_MASK, K_GLN, K_GEMM_UQKV, K_ATTN_FULL, K_GEMM_OUT, K_GEMM_KV, K_GEMM_T, K_ATTN_TARGET, K_BWD, K_V2,
 K_GLN_T, K_GEMM_OUT_T) = range(12)


class MtfmError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status}) {detail}".rstrip())


class CBatch(ctypes.Structure):
    _fields_ = [("n_users", c_int32), ("split", c_int32), ("lens_h", c_void_p), ("lens_d", c_void_p),
                ("ts_r_d", c_void_p), ("ts_t_d", c_void_p)]


class CDims(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("ln_eps", c_float), ("dtype", c_int32)]


FULL_W = ("ln1_g", "ln1_b", "w_uqkv", "ln2_g", "ln2_b", "w_o", "w_uqkv_s24", "w_o_s24")
TARGET_W = ("ln1_g", "ln1_b", "w_u", "w_q", "w_kv", "ln2_g", "ln2_b", "w_o", "w_t_s24", "w_kv_s24", "w_o_s24")


class CFullW(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in FULL_W]


class CTargetW(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in TARGET_W]


class CFullGrad(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("ln1_g", "ln1_b", "w_uqkv", "ln2_g", "ln2_b", "w_o")]


class CTargetGrad(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("ln1_g", "ln1_b", "w_u", "w_q", "w_kv", "ln2_g", "ln2_b", "w_o")]


class CFfnW(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("ln_g", "ln_b", "w_gate", "w_up", "w_down")]


class CMetaLayout(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in (
        "n_rows", "n_t_rows", "n_parents", "n_ctx_rows", "n_full_tiles", "n_target_tiles", "n_key_tiles",
        "off_user", "off_p",
        "off_n", "off_type", "off_full_tiles", "off_target_tiles", "off_ctx_rows", "off_parent_row",
        "n_full_order", "n_target_order", "off_full_order", "off_target_order",
        "off_tsort_q", "off_tsort_g", "off_target_tiles_sorted", "total_bytes")]


_lib = None


def lib():
    """The loaded libmtfm (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmtfm.so is not built ({LIB_PATH}); run python -m hybrid_masked_attention_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.mtfm_meta_bytes.argtypes = [P(CBatch)]; L.mtfm_meta_bytes.restype = c_size_t
    L.mtfm_meta_layout_of.argtypes = [P(CBatch), P(CMetaLayout)]; L.mtfm_meta_layout_of.restype = c_int32
    L.mtfm_mask_build.argtypes = [P(CBatch), c_void_p, c_size_t, c_void_p]; L.mtfm_mask_build.restype = c_int32
    L.mtfm_mask_dense.argtypes = [P(CBatch), c_void_p, c_int32, c_void_p, c_void_p]
    L.mtfm_mask_dense.restype = c_int32
    L.mtfm_validate_batch.argtypes = [P(CBatch), c_void_p, c_void_p]; L.mtfm_validate_batch.restype = c_int32
    L.mtfm_s24_pack_bytes.argtypes = [c_int32, c_int32]; L.mtfm_s24_pack_bytes.restype = c_size_t
    L.mtfm_s24_pack.argtypes = [P(c_void_p), P(c_int32), c_int32, c_int32, c_void_p, c_size_t, c_void_p]
    L.mtfm_s24_pack.restype = c_int32
    L.mtfm_workspace_bytes.argtypes = [P(CBatch), P(CDims), c_int32]; L.mtfm_workspace_bytes.restype = c_size_t
    L.mtfm_backbone_workspace_bytes.argtypes = [P(CBatch), P(CDims), c_int32]
    L.mtfm_backbone_workspace_bytes.restype = c_size_t
    L.mtfm_workspace_probe.argtypes = [P(CBatch), P(CDims), c_int32, P(c_int64), P(c_int64)]
    L.mtfm_workspace_probe.restype = c_int32
    L.mtfm_attn_full.argtypes = [P(CBatch), P(CDims), c_void_p, P(CFullW), c_void_p, c_void_p, c_void_p, c_size_t,
                                 c_void_p]
    L.mtfm_attn_full.restype = c_int32
    L.mtfm_attn_target.argtypes = [P(CBatch), P(CDims), c_void_p, P(CTargetW), c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p]
    L.mtfm_attn_target.restype = c_int32
    L.mtfm_backbone_fwd.argtypes = [P(CBatch), P(CDims), c_int32, c_int32, c_void_p, P(CFullW), P(CTargetW),
                                    c_void_p, c_void_p, c_size_t, c_void_p]
    L.mtfm_backbone_fwd.restype = c_int32
    L.mtfm_attn_full_bwd.argtypes = [P(CBatch), P(CDims), c_void_p, P(CFullW), c_void_p, c_void_p, c_void_p,
                                     P(CFullGrad), c_void_p, c_size_t, c_void_p]
    L.mtfm_attn_full_bwd.restype = c_int32
    L.mtfm_attn_target_bwd.argtypes = [P(CBatch), P(CDims), c_void_p, P(CTargetW), c_void_p, c_void_p, c_void_p,
                                       P(CTargetGrad), c_void_p, c_size_t, c_void_p]
    L.mtfm_attn_target_bwd.restype = c_int32
    L.mtfm_backbone_bwd_workspace_bytes.argtypes = [P(CBatch), P(CDims), c_int32, c_int32]
    L.mtfm_backbone_bwd_workspace_bytes.restype = c_size_t
    L.mtfm_backbone_bwd_min_workspace_bytes.argtypes = [P(CBatch), P(CDims), c_int32, c_int32]
    L.mtfm_backbone_bwd_min_workspace_bytes.restype = c_size_t
    L.mtfm_backbone_bwd.argtypes = [P(CBatch), P(CDims), c_int32, c_int32, c_void_p, P(CFullW), P(CTargetW),
                                    c_void_p, c_void_p, c_void_p, P(CFullGrad), P(CTargetGrad), c_void_p, c_size_t,
                                    c_void_p]
    L.mtfm_backbone_bwd.restype = c_int32
    L.mtfm_kv_cache_bytes.argtypes = [P(CBatch), P(CDims), c_int32, c_int32]; L.mtfm_kv_cache_bytes.restype = c_size_t
    L.mtfm_serve_workspace_bytes.argtypes = [P(CBatch), P(CDims), c_int32, c_int32]
    L.mtfm_serve_workspace_bytes.restype = c_size_t
    L.mtfm_serve_context.argtypes = [P(CBatch), P(CDims), c_int32, c_int32, c_void_p, P(CFullW), P(CTargetW),
                                     c_void_p, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    L.mtfm_serve_context.restype = c_int32
    L.mtfm_serve_targets.argtypes = [P(CBatch), P(CDims), c_int32, c_int32, c_void_p, P(CFullW), P(CTargetW),
                                     c_void_p, c_size_t, c_void_p, c_void_p, c_size_t, c_void_p]
    L.mtfm_serve_targets.restype = c_int32
    L.mtfm_serve_targets_noalloc_max_bytes.argtypes = []; L.mtfm_serve_targets_noalloc_max_bytes.restype = c_size_t
    L.mtfm_serve_targets_noalloc.argtypes = [P(CBatch), P(CDims), c_int32, c_int32, c_void_p, P(CFullW),
                                             P(CTargetW), c_void_p, c_size_t, c_void_p, c_void_p]
    L.mtfm_serve_targets_noalloc.restype = c_int32
    L.mtfm_autosplit.argtypes = [P(CBatch), P(CDims), c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    L.mtfm_autosplit.restype = c_int32
    L.mtfm_token_ffn_workspace_bytes.argtypes = [P(CBatch), P(CDims), c_int32]
    L.mtfm_token_ffn_workspace_bytes.restype = c_size_t
    L.mtfm_token_ffn.argtypes = [P(CBatch), P(CDims), c_int32, c_void_p, P(CFfnW), c_void_p, c_void_p, c_size_t,
                                 c_void_p]
    L.mtfm_token_ffn.restype = c_int32
    L.mtfm_token_pool.argtypes = [P(CBatch), P(CDims), c_void_p, c_void_p, c_void_p, c_void_p]
    L.mtfm_token_pool.restype = c_int32
    L.mtfm_backbone_v2_workspace_bytes.argtypes = [P(CBatch), P(CDims), c_int32, c_int32]
    L.mtfm_backbone_v2_workspace_bytes.restype = c_size_t
    L.mtfm_backbone_v2_fwd.argtypes = [P(CBatch), P(CDims), c_int32, c_int32, c_int32, c_void_p, P(CFullW),
                                       P(CTargetW), P(CFfnW), c_void_p, c_void_p, c_size_t, c_void_p]
    L.mtfm_backbone_v2_fwd.restype = c_int32
    L.mtfm_timing_enable.argtypes = [ctypes.c_uint32]; L.mtfm_timing_enable.restype = c_int32
    L.mtfm_timing_read.argtypes = [c_int32, P(c_int64), P(ctypes.c_double)]; L.mtfm_timing_read.restype = c_int32
    L.mtfm_status_str.argtypes = [c_int32]; L.mtfm_status_str.restype = c_char_p
    L.mtfm_last_error.argtypes = []; L.mtfm_last_error.restype = c_char_p
    _lib = L
    return L


def status_str(s: int) -> str:
    try:
        return lib().mtfm_status_str(int(s)).decode()
    except Exception:  # noqa: BLE001 - used while formatting another error
        return str(s)


def _check(status: int, where: str):
    if status != OK:
        detail = lib().mtfm_last_error().decode() if status == E_HIP else ""
        raise MtfmError(status, where, detail)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


# ---------------------------------------------------------------------------
class DeviceBatch:
    """A jagged batch on the device plus the host lengths, as the C struct wants it.

    lens: int32 [B, 3] (L_H, L_R, L_T parents); ts_r / ts_t int32 (numpy or
    torch).  `device` is a torch device string or None for a host-only batch
    (enough for sizes and argument checks).
    """

    def __init__(self, lens, split: int, ts_r, ts_t, device: Optional[str] = "cuda"):
        import torch
        self.lens_h = torch.as_tensor(np.ascontiguousarray(np.asarray(lens, dtype=np.int32).reshape(-1, 3)))
        self.split = int(split)
        self.n_users = int(self.lens_h.shape[0])
        ts_r = torch.as_tensor(np.ascontiguousarray(np.asarray(ts_r, dtype=np.int32)))
        ts_t = torch.as_tensor(np.ascontiguousarray(np.asarray(ts_t, dtype=np.int32)))
        if device is not None:
            self.lens_d = self.lens_h.to(device)
            self.ts_r_d = ts_r.to(device)
            self.ts_t_d = ts_t.to(device)
        else:
            self.lens_d = self.ts_r_d = self.ts_t_d = None
        self.c = CBatch(self.n_users, self.split, _ptr(self.lens_h), _ptr(self.lens_d),
                        _ptr(self.ts_r_d) if (self.ts_r_d is not None and self.ts_r_d.numel()) else None,
                        _ptr(self.ts_t_d) if (self.ts_t_d is not None and self.ts_t_d.numel()) else None)

    @classmethod
    def from_synth(cls, b, device="cuda"):
        return cls(b.lens, b.split, b.ts_r, b.ts_t, device)


def make_dims(d_model, n_q_heads, n_kv_heads, head_dim, ln_eps=1e-5, dtype=BF16) -> CDims:
    return CDims(int(d_model), int(n_q_heads), int(n_kv_heads), int(head_dim), float(ln_eps), int(dtype))


def meta_layout(batch: DeviceBatch) -> CMetaLayout:
    out = CMetaLayout()
    _check(lib().mtfm_meta_layout_of(ctypes.byref(batch.c), ctypes.byref(out)), "mtfm_meta_layout_of")
    return out


def meta_bytes(batch: DeviceBatch) -> int:
    return int(lib().mtfm_meta_bytes(ctypes.byref(batch.c)))


def mask_build(batch: DeviceBatch, meta=None, stream=None):
    """Build the mask metadata into `meta` (a uint8 device tensor; allocated if None)."""
    import torch
    nb = meta_bytes(batch)
    if meta is None:
        meta = torch.empty(max(nb, 1), dtype=torch.uint8, device=batch.lens_d.device)
    _check(lib().mtfm_mask_build(ctypes.byref(batch.c), _ptr(meta), meta.numel(), _stream(stream)), "mtfm_mask_build")
    return meta


def mask_dense(batch: DeviceBatch, meta, user: int, stream=None):
    """Debug: the dense [N][N] uint8 visibility matrix of one user (device tensor), from the metadata."""
    import torch
    lh, lr, lt = (int(v) for v in batch.lens_h[user])
    n = lh + lr + batch.split * lt
    out = torch.empty((n, n), dtype=torch.uint8, device=batch.lens_d.device)
    _check(lib().mtfm_mask_dense(ctypes.byref(batch.c), _ptr(meta), int(user), _ptr(out) if n else None,
                                 _stream(stream)), "mtfm_mask_dense")
    return out


def validate_batch(batch: DeviceBatch, stream=None) -> int:
    """Debug: bit mask of the data-level contract violations of the batch (0 = none); reads the flag back."""
    import torch
    flags = torch.full((1,), -1, dtype=torch.int32, device=batch.lens_d.device)
    _check(lib().mtfm_validate_batch(ctypes.byref(batch.c), _ptr(flags), _stream(stream)), "mtfm_validate_batch")
    return int(flags.item())


def meta_views(meta, layout: CMetaLayout, n_users: int) -> Dict[str, "object"]:
    """Typed views of the metadata arrays (torch tensors aliasing `meta`)."""
    import torch

    def view(off, count, dtype, shape=None):
        itemsize = torch.empty(0, dtype=dtype).element_size()
        t = meta[off:off + count * itemsize].view(dtype)
        return t.view(*shape) if shape else t
    L = layout
    return {
        "user": view(L.off_user, UT_COUNT * (n_users + 1), torch.int32, (UT_COUNT, n_users + 1)),
        "p": view(L.off_p, L.n_rows, torch.int32),
        "n": view(L.off_n, L.n_rows, torch.int32),
        "row_type": view(L.off_type, L.n_rows, torch.uint8),
        "full_tiles": view(L.off_full_tiles, L.n_full_tiles * 8, torch.int32, (L.n_full_tiles, 8)),
        "target_tiles": view(L.off_target_tiles, L.n_target_tiles * 8, torch.int32, (L.n_target_tiles, 8)),
        "ctx_rows": view(L.off_ctx_rows, L.n_ctx_rows, torch.int32),
        "parent_row": view(L.off_parent_row, L.n_parents, torch.int32),
        "full_order": view(L.off_full_order, L.n_full_order, torch.int32),
        "target_order": view(L.off_target_order, L.n_target_order, torch.int32),
        "tsort_q": view(L.off_tsort_q, L.n_t_rows, torch.int32),
        "tsort_g": view(L.off_tsort_g, L.n_t_rows, torch.int32),
        "target_tiles_sorted": view(L.off_target_tiles_sorted, L.n_target_tiles * 8, torch.int32,
                                    (L.n_target_tiles, 8)),
    }


def workspace_bytes(batch: DeviceBatch, dims: CDims, op: int) -> int:
    return int(lib().mtfm_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(op)))


def backbone_workspace_bytes(batch: DeviceBatch, dims: CDims, k_target: int) -> int:
    return int(lib().mtfm_backbone_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(k_target)))


def workspace(batch: DeviceBatch, dims: CDims, op: int, device="cuda", k_target: int = 0):
    """Workspace for `op`; for the backbone, pass k_target to size the bf16
    path that computes a block's target-layer context stage once."""
    import torch
    n = backbone_workspace_bytes(batch, dims, k_target) if (op == OP_BACKBONE and k_target) else \
        workspace_bytes(batch, dims, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def workspace_probe(batch: DeviceBatch, dims: CDims, op: int):
    a, y = c_int64(), c_int64()
    _check(lib().mtfm_workspace_probe(ctypes.byref(batch.c), ctypes.byref(dims), int(op), ctypes.byref(a),
                                      ctypes.byref(y)), "mtfm_workspace_probe")
    return int(a.value), int(y.value)


def full_w(w: Dict[str, "object"]) -> CFullW:
    """Weight struct of a full layer; the packed 2:4 fields are taken when the dict has them."""
    return CFullW(*[_ptr(w.get(n)) for n in FULL_W])


def target_w(w: Dict[str, "object"]) -> CTargetW:
    """Weight struct of a target layer; the packed 2:4 fields are taken when the dict has them."""
    return CTargetW(*[_ptr(w.get(n)) for n in TARGET_W])


def s24_pack_bytes(rows: int, k: int) -> int:
    return int(lib().mtfm_s24_pack_bytes(int(rows), int(k)))


def s24_pack(segs, stream=None):
    """2:4-prune and pack bf16 device matrices [rows_i][k] (stacked in order) -> uint8 device tensor."""
    import torch
    k = int(segs[0].shape[-1])
    rows = [int(t.shape[0]) for t in segs]
    if not all(t.dtype == torch.bfloat16 and t.is_contiguous() and t.dim() == 2 and int(t.shape[-1]) == k
               for t in segs):
        raise ValueError("s24_pack: segments must be contiguous 2-D bf16 tensors of one width")
    nbytes = s24_pack_bytes(sum(rows), k)
    out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=segs[0].device)
    ptrs = (c_void_p * len(segs))(*[t.data_ptr() for t in segs])
    nrows = (c_int32 * len(segs))(*rows)
    _check(lib().mtfm_s24_pack(ptrs, nrows, len(segs), k, _ptr(out), nbytes, _stream(stream)), "mtfm_s24_pack")
    return out


def pack_full_s24(w: Dict[str, "object"], stream=None) -> Dict[str, "object"]:
    """The packed 2:4 projections of a full layer (keys w_uqkv_s24, w_o_s24)."""
    return {"w_uqkv_s24": s24_pack([w["w_uqkv"]], stream), "w_o_s24": s24_pack([w["w_o"]], stream)}


def pack_target_s24(w: Dict[str, "object"], split: int, stream=None) -> Dict[str, "object"]:
    """The packed 2:4 projections of a target layer (keys w_t_s24, w_kv_s24, w_o_s24); w_q is [split][H*dh][d]."""
    segs = []
    for z in range(split):
        segs += [w["w_u"], w["w_q"][z], w["w_kv"]]
    return {"w_t_s24": s24_pack(segs, stream), "w_kv_s24": s24_pack([w["w_kv"]], stream),
            "w_o_s24": s24_pack([w["w_o"]], stream)}


def attn_full(batch, dims, meta, w, x_in, x_out, ws, stream=None):
    cw = full_w(w)
    _check(lib().mtfm_attn_full(ctypes.byref(batch.c), ctypes.byref(dims), _ptr(meta), ctypes.byref(cw),
                                _ptr(x_in), _ptr(x_out), _ptr(ws), ws.numel(), _stream(stream)), "mtfm_attn_full")
    return x_out


def attn_target(batch, dims, meta, w, x_in, x_out, ws, stream=None):
    cw = target_w(w)
    _check(lib().mtfm_attn_target(ctypes.byref(batch.c), ctypes.byref(dims), _ptr(meta), ctypes.byref(cw),
                                  _ptr(x_in), _ptr(x_out), _ptr(ws), ws.numel(), _stream(stream)), "mtfm_attn_target")
    return x_out


def backbone_fwd(batch, dims, n_blocks, k_target, meta, full: Sequence[Dict], tgt: Sequence[Dict], x_inout, ws,
                 stream=None):
    fa = (CFullW * max(1, len(full)))(*[full_w(w) for w in full])
    ta = (CTargetW * max(1, len(tgt)))(*[target_w(w) for w in tgt])
    _check(lib().mtfm_backbone_fwd(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks), int(k_target),
                                   _ptr(meta), fa, ta, _ptr(x_inout), _ptr(ws), ws.numel(), _stream(stream)),
           "mtfm_backbone_fwd")
    return x_inout


def attn_full_bwd(batch, dims, meta, w, x_in, dy, dx, grads: Dict, ws, stream=None):
    cw = full_w(w)
    cg = CFullGrad(*[_ptr(grads[n]) for n in ("ln1_g", "ln1_b", "w_uqkv", "ln2_g", "ln2_b", "w_o")])
    _check(lib().mtfm_attn_full_bwd(ctypes.byref(batch.c), ctypes.byref(dims), _ptr(meta), ctypes.byref(cw),
                                    _ptr(x_in), _ptr(dy), _ptr(dx), ctypes.byref(cg), _ptr(ws), ws.numel(),
                                    _stream(stream)), "mtfm_attn_full_bwd")
    return dx


def attn_target_bwd(batch, dims, meta, w, x_in, dy, dx, grads: Dict, ws, stream=None):
    cw = target_w(w)
    cg = CTargetGrad(*[_ptr(grads[n]) for n in ("ln1_g", "ln1_b", "w_u", "w_q", "w_kv", "ln2_g", "ln2_b", "w_o")])
    _check(lib().mtfm_attn_target_bwd(ctypes.byref(batch.c), ctypes.byref(dims), _ptr(meta), ctypes.byref(cw),
                                      _ptr(x_in), _ptr(dy), _ptr(dx), ctypes.byref(cg), _ptr(ws), ws.numel(),
                                      _stream(stream)), "mtfm_attn_target_bwd")
    return dx


FULL_GRAD_KEYS = ("ln1_g", "ln1_b", "w_uqkv", "ln2_g", "ln2_b", "w_o")
TARGET_GRAD_KEYS = ("ln1_g", "ln1_b", "w_u", "w_q", "w_kv", "ln2_g", "ln2_b", "w_o")


def backbone_bwd_workspace_bytes(batch: DeviceBatch, dims: CDims, n_blocks: int, k_target: int) -> int:
    return int(lib().mtfm_backbone_bwd_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks),
                                                       int(k_target)))


def backbone_bwd_min_workspace_bytes(batch: DeviceBatch, dims: CDims, n_blocks: int, k_target: int) -> int:
    """Smallest workspace mtfm_backbone_bwd accepts (each layer backward then recomputes its intermediates)."""
    return int(lib().mtfm_backbone_bwd_min_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks),
                                                           int(k_target)))


def backbone_bwd(batch, dims, n_blocks, k_target, meta, full: Sequence[Dict], tgt: Sequence[Dict], x_in, dy, dx,
                 full_grads: Sequence[Dict], tgt_grads: Sequence[Dict], ws, stream=None):
    """dL/dX_in into dx and every layer's gradients (dicts of fp32 tensors shaped like the weights)."""
    fa = (CFullW * max(1, len(full)))(*[full_w(w) for w in full])
    ta = (CTargetW * max(1, len(tgt)))(*[target_w(w) for w in tgt])
    fg = (CFullGrad * max(1, len(full_grads)))(*[CFullGrad(*[_ptr(g[n]) for n in FULL_GRAD_KEYS])
                                                 for g in full_grads])
    tg = (CTargetGrad * max(1, len(tgt_grads)))(*[CTargetGrad(*[_ptr(g[n]) for n in TARGET_GRAD_KEYS])
                                                  for g in tgt_grads])
    _check(lib().mtfm_backbone_bwd(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks), int(k_target),
                                   _ptr(meta), fa, ta, _ptr(x_in), _ptr(dy), _ptr(dx), fg, tg, _ptr(ws), ws.numel(),
                                   _stream(stream)), "mtfm_backbone_bwd")
    return dx


def kv_cache_bytes(batch: DeviceBatch, dims: CDims, n_blocks: int, k_target: int) -> int:
    return int(lib().mtfm_kv_cache_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks), int(k_target)))


def serve_workspace_bytes(batch: DeviceBatch, dims: CDims, k_target: int, phase: int) -> int:
    return int(lib().mtfm_serve_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(k_target),
                                                int(phase)))


def serve_context(batch, dims, n_blocks, k_target, meta, full: Sequence[Dict], tgt: Sequence[Dict], x_inout,
                  kv_cache, ws, stream=None):
    """Context rows through the stack (in place) and every layer's K / V^T of them into kv_cache."""
    fa = (CFullW * max(1, len(full)))(*[full_w(w) for w in full])
    ta = (CTargetW * max(1, len(tgt)))(*[target_w(w) for w in tgt])
    _check(lib().mtfm_serve_context(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks), int(k_target),
                                    _ptr(meta), fa, ta, _ptr(x_inout), _ptr(kv_cache), kv_cache.numel(), _ptr(ws),
                                    ws.numel(), _stream(stream)), "mtfm_serve_context")
    return x_inout


def serve_targets(batch, dims, n_blocks, k_target, meta, full: Sequence[Dict], tgt: Sequence[Dict], kv_cache,
                  x_t, ws, stream=None):
    """T rows ([split * sum L_T][d], T-row order) through the stack (in place) against the cached context."""
    fa = (CFullW * max(1, len(full)))(*[full_w(w) for w in full])
    ta = (CTargetW * max(1, len(tgt)))(*[target_w(w) for w in tgt])
    _check(lib().mtfm_serve_targets(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks), int(k_target),
                                    _ptr(meta), fa, ta, _ptr(kv_cache), kv_cache.numel(), _ptr(x_t), _ptr(ws),
                                    ws.numel(), _stream(stream)), "mtfm_serve_targets")
    return x_t


def serve_targets_noalloc_max_bytes() -> int:
    return int(lib().mtfm_serve_targets_noalloc_max_bytes())


def serve_targets_noalloc(batch, dims, n_blocks, k_target, meta, full: Sequence[Dict], tgt: Sequence[Dict],
                          kv_cache, x_t, stream=None):
    """serve_targets with the library's static per-GPU scratch instead of a workspace (allocates nothing)."""
    fa = (CFullW * max(1, len(full)))(*[full_w(w) for w in full])
    ta = (CTargetW * max(1, len(tgt)))(*[target_w(w) for w in tgt])
    _check(lib().mtfm_serve_targets_noalloc(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks), int(k_target),
                                            _ptr(meta), fa, ta, _ptr(kv_cache), kv_cache.numel(), _ptr(x_t),
                                            _stream(stream)), "mtfm_serve_targets_noalloc")
    return x_t


FFN_KEYS = ("ln_g", "ln_b", "w_gate", "w_up", "w_down")


def ffn_w(w: Dict[str, "object"]) -> CFfnW:
    return CFfnW(*[_ptr(w[n]) for n in FFN_KEYS])


def autosplit(batch, dims, d_in, meta, feats, w_split, x, stream=None):
    """The T rows of x from the parents' features ([n_parents][d_in]) through the AutoSplit map."""
    _check(lib().mtfm_autosplit(ctypes.byref(batch.c), ctypes.byref(dims), int(d_in), _ptr(meta), _ptr(feats),
                                _ptr(w_split), _ptr(x), _stream(stream)), "mtfm_autosplit")
    return x


def token_ffn_workspace_bytes(batch: DeviceBatch, dims: CDims, d_ff: int) -> int:
    return int(lib().mtfm_token_ffn_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(d_ff)))


def token_ffn(batch, dims, d_ff, meta, w: Dict, x, ws, stream=None):
    cw = ffn_w(w)
    _check(lib().mtfm_token_ffn(ctypes.byref(batch.c), ctypes.byref(dims), int(d_ff), _ptr(meta), ctypes.byref(cw),
                                _ptr(x), _ptr(ws), ws.numel(), _stream(stream)), "mtfm_token_ffn")
    return x


def token_pool(batch, dims, meta, x, out, stream=None):
    _check(lib().mtfm_token_pool(ctypes.byref(batch.c), ctypes.byref(dims), _ptr(meta), _ptr(x), _ptr(out),
                                 _stream(stream)), "mtfm_token_pool")
    return out


def backbone_v2_workspace_bytes(batch: DeviceBatch, dims: CDims, k_target: int, d_ff: int) -> int:
    return int(lib().mtfm_backbone_v2_workspace_bytes(ctypes.byref(batch.c), ctypes.byref(dims), int(k_target),
                                                      int(d_ff)))


def backbone_v2_fwd(batch, dims, n_blocks, k_target, d_ff, meta, full: Sequence[Dict], tgt: Sequence[Dict],
                    ffn: Sequence[Dict], x_inout, ws, stream=None):
    fa = (CFullW * max(1, len(full)))(*[full_w(w) for w in full])
    ta = (CTargetW * max(1, len(tgt)))(*[target_w(w) for w in tgt])
    fn = (CFfnW * max(1, len(ffn)))(*[ffn_w(w) for w in ffn])
    _check(lib().mtfm_backbone_v2_fwd(ctypes.byref(batch.c), ctypes.byref(dims), int(n_blocks), int(k_target),
                                      int(d_ff), _ptr(meta), fa, ta, fn, _ptr(x_inout), _ptr(ws), ws.numel(),
                                      _stream(stream)), "mtfm_backbone_v2_fwd")
    return x_inout


def timing_enable(classes: Sequence[int]):
    """Bracket launches of the given kernel classes with HIP events (empty = off)."""
    mask = 0
    for k in classes:
        mask |= 1 << int(k)
    _check(lib().mtfm_timing_enable(mask), "mtfm_timing_enable")


def timing_read(kclass: int):
    """(launches, total ms) recorded for a kernel class since the last read."""
    n, ms = c_int64(), ctypes.c_double()
    _check(lib().mtfm_timing_read(int(kclass), ctypes.byref(n), ctypes.byref(ms)), "mtfm_timing_read")
    return int(n.value), float(ms.value)
