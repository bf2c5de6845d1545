"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np

from oracle import model as om

# Activation bar: max|gpu - ref| <= TOL * max|ref| over each compared tensor
# (bf16 storage, fp32 accumulation).  The fp32 path gets a tighter bar.
TOL_BF16 = 1e-2
TOL_F32 = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return diff / scale if scale > 0 else diff


def half_ulp(v, dtype):
    """Half the spacing of representable numbers at |v| (bf16: 8 significant bits, fp32: 24)."""
    bits = 8 if dtype == "bf16" else 24
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 1e-30)
    return np.exp2(np.floor(np.log2(a)) - bits)


def branch_err(out_gpu, out_ref, x_ref, dtype, roundings=1):
    """Error of the residual branch dX = X' - X seen through the stored X'.

    X' is stored in `dtype`, so it carries up to half an ulp of |X'| of
    rounding whatever the branch is (`roundings` such roundings when X passed
    through that many stored layer outputs: the residual path carries each
    one through unchanged); that allowance is removed before the error is
    taken relative to max|dX_ref|.
    """
    out_gpu = np.asarray(out_gpu, np.float64)
    out_ref = np.asarray(out_ref, np.float64)
    allow = roundings * half_ulp(np.maximum(np.abs(out_gpu), np.abs(out_ref)), dtype)
    excess = np.maximum(np.abs(out_gpu - out_ref) - allow, 0.0)
    scale = float(np.max(np.abs(out_ref - np.asarray(x_ref, np.float64))))
    return float(excess.max()) / scale if scale > 0 else float(excess.max())


class Report:
    """Collects every comparison of a case, prints them, then asserts all."""

    def __init__(self, tol):
        self.tol = tol
        self.bad = []

    def close(self, name, got, ref):
        self.value(name, rel_err(got, ref))

    def branch(self, name, out_gpu, out_ref, x_ref, dtype, roundings=1):
        self.value(name, branch_err(out_gpu, out_ref, x_ref, dtype, roundings))

    def value(self, name, e):
        say(f"  {name}: {e:.3e} (bar {self.tol:.0e})")
        if not e <= self.tol:
            self.bad.append(f"{name}: {e:.3e} > {self.tol:.0e}")

    def check(self):
        assert not self.bad, "; ".join(self.bad)


def assert_close(name, got, ref, tol):
    r = Report(tol)
    r.close(name, got, ref)
    r.check()


def rounded_inputs(wl):
    """Inputs as the device sees them: bf16-rounded for the bf16 path."""
    if wl.dtype != "bf16":
        return wl.x.astype(np.float64), wl.full, wl.target
    r = om.bf16_round
    full = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl.full]
    tgt = [{k: (v if k.startswith("ln") else r(v)) for k, v in w.items()} for w in wl.target]
    return r(wl.x), full, tgt


def to_np(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def ws_tensor(ws, off, rows, width, dtype):
    """A [rows, width] view of the workspace at byte offset `off`."""
    import torch
    es = 2 if dtype == "bf16" else 4
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return ws[off:off + rows * width * es].view(tdt).view(rows, width)


def target_key_splits(batch, dims):
    """Key splits the library gives the target attention on its inference paths (the host rule:
    fill ~1,024 workgroup slots, at least 8 key tiles of the longest context per run, at most 16
    runs, fp32 partials within 16 MiB; 1 = none)."""
    lens = np.asarray(batch.lens, np.int64)
    t_rows = int((batch.split * lens[:, 2]).sum()) if len(lens) else 0
    if t_rows == 0:
        return 1
    tiles = int(((batch.split * lens[:, 2] + 63) // 64).sum())
    wgs = max(2 * tiles * dims.n_kv_heads, 1)
    part = max(t_rows * dims.n_q_heads * dims.head_dim * 4, 1)
    ctx = int((lens[:, 0] + lens[:, 1]).max())
    ks = min(1024 // wgs, (ctx + 63) // 64 // 8, 16, (16 << 20) // part)
    return ks if ks >= 2 else 1
