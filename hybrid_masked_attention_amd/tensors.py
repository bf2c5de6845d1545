"""Host-to-device marshalling of batches, activations and weights.

Takes plain host arrays (any object with the attributes used below) and
returns the torch device tensors the binding passes to libmtfm: projection
weights and activations in the layer dtype, group-LayerNorm parameters in
fp32.  No computation besides dtype casts.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from . import binding as B

_FULL_KEYS = ("ln1_g", "ln1_b", "w_uqkv", "ln2_g", "ln2_b", "w_o")
_TARGET_KEYS = ("ln1_g", "ln1_b", "w_u", "w_q", "w_kv", "ln2_g", "ln2_b", "w_o")


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(a, dtype: str, device="cuda"):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=torch_dtype(dtype)).contiguous()


def weights_to_device(w: Dict[str, np.ndarray], dtype: str, device="cuda", keys=None):
    import torch
    out = {}
    for k, v in w.items():
        if keys is not None and k not in keys:
            continue
        if k.startswith("ln"):
            out[k] = torch.as_tensor(np.ascontiguousarray(v, dtype=np.float32)).to(device)
        else:
            out[k] = to_device(v, dtype, device)
    return out


def dims_of(d, dtype: str) -> B.CDims:
    return B.make_dims(d.d_model, d.n_q_heads, d.n_kv_heads, d.head_dim, d.ln_eps,
                       B.BF16 if dtype == "bf16" else B.F32)


class DeviceWorkload:
    """Device copies of a workload: batch, dims, X, per-layer weights."""

    def __init__(self, wl, device="cuda"):
        self.batch = B.DeviceBatch.from_synth(wl.batch, device)
        self.dims = dims_of(wl.dims, wl.dtype)
        self.dtype = wl.dtype
        self.x = to_device(wl.x, wl.dtype, device)
        self.full: List[Dict] = [weights_to_device(w, wl.dtype, device, _FULL_KEYS) for w in wl.full]
        self.target: List[Dict] = [weights_to_device(w, wl.dtype, device, _TARGET_KEYS) for w in wl.target]
        self.device = device
        self.split = int(wl.batch.split)

    def pack_s24(self, stream=None):
        """Add every layer's packed 2:4 projections to its weights: the forward and serving
        entry points then compute those projections with the pruned weights (bf16)."""
        for w in self.full:
            w.update(B.pack_full_s24(w, stream))
        for w in self.target:
            w.update(B.pack_target_s24(w, self.split, stream))
        return self
