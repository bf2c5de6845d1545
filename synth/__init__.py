"""Seeded synthetic inputs for the hybrid H/R/T attention backbone.

This module only draws numbers: jagged lengths, timestamps, activations,
weights and group-LayerNorm parameters.  It holds none of the method's
arithmetic (no mask, no attention, no normalisation), so both the CPU oracle
and the HIP path can be fed from it without sharing any computation.

The pages measure on private logs; these batches stand in for them with the
shapes the pages describe: thousand-token user sequences made of history (H),
real-time (R) and target (T) tokens, integer timestamps, and per-user
aggregation of targets (explainer [dingyadong.top, "美团推荐大模型 MTFM ...
深度硬核解析"] §2.1.3 and §3; Meituan blog ["MTFM：美团统一推荐基座大模型在外卖
多业务场景的落地实践"] §4.1).

Generation order for a config with seed s (numpy ``default_rng(s)``):
lengths, R timestamps (uniform ints in [0, 1000), sorted per user), target
exposure timestamps (uniform ints), activations X, weights, GLN parameters.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

TS_HIGH = 1000


@dataclass
class Batch:
    """A jagged user-level batch.

    lens[u] = (L_H, L_R, L_T) with L_T counted in parent targets; each parent
    expands into ``split`` T rows (target-major sub-token order).  Rows of a
    user are ordered H, R, T and users are packed back to back.
    """

    lens: np.ndarray          # [B, 3] int32
    split: int                # S = 1 or 4
    ts_r: np.ndarray          # [sum L_R] int32, ascending within each user
    ts_t: np.ndarray          # [sum L_T] int32, one exposure time per parent

    @property
    def n_users(self) -> int:
        return int(self.lens.shape[0])

    @property
    def user_rows(self) -> np.ndarray:
        l = self.lens.astype(np.int64)
        return l[:, 0] + l[:, 1] + self.split * l[:, 2]

    @property
    def row_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.user_rows)]).astype(np.int64)

    @property
    def total_rows(self) -> int:
        return int(self.user_rows.sum())

    @property
    def total_t_rows(self) -> int:
        return int(self.split * self.lens[:, 2].astype(np.int64).sum())

    @property
    def r_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens[:, 1].astype(np.int64))])

    @property
    def t_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens[:, 2].astype(np.int64))])

    def user(self, u: int) -> "Batch":
        """The one-user batch holding user ``u``."""
        return self.subset([u])

    def subset(self, users: List[int]) -> "Batch":
        ro, to = self.r_off, self.t_off
        ts_r = np.concatenate([self.ts_r[ro[u]:ro[u + 1]] for u in users]) if users else np.zeros(0, np.int32)
        ts_t = np.concatenate([self.ts_t[to[u]:to[u + 1]] for u in users]) if users else np.zeros(0, np.int32)
        return Batch(self.lens[users].copy(), self.split, ts_r.astype(np.int32), ts_t.astype(np.int32))

    def rows_of(self, users: List[int]) -> np.ndarray:
        off = self.row_off
        return np.concatenate([np.arange(off[u], off[u + 1]) for u in users]) if users else np.zeros(0, np.int64)


@dataclass
class Dims:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ln_eps: float = 1e-5


@dataclass
class Workload:
    name: str
    batch: Batch
    dims: Dims
    dtype: str                           # "f32" or "bf16"
    x: np.ndarray                        # [total_rows, d_model] float32
    full: List[Dict[str, np.ndarray]] = field(default_factory=list)
    target: List[Dict[str, np.ndarray]] = field(default_factory=list)
    n_blocks: int = 0
    k_target: int = 0
    dy: Optional[np.ndarray] = None      # upstream gradient for backward configs


def _sorted_ts(rng, n):
    return np.sort(rng.integers(0, TS_HIGH, size=n)).astype(np.int32)


def make_batch(rng, lens: np.ndarray, split: int) -> Batch:
    lens = np.asarray(lens, dtype=np.int32).reshape(-1, 3)
    ts_r = [_sorted_ts(rng, int(l)) for l in lens[:, 1]]
    ts_t = [rng.integers(0, TS_HIGH, size=int(l)).astype(np.int32) for l in lens[:, 2]]
    cat = lambda xs: np.concatenate(xs).astype(np.int32) if xs else np.zeros(0, np.int32)
    return Batch(lens, split, cat(ts_r), cat(ts_t))


def gln_params(rng, width: int) -> Dict[str, np.ndarray]:
    """Per-row-type (H, R, T) affine parameters, [3, width] each.

    gamma = 1 + 0.1 N(0,1) and beta = 0.1 N(0,1) so that the type indexing is
    exercised (the pages fix no values for them).
    """
    return {"g": (1.0 + 0.1 * rng.standard_normal((3, width))).astype(np.float32),
            "b": (0.1 * rng.standard_normal((3, width))).astype(np.float32)}


def full_weights(rng, dims: Dims, w_std: float, wo_std: float) -> Dict[str, np.ndarray]:
    d, H, G, dh = dims.d_model, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    w1 = (w_std * rng.standard_normal((2 * H * dh + 2 * G * dh, d))).astype(np.float32)
    wo = (wo_std * rng.standard_normal((d, H * dh))).astype(np.float32)
    p1, p2 = gln_params(rng, d), gln_params(rng, H * dh)
    return {"w_uqkv": w1, "w_o": wo, "ln1_g": p1["g"], "ln1_b": p1["b"],
            "ln2_g": p2["g"], "ln2_b": p2["b"]}


def target_weights(rng, dims: Dims, split: int, w_std: float, wo_std: float) -> Dict[str, np.ndarray]:
    d, H, G, dh = dims.d_model, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    w_u = (w_std * rng.standard_normal((H * dh, d))).astype(np.float32)
    w_q = (w_std * rng.standard_normal((split, H * dh, d))).astype(np.float32)
    w_kv = (w_std * rng.standard_normal((2 * G * dh, d))).astype(np.float32)
    wo = (wo_std * rng.standard_normal((d, H * dh))).astype(np.float32)
    p1, p2 = gln_params(rng, d), gln_params(rng, H * dh)
    return {"w_u": w_u, "w_q": w_q, "w_kv": w_kv, "w_o": wo, "ln1_g": p1["g"], "ln1_b": p1["b"],
            "ln2_g": p2["g"], "ln2_b": p2["b"]}


def ffn_weights(rng, dims: Dims, split: int, d_ff: int, w_std: float, wo_std: float) -> Dict[str, np.ndarray]:
    """Per-sub-token SwiGLU FFN of one target layer (V2): gate, up [split][d_ff][d], down [split][d][d_ff]."""
    d = dims.d_model
    p = gln_params(rng, d)
    return {"ln_g": p["g"], "ln_b": p["b"],
            "w_gate": (w_std * rng.standard_normal((split, d_ff, d))).astype(np.float32),
            "w_up": (w_std * rng.standard_normal((split, d_ff, d))).astype(np.float32),
            "w_down": (wo_std * rng.standard_normal((split, d, d_ff))).astype(np.float32)}


# --------------------------------------------------------------------------
# The five workloads.

def config0(seed: int = 0) -> Workload:
    """Tiny fp32 full-attention layer: 1 user, 32 H / 16 R / 8 T, d 64, 2Q/1KV, dh 32."""
    rng = np.random.default_rng(seed)
    batch = make_batch(rng, [[32, 16, 8]], 1)
    dims = Dims(64, 2, 1, 32)
    x = (0.02 * rng.standard_normal((batch.total_rows, dims.d_model))).astype(np.float32)
    w = full_weights(rng, dims, 0.02, 0.02)
    return Workload("cfg0_tiny_full_f32", batch, dims, "f32", x, full=[w])


def _cfg1_lens(rng, n_users=32):
    lh = rng.integers(256, 769, size=n_users)
    lr = rng.integers(32, 129, size=n_users)
    lt = rng.integers(16, 65, size=n_users)
    return np.stack([lh, lr, lt], 1).astype(np.int32)


def config1(seed: int = 1, n_users: int = 32) -> Workload:
    """One bf16 full-attention layer over 32 jagged users; d 512, 8Q/2KV, dh 64."""
    rng = np.random.default_rng(seed)
    batch = make_batch(rng, _cfg1_lens(rng, n_users), 1)
    dims = Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    w = full_weights(rng, dims, 0.02, 0.02)
    return Workload("cfg1_full_bf16", batch, dims, "bf16", x, full=[w])


def config2(split: int = 1, seed: int = 2, n_users: int = 32) -> Workload:
    """One bf16 target-attention layer on config 1's batch; split 1 (V1) or 4 (V2 sub-tokens)."""
    rng1 = np.random.default_rng(1)
    b1 = make_batch(rng1, _cfg1_lens(rng1, n_users), 1)
    batch = Batch(b1.lens, split, b1.ts_r, b1.ts_t)
    rng = np.random.default_rng(seed)
    dims = Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    w = target_weights(rng, dims, split, 0.02, 0.02)
    return Workload(f"cfg2_target_s{split}_bf16", batch, dims, "bf16", x, target=[w])


def cfg3_lens(rng, n_users):
    n = rng.integers(1000, 2001, size=n_users)
    lt = np.rint(0.1 * n).astype(np.int64)
    lr = np.rint(0.2 * n).astype(np.int64)
    lh = n - lt - lr
    return np.stack([lh, lr, lt], 1).astype(np.int32)


def config3(seed: int = 3, n_users: int = 160, n_blocks: int = 4, k_target: int = 3,
            weights: bool = True) -> Workload:
    """16-layer hybrid backbone (4 x (1 full + 3 target)), 160 users of 1000..2000 tokens."""
    rng = np.random.default_rng(seed)
    batch = make_batch(rng, cfg3_lens(rng, n_users), 1)
    dims = Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    n_layers = n_blocks * (1 + k_target)
    wo = 0.02 / np.sqrt(n_layers)
    full, tgt = [], []
    if weights:
        for _ in range(n_blocks):
            full.append(full_weights(rng, dims, 0.02, wo))
            for _ in range(k_target):
                tgt.append(target_weights(rng, dims, 1, 0.02, wo))
    return Workload("cfg3_backbone16_bf16", batch, dims, "bf16", x, full=full, target=tgt,
                    n_blocks=n_blocks, k_target=k_target)


def config4(seed: int = 4, n_users: int = 64, lens=(4096, 512, 256), arrays: bool = True) -> Workload:
    """Long-sequence fwd+bwd of one full and one target layer, V2 layout (split 4)."""
    rng = np.random.default_rng(seed)
    batch = make_batch(rng, np.tile(np.asarray(lens, np.int32), (n_users, 1)), 4)
    dims = Dims(1024, 16, 4, 64)
    if not arrays:
        return Workload("cfg4_long_fwd_bwd_bf16", batch, dims, "bf16", np.zeros((0, dims.d_model), np.float32),
                        n_blocks=1, k_target=1)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    full = full_weights(rng, dims, 0.02, 0.02)
    tgt = target_weights(rng, dims, 4, 0.02, 0.02)
    dy = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    return Workload("cfg4_long_fwd_bwd_bf16", batch, dims, "bf16", x, full=[full], target=[tgt],
                    n_blocks=1, k_target=1, dy=dy)


def config3_v2(seed: int = 3, n_users: int = 160, n_blocks: int = 4, k_target: int = 3, d_in: int = 512,
               d_ff: int = 1024):
    """Config 3's users with the V2 target side: each parent a feature vector of width d_in split into
    4 sub-tokens by AutoSplit, a per-sub-token SwiGLU FFN (hidden d_ff) after every target layer.
    Returns (workload with the context rows of X filled, T rows zero; parent features; AutoSplit weight;
    FFN weights per target layer)."""
    rng = np.random.default_rng(seed)
    lens = cfg3_lens(rng, n_users)
    batch = make_batch(rng, lens, 4)
    dims = Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    n_layers = n_blocks * (1 + k_target)
    wo = 0.02 / np.sqrt(n_layers)
    full, tgt, ffn = [], [], []
    for _ in range(n_blocks):
        full.append(full_weights(rng, dims, 0.02, wo))
        for _ in range(k_target):
            tgt.append(target_weights(rng, dims, 4, 0.02, wo))
            ffn.append(ffn_weights(rng, dims, 4, d_ff, 0.02, wo))
    feats = rng.standard_normal((int(lens[:, 2].sum()), d_in))
    w_split = (rng.standard_normal((4 * dims.d_model, d_in)) / np.sqrt(d_in)).astype(np.float32)
    t_rows = np.concatenate([np.arange(batch.row_off[u] + lens[u, 0] + lens[u, 1], batch.row_off[u + 1])
                             for u in range(n_users)])
    x[t_rows] = 0.0
    wl = Workload("cfg3_v2_backbone16_bf16", batch, dims, "bf16", x, full=full, target=tgt, n_blocks=n_blocks,
                  k_target=k_target)
    return wl, feats.astype(np.float32), w_split, ffn


def random_small(rng, n_users: int, split: int, dims: Dims, max_h=12, max_r=8, max_t=5,
                 allow_empty=True) -> Batch:
    """Tiny random users with ties, empty parts and small timestamp ranges (for brute force)."""
    lens = []
    for _ in range(n_users):
        lo = 0 if allow_empty else 1
        lh = int(rng.integers(lo, max_h + 1))
        lr = int(rng.integers(0 if allow_empty else 1, max_r + 1))
        lt = int(rng.integers(0 if allow_empty else 1, max_t + 1))
        if lh + lr + lt == 0:
            lh = 1
        lens.append((lh, lr, lt))
    lens = np.asarray(lens, np.int32)
    # a small timestamp range makes ties between R actions and exposures likely
    hi = int(rng.integers(2, 40))
    ts_r = np.concatenate([np.sort(rng.integers(0, hi, size=l)) for l in lens[:, 1]] or [[]]).astype(np.int32)
    ts_t = np.concatenate([rng.integers(0, hi + 1, size=l) for l in lens[:, 2]] or [[]]).astype(np.int32)
    return Batch(lens, split, ts_r, ts_t)
