"""Forward pass of the hybrid HSTU-style backbone, in float64 numpy.

Layer equations ([explainer] §4.1 and §4.2):

  full layer:    U, Q_h, K_g, V_g = Split(phi1(f1(X~)))
                 A_h = phi2(Q_h K_g^T (.) M) V_g,   g = h // r,  r = H / G
                 X'  = f2(GLN(A) (.) U) + X
  target layer:  U_T, Q_T,h = Split(phi1(f_uq(X~_T)));  K_g, V_g = Split(phi1(f_kv(X~)))
                 A_T,h = phi2(Q_T,h K_g^T (.) M_T) V_g
                 X'_T = f2(GLN(A_T) (.) U_T) + X_T;   X'_{H,R} = X_{H,R}

Readings where the pages leave a step open (each also listed in the design
notes):
  * phi1 = SiLU on all of U, Q, K, V (HSTU layer; the backbone is HSTU per
    [digest], and [blog] §6.1 names SiLU fusion in the attention kernel).
  * phi2(s) = SiLU(s / sqrt(head_dim)) applied elementwise, masked entries zero
    (SiLU(0) = 0, so masking before or after phi2 is the same), and each row is
    divided by n_i = number of keys that row sees.
  * GLN = LayerNorm over the whole row (d_model before f1/f_kv/f_uq, H*dh after
    attention) with biased variance, eps passed in, and affine parameters
    gamma[type], beta[type] picked by the row's token type H/R/T ([blog] §6.1:
    one [G, D] parameter matrix indexed per token by its group id).
  * f1, f2, f_uq, f_kv are bias-free linear maps, y = x W^T.
  * Split order [U | Q | K | V], heads contiguous; query head h uses KV group
    h // r ([explainer] §4.1 GQA).
  * V2 sub-tokens ([blog] §3.3.2): target rows are target-major, sub-token k
    uses its own Q projection W_q[k]; U, K, V projections are shared.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional

import numpy as np

from . import mask as _mask
from .mask import dense_mask_fast  # noqa: F401  (re-exported)


def silu(x):
    return x / (1.0 + np.exp(-x))


def gln(x, gamma, beta, types, eps):
    """Group LayerNorm: row-wise LayerNorm, affine parameters chosen by row type."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    xhat = (x - mu) / np.sqrt(var + eps)
    g = np.asarray(gamma, np.float64)[types]
    b = np.asarray(beta, np.float64)[types]
    return xhat * g + b


def masked_attention(q, k, v, m, n_q_heads, n_kv_heads, head_dim):
    """A = concat_h (SiLU(Q_h K_g^T / sqrt(dh)) (.) M) V_g / n   (one user).

    q: [Nq, H*dh], k, v: [Nk, G*dh], m: [Nq, Nk] 0/1.  Every row must see at
    least one key (true under the mask rules: H rows see H, R rows see
    themselves, T rows see themselves).
    """
    r = n_q_heads // n_kv_heads
    n = m.sum(axis=1).astype(np.float64)[:, None]
    out = np.zeros((q.shape[0], n_q_heads * head_dim))
    for h in range(n_q_heads):
        g = h // r
        qh = q[:, h * head_dim:(h + 1) * head_dim]
        kg = k[:, g * head_dim:(g + 1) * head_dim]
        vg = v[:, g * head_dim:(g + 1) * head_dim]
        s = (qh @ kg.T) / np.sqrt(head_dim)
        p = silu(s) * m
        out[:, h * head_dim:(h + 1) * head_dim] = (p @ vg) / n
    return out


def _split_uqkv(z, dims):
    hd, gd = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    return z[:, :hd], z[:, hd:2 * hd], z[:, 2 * hd:2 * hd + gd], z[:, 2 * hd + gd:2 * hd + 2 * gd]


def full_layer_user(x, m, types, w: Dict[str, np.ndarray], dims, return_parts=False):
    """One user's full-attention layer ([explainer] §4.1)."""
    x = np.asarray(x, np.float64)
    xt = gln(x, w["ln1_g"], w["ln1_b"], types, dims.ln_eps)
    z = silu(xt @ np.asarray(w["w_uqkv"], np.float64).T)
    u, q, k, v = _split_uqkv(z, dims)
    a = masked_attention(q, k, v, m, dims.n_q_heads, dims.n_kv_heads, dims.head_dim)
    y = gln(a, w["ln2_g"], w["ln2_b"], types, dims.ln_eps) * u
    out = y @ np.asarray(w["w_o"], np.float64).T + x
    if return_parts:
        return out, {"a": a, "y": y, "u": u, "q": q, "k": k, "v": v}
    return out


def full_layer_rows(x, l_h, l_r, l_t, split, ts_r, ts_t, w: Dict[str, np.ndarray], dims, rows):
    """Selected rows of one user's full-attention layer ([explainer] §4.1).

    The equations of `full_layer_user` for the query rows `rows` only, each
    row's mask from `mask.mask_row`: for users too long for an N x N mask.
    K and V are projected for every row of the user (any of them may be a
    key); U and Q for the selected rows.
    """
    x = np.asarray(x, np.float64)
    rows = np.asarray(rows, np.int64)
    hd, gd = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    types = _mask.row_types(l_h, l_r, l_t, split)
    xt = gln(x, w["ln1_g"], w["ln1_b"], types, dims.ln_eps)
    w1 = np.asarray(w["w_uqkv"], np.float64)
    kv = silu(xt @ w1[2 * hd:2 * hd + 2 * gd].T)
    k, v = kv[:, :gd], kv[:, gd:]
    uq = silu(xt[rows] @ w1[:2 * hd].T)
    u, q = uq[:, :hd], uq[:, hd:]
    m = np.stack([_mask.mask_row(int(i), l_h, l_r, l_t, split, ts_r, ts_t) for i in rows])
    a = masked_attention(q, k, v, m, dims.n_q_heads, dims.n_kv_heads, dims.head_dim)
    y = gln(a, w["ln2_g"], w["ln2_b"], types[rows], dims.ln_eps) * u
    return y @ np.asarray(w["w_o"], np.float64).T + x[rows]


def target_layer_user(x, m, types, l_ctx, split, w: Dict[str, np.ndarray], dims, return_parts=False):
    """One user's target-attention layer ([explainer] §4.2; V2 per-sub-token Q, [blog] §3.3.2)."""
    x = np.asarray(x, np.float64)
    hd = dims.n_q_heads * dims.head_dim
    gd = dims.n_kv_heads * dims.head_dim
    xt = gln(x, w["ln1_g"], w["ln1_b"], types, dims.ln_eps)
    kv = silu(xt @ np.asarray(w["w_kv"], np.float64).T)
    k, v = kv[:, :gd], kv[:, gd:2 * gd]
    xt_t = xt[l_ctx:]
    nt = xt_t.shape[0]
    u_t = silu(xt_t @ np.asarray(w["w_u"], np.float64).T)
    q_t = np.zeros((nt, hd))
    wq = np.asarray(w["w_q"], np.float64)
    for i in range(nt):
        q_t[i] = silu(xt_t[i] @ wq[i % split].T)
    m_t = m[l_ctx:]
    a_t = masked_attention(q_t, k, v, m_t, dims.n_q_heads, dims.n_kv_heads, dims.head_dim)
    y_t = gln(a_t, w["ln2_g"], w["ln2_b"], types[l_ctx:], dims.ln_eps) * u_t
    out = x.copy()
    out[l_ctx:] = y_t @ np.asarray(w["w_o"], np.float64).T + x[l_ctx:]
    if return_parts:
        return out, {"a": a_t, "y": y_t, "u": u_t, "q": q_t, "k": k, "v": v}
    return out


def _user_views(batch):
    ro, to, off = batch.r_off, batch.t_off, batch.row_off
    for u in range(batch.n_users):
        l_h, l_r, l_t = (int(v) for v in batch.lens[u])
        yield u, l_h, l_r, l_t, batch.ts_r[ro[u]:ro[u + 1]], batch.ts_t[to[u]:to[u + 1]], int(off[u]), int(off[u + 1])


def user_mask(batch, u):
    l_h, l_r, l_t = (int(v) for v in batch.lens[u])
    ro, to = batch.r_off, batch.t_off
    return dense_mask_fast(l_h, l_r, l_t, batch.split, batch.ts_r[ro[u]:ro[u + 1]], batch.ts_t[to[u]:to[u + 1]])


def full_layer(batch, x, w, dims, return_parts=False):
    """Full-attention layer over a jagged batch, one user at a time."""
    out = np.zeros(x.shape, np.float64)
    parts = {"a": [], "y": []}
    for u, l_h, l_r, l_t, ts_r, ts_t, r0, r1 in _user_views(batch):
        m = dense_mask_fast(l_h, l_r, l_t, batch.split, ts_r, ts_t)
        types = _mask.row_types(l_h, l_r, l_t, batch.split)
        res = full_layer_user(x[r0:r1], m, types, w, dims, return_parts)
        if return_parts:
            out[r0:r1] = res[0]
            parts["a"].append(res[1]["a"]); parts["y"].append(res[1]["y"])
        else:
            out[r0:r1] = res
    if return_parts:
        return out, {k: np.concatenate(v) if v else np.zeros((0, dims.n_q_heads * dims.head_dim)) for k, v in parts.items()}
    return out


def target_layer(batch, x, w, dims, return_parts=False):
    """Target-attention layer over a jagged batch; A and Y parts cover T rows only."""
    out = np.zeros(x.shape, np.float64)
    parts = {"a": [], "y": []}
    for u, l_h, l_r, l_t, ts_r, ts_t, r0, r1 in _user_views(batch):
        m = dense_mask_fast(l_h, l_r, l_t, batch.split, ts_r, ts_t)
        types = _mask.row_types(l_h, l_r, l_t, batch.split)
        res = target_layer_user(x[r0:r1], m, types, l_h + l_r, batch.split, w, dims, return_parts)
        if return_parts:
            out[r0:r1] = res[0]
            parts["a"].append(res[1]["a"]); parts["y"].append(res[1]["y"])
        else:
            out[r0:r1] = res
    if return_parts:
        return out, {k: np.concatenate(v) if v else np.zeros((0, dims.n_q_heads * dims.head_dim)) for k, v in parts.items()}
    return out


def backbone_user(x, m, types, l_ctx, split, full_ws: List[Dict], tgt_ws: List[Dict], dims,
                  n_blocks: int, k_target: int, boundary: Optional[Callable] = None):
    """Hybrid stack: n_blocks x (1 full layer + k_target target layers).

    [explainer] §4 (B blocks of 1 full + K target layers); [blog] §3.3.1
    (16 layers = 4 blocks of 1 full + 3 target).  The mask is built once and
    shared by every layer.  ``boundary`` (e.g. bf16 rounding) is applied to X
    after every layer when mirroring a reduced-precision run.
    """
    b = boundary or (lambda a: a)
    x = b(np.asarray(x, np.float64))
    for blk in range(n_blocks):
        x = b(full_layer_user(x, m, types, full_ws[blk], dims))
        for t in range(k_target):
            x = b(target_layer_user(x, m, types, l_ctx, split, tgt_ws[blk * k_target + t], dims))
    return x


def backbone(batch, x, full_ws, tgt_ws, dims, n_blocks, k_target, boundary=None, users=None):
    """Backbone over a batch (or over the listed users only, returned in that order)."""
    users = list(range(batch.n_users)) if users is None else list(users)
    outs = []
    off = batch.row_off
    for u in users:
        l_h, l_r, l_t = (int(v) for v in batch.lens[u])
        m = user_mask(batch, u)
        types = _mask.row_types(l_h, l_r, l_t, batch.split)
        outs.append(backbone_user(x[off[u]:off[u + 1]], m, types, l_h + l_r, batch.split,
                                  full_ws, tgt_ws, dims, n_blocks, k_target, boundary))
    return np.concatenate(outs) if outs else np.zeros((0, x.shape[1]))


def bf16_round(a):
    """Round to the nearest bfloat16 (ties to even) and back, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()
