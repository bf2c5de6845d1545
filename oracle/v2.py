"""V2 target side ([blog] §3.3.2 "Target Scale-Up"), float64 numpy.

Test infrastructure only (tests, the smoke check and the benchmark's CPU
baseline use it); no product code imports it.

What the page fixes: each target's user, context and item features pass
through one linear map to 4 token embeddings (AutoSplit); in the target
attention layers each of the 4 tokens has its own Q projection and its own
SwiGLU FFN; the 4 tokens are crossed by RankMixer's zero-parameter token
mixing, since otherwise they would not interact before the mean pooling that
ends the target side.  The page gives no formulas; the readings used here
(each also in the design notes):

  * AutoSplit: bias-free linear map of a parent's feature vector (width d_in)
    to split * d_model values; sub-token z takes columns [z d, (z + 1) d).
  * Per-sub-token SwiGLU FFN after every target layer, on the T rows only,
    pre-normalised and residual like the layers:
        X_T <- X_T + W_down[z] (SiLU(W_gate[z] X~) (.) (W_up[z] X~)),
        X~ = LayerNorm(X_T) with the FFN's own gamma, beta (T-row parameters),
    bias-free, hidden width d_ff.
  * Token mixing right after that FFN (RankMixer's mixing as published: cut
    each of the S tokens of a parent into S equal chunks; output token c is
    the concatenation over z of chunk c of input token z), S = 1 the identity.
  * Mean pooling after the last layer: one vector per parent, the mean of its
    S sub-token rows.
  * The full (self-attention) layers stay as in the V1 stack; only the target
    side gets the FFN and the mixing.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import mask as _mask
from .model import full_layer_user, gln, silu, target_layer_user, user_mask


def autosplit(feats, w_split, split):
    """[P][d_in] parent features -> [P * split][d] T rows (sub-token z of parent m at m * split + z)."""
    f = np.asarray(feats, np.float64)
    w = np.asarray(w_split, np.float64)
    out = f @ w.T                                   # [P][split * d]
    d = w.shape[0] // split
    return out.reshape(f.shape[0] * split, d)


def token_mix(xt, split):
    """RankMixer token mixing over each parent's S sub-tokens (rows in T-row order)."""
    x = np.asarray(xt, np.float64)
    n, d = x.shape
    if split == 1:
        return x.copy()
    assert d % split == 0 and n % split == 0
    p = n // split
    grid = x.reshape(p, split, split, d // split)   # [parent][token z][chunk c][width]
    return grid.transpose(0, 2, 1, 3).reshape(n, d)  # token c holds chunk c of every token z, z in order


def token_ffn(xt, w: Dict[str, np.ndarray], split, eps):
    """Per-sub-token SwiGLU FFN with pre-norm and residual on T rows (T-row order)."""
    x = np.asarray(xt, np.float64)
    types = np.full(x.shape[0], _mask.T_TYPE)
    xn = gln(x, w["ln_g"], w["ln_b"], types, eps)
    out = x.copy()
    for z in range(split):
        rows = slice(z, None, split)
        g = xn[rows] @ np.asarray(w["w_gate"][z], np.float64).T
        u = xn[rows] @ np.asarray(w["w_up"][z], np.float64).T
        out[rows] += (silu(g) * u) @ np.asarray(w["w_down"][z], np.float64).T
    return out


def mean_pool(xt, split):
    """[P * split][d] -> [P][d]: mean over each parent's sub-tokens."""
    x = np.asarray(xt, np.float64)
    return x.reshape(x.shape[0] // split, split, x.shape[1]).mean(axis=1)


def _t_rows_of_user(l_h, l_r, l_t, split):
    return np.arange(l_h + l_r, l_h + l_r + split * l_t)


def backbone_v2_user(x, m, types, l_ctx, split, full_ws: List[Dict], tgt_ws: List[Dict], ffn_ws: List[Dict], dims,
                     n_blocks, k_target, boundary=None):
    """The hybrid stack with the V2 target side: after every target layer, the T rows get the
    per-sub-token FFN and the token mixing."""
    b = boundary or (lambda a: a)
    x = b(np.asarray(x, np.float64))
    t = np.arange(l_ctx, x.shape[0])
    for blk in range(n_blocks):
        x = b(full_layer_user(x, m, types, full_ws[blk], dims))
        for k in range(k_target):
            i = blk * k_target + k
            x = b(target_layer_user(x, m, types, l_ctx, split, tgt_ws[i], dims))
            if len(t):
                x = x.copy()
                x[t] = b(token_mix(token_ffn(x[t], ffn_ws[i], split, dims.ln_eps), split))
    return x


def backbone_v2(batch, x, full_ws, tgt_ws, ffn_ws, dims, n_blocks, k_target, boundary=None, users=None):
    """V2 stack over a batch (or the listed users, in that order); rows as in the input."""
    users = list(range(batch.n_users)) if users is None else list(users)
    outs = []
    off = batch.row_off
    for u in users:
        l_h, l_r, l_t = (int(v) for v in batch.lens[u])
        mm = user_mask(batch, u)
        types = _mask.row_types(l_h, l_r, l_t, batch.split)
        outs.append(backbone_v2_user(x[off[u]:off[u + 1]], mm, types, l_h + l_r, batch.split, full_ws, tgt_ws,
                                     ffn_ws, dims, n_blocks, k_target, boundary))
    return np.concatenate(outs) if outs else np.zeros((0, x.shape[1]))


def t_rows(batch, users: Optional[List[int]] = None):
    """Packed rows of the T rows of the listed users (all by default), T-row order."""
    users = list(range(batch.n_users)) if users is None else list(users)
    off = batch.row_off
    r = [off[u] + _t_rows_of_user(*(int(v) for v in batch.lens[u]), batch.split) for u in users]
    return np.concatenate(r) if r else np.zeros(0, np.int64)
