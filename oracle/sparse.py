"""2:4 structured pruning of projection weights ([explainer] §5.2.1), float64 numpy.

Test infrastructure only (tests, the smoke check and the benchmark's CPU
baseline use it); no product code imports it.

What the page fixes: in the linear projections that produce U, V, Q, K and
the output, of every 4 consecutive weight parameters the 2 smaller ones are
set to zero, for inference on sparse matrix hardware.  Readings used here
(each also in the design notes):

  * "consecutive" runs along a weight row, i.e. along the input (reduction)
    dimension of y = x W^T, in groups 4g .. 4g + 3 -- the axis the sparse
    matrix instructions compress;
  * "smaller" compares magnitudes; of equal magnitudes the one at the lower
    position is kept (any fixed rule would do; this one is stated so that
    the result is unique);
  * a pruned layer is the same layer computed with the pruned weights: the
    sparse kernels must reproduce the dense layer on those weights.
"""
from __future__ import annotations

import numpy as np


def prune_24(w):
    """Zero the 2 smaller-magnitude entries of every group of 4 consecutive entries along the last axis.

    The last axis must be a multiple of 4.  Returns a float64 copy."""
    a = np.array(w, dtype=np.float64, copy=True)
    k = a.shape[-1]
    assert k % 4 == 0, "the last axis must be a multiple of 4"
    g = a.reshape(-1, k // 4, 4)
    mag = np.abs(g)
    out = np.zeros_like(g)
    for r in range(g.shape[0]):
        for q in range(g.shape[1]):
            # rank by magnitude, larger first; of equal magnitudes the lower position first
            order = sorted(range(4), key=lambda p: (-mag[r, q, p], p))
            for p in order[:2]:
                out[r, q, p] = g[r, q, p]
    return out.reshape(a.shape)


def keep_mask_24(w):
    """Boolean mask of the entries prune_24 keeps (exactly 2 per group of 4)."""
    a = np.asarray(w, dtype=np.float64)
    k = a.shape[-1]
    g = np.abs(a.reshape(-1, k // 4, 4))
    keep = np.zeros(g.shape, dtype=bool)
    for r in range(g.shape[0]):
        for q in range(g.shape[1]):
            order = sorted(range(4), key=lambda p: (-g[r, q, p], p))
            keep[r, q, order[0]] = keep[r, q, order[1]] = True
    return keep.reshape(a.shape)


def prune_full_weights(w):
    """A full layer's weights with its projections pruned (U, Q, K, V and the output); GLN parameters kept."""
    out = dict(w)
    for k in ("w_uqkv", "w_o"):
        out[k] = prune_24(w[k])
    return out


def prune_target_weights(w):
    """A target layer's weights with its projections pruned (U, Q[k], K|V and the output)."""
    out = dict(w)
    for k in ("w_u", "w_q", "w_kv", "w_o"):
        out[k] = prune_24(w[k])
    return out
