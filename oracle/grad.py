"""Backward of the full- and target-attention layers, derived by hand, float64.

For a layer X' = layer(X) and an upstream gradient dY, these return the
gradients of L = sum(X' * dY) with respect to X, every weight and the GLN
parameters.  The forward equations are those of oracle.model ([explainer] §4.1,
§4.2).  Derivative facts used:

  SiLU'(x)        = s (1 + x (1 - s)),  s = sigmoid(x)
  LayerNorm'      : xhat = (x - mu) / sqrt(var + eps) over a row of width D;
                    dx = (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)) / sqrt(var + eps)
  y = x W^T       : dx = dy W,  dW = dy^T x
  A_h = (P_h V_g) / n, P_h = SiLU(S_h) (.) M, S_h = Q_h K_g^T / sqrt(dh):
                    dV_g += P_h^T (dA_h / n),  dP_h = (dA_h / n) V_g^T,
                    dS_h = dP_h (.) M (.) SiLU'(S_h),
                    dQ_h = dS_h K_g / sqrt(dh),  dK_g += dS_h^T Q_h / sqrt(dh)

Pinned by central finite differences in the not-gpu tests.
"""
from __future__ import annotations

import numpy as np

from . import mask as _mask
from .model import silu, dense_mask_fast


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def dsilu(x):
    s = _sig(x)
    return s * (1.0 + x * (1.0 - s))


def _ln_fwd(x, eps):
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    return (x - mu) * rstd, rstd


def _ln_bwd(dxhat, xhat, rstd):
    return (dxhat - dxhat.mean(axis=1, keepdims=True)
            - xhat * (dxhat * xhat).mean(axis=1, keepdims=True)) * rstd


def _gln_param_grads(dout, xhat, types, n_types=3):
    dg = np.zeros((n_types, xhat.shape[1]))
    db = np.zeros((n_types, xhat.shape[1]))
    for t in range(n_types):
        sel = types == t
        dg[t] = (dout[sel] * xhat[sel]).sum(axis=0)
        db[t] = dout[sel].sum(axis=0)
    return dg, db


def _attn_fwd(q, k, v, m, H, G, dh):
    r = H // G
    n = m.sum(axis=1).astype(np.float64)[:, None]
    a = np.zeros((q.shape[0], H * dh))
    cache = []
    for h in range(H):
        g = h // r
        qh, kg, vg = q[:, h * dh:(h + 1) * dh], k[:, g * dh:(g + 1) * dh], v[:, g * dh:(g + 1) * dh]
        s = (qh @ kg.T) / np.sqrt(dh)
        p = silu(s) * m
        a[:, h * dh:(h + 1) * dh] = (p @ vg) / n
        cache.append((s, p))
    return a, (n, cache)


def _attn_bwd(da, q, k, v, m, H, G, dh, saved):
    n, cache = saved
    r = H // G
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    for h in range(H):
        g = h // r
        s, p = cache[h]
        qh, kg, vg = q[:, h * dh:(h + 1) * dh], k[:, g * dh:(g + 1) * dh], v[:, g * dh:(g + 1) * dh]
        dan = da[:, h * dh:(h + 1) * dh] / n
        dv[:, g * dh:(g + 1) * dh] += p.T @ dan
        dp = dan @ vg.T
        ds = dp * m * dsilu(s)
        dq[:, h * dh:(h + 1) * dh] = ds @ kg / np.sqrt(dh)
        dk[:, g * dh:(g + 1) * dh] += ds.T @ qh / np.sqrt(dh)
    return dq, dk, dv


def full_layer_user_bwd(x, m, types, w, dims, dy):
    """Gradients of sum(full_layer(x) * dy) for one user."""
    H, G, dh, eps = dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ln_eps
    hd, gd = H * dh, G * dh
    x = np.asarray(x, np.float64); dy = np.asarray(dy, np.float64)
    w1 = np.asarray(w["w_uqkv"], np.float64); wo = np.asarray(w["w_o"], np.float64)
    g1, b1 = np.asarray(w["ln1_g"], np.float64), np.asarray(w["ln1_b"], np.float64)
    g2, b2 = np.asarray(w["ln2_g"], np.float64), np.asarray(w["ln2_b"], np.float64)
    # forward, keeping what the backward needs
    xhat, rstd1 = _ln_fwd(x, eps)
    xt = xhat * g1[types] + b1[types]
    hpre = xt @ w1.T
    z = silu(hpre)
    u, q, k, v = z[:, :hd], z[:, hd:2 * hd], z[:, 2 * hd:2 * hd + gd], z[:, 2 * hd + gd:]
    a, saved = _attn_fwd(q, k, v, m, H, G, dh)
    ahat, rstd2 = _ln_fwd(a, eps)
    yt = ahat * g2[types] + b2[types]
    y = yt * u
    # backward
    dwo = dy.T @ y
    dyv = dy @ wo
    du = dyv * yt
    dyt = dyv * u
    dg2, db2 = _gln_param_grads(dyt, ahat, types)
    da = _ln_bwd(dyt * g2[types], ahat, rstd2)
    dq, dk, dv = _attn_bwd(da, q, k, v, m, H, G, dh, saved)
    dz = np.concatenate([du, dq, dk, dv], axis=1)
    dh_ = dz * dsilu(hpre)
    dw1 = dh_.T @ xt
    dxt = dh_ @ w1
    dg1, db1 = _gln_param_grads(dxt, xhat, types)
    dx = dy + _ln_bwd(dxt * g1[types], xhat, rstd1)
    return {"x": dx, "w_uqkv": dw1, "w_o": dwo, "ln1_g": dg1, "ln1_b": db1, "ln2_g": dg2, "ln2_b": db2}


def target_layer_user_bwd(x, m, types, l_ctx, split, w, dims, dy):
    """Gradients of sum(target_layer(x) * dy) for one user."""
    H, G, dh, eps = dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ln_eps
    hd, gd = H * dh, G * dh
    x = np.asarray(x, np.float64); dy = np.asarray(dy, np.float64)
    wu = np.asarray(w["w_u"], np.float64); wq = np.asarray(w["w_q"], np.float64)
    wkv = np.asarray(w["w_kv"], np.float64); wo = np.asarray(w["w_o"], np.float64)
    g1, b1 = np.asarray(w["ln1_g"], np.float64), np.asarray(w["ln1_b"], np.float64)
    g2, b2 = np.asarray(w["ln2_g"], np.float64), np.asarray(w["ln2_b"], np.float64)
    tt = types[l_ctx:]
    xhat, rstd1 = _ln_fwd(x, eps)
    xt = xhat * g1[types] + b1[types]
    kv_pre = xt @ wkv.T
    kv = silu(kv_pre)
    k, v = kv[:, :gd], kv[:, gd:]
    xt_t = xt[l_ctx:]
    nt = xt_t.shape[0]
    sub = np.arange(nt) % split
    u_pre = xt_t @ wu.T
    q_pre = np.stack([xt_t[i] @ wq[sub[i]].T for i in range(nt)]) if nt else np.zeros((0, hd))
    u_t, q_t = silu(u_pre), silu(q_pre)
    m_t = m[l_ctx:]
    a, saved = _attn_fwd(q_t, k, v, m_t, H, G, dh)
    ahat, rstd2 = _ln_fwd(a, eps) if nt else (a, np.zeros((0, 1)))
    yt = ahat * g2[tt] + b2[tt]
    y = yt * u_t
    dy_t = dy[l_ctx:]
    dwo = dy_t.T @ y
    dyv = dy_t @ wo
    du = dyv * yt
    dyt = dyv * u_t
    dg2, db2 = _gln_param_grads(dyt, ahat, tt)
    da = _ln_bwd(dyt * g2[tt], ahat, rstd2) if nt else da_empty(hd)
    dq, dk, dv = _attn_bwd(da, q_t, k, v, m_t, H, G, dh, saved)
    du_pre = du * dsilu(u_pre)
    dq_pre = dq * dsilu(q_pre)
    dkv_pre = np.concatenate([dk, dv], axis=1) * dsilu(kv_pre)
    dwu = du_pre.T @ xt_t
    dwq = np.zeros_like(wq)
    for s in range(split):
        sel = sub == s
        dwq[s] = dq_pre[sel].T @ xt_t[sel]
    dwkv = dkv_pre.T @ xt
    dxt = dkv_pre @ wkv
    dxt[l_ctx:] += du_pre @ wu
    for i in range(nt):
        dxt[l_ctx + i] += dq_pre[i] @ wq[sub[i]]
    dg1, db1 = _gln_param_grads(dxt, xhat, types)
    dx = dy.copy()
    dx += _ln_bwd(dxt * g1[types], xhat, rstd1)
    return {"x": dx, "w_u": dwu, "w_q": dwq, "w_kv": dwkv, "w_o": dwo,
            "ln1_g": dg1, "ln1_b": db1, "ln2_g": dg2, "ln2_b": db2}


def da_empty(width):
    return np.zeros((0, width))


def _batch_bwd(batch, x, dy, fn):
    grads = None
    off = batch.row_off
    ro, to = batch.r_off, batch.t_off
    dx = np.zeros(x.shape, np.float64)
    for u in range(batch.n_users):
        l_h, l_r, l_t = (int(v) for v in batch.lens[u])
        m = dense_mask_fast(l_h, l_r, l_t, batch.split, batch.ts_r[ro[u]:ro[u + 1]], batch.ts_t[to[u]:to[u + 1]])
        types = _mask.row_types(l_h, l_r, l_t, batch.split)
        g = fn(x[off[u]:off[u + 1]], m, types, l_h + l_r, dy[off[u]:off[u + 1]])
        dx[off[u]:off[u + 1]] = g.pop("x")
        if grads is None:
            grads = g
        else:
            for kk in grads:
                grads[kk] = grads[kk] + g[kk]
    grads["x"] = dx
    return grads


def full_layer_bwd(batch, x, w, dims, dy):
    """Batch gradients of sum(full_layer(x) * dy); weight gradients summed over users."""
    return _batch_bwd(batch, x, dy, lambda xu, m, t, lc, dyu: full_layer_user_bwd(xu, m, t, w, dims, dyu))


def target_layer_bwd(batch, x, w, dims, dy):
    """Batch gradients of sum(target_layer(x) * dy); weight gradients summed over users."""
    return _batch_bwd(batch, x, dy,
                      lambda xu, m, t, lc, dyu: target_layer_user_bwd(xu, m, t, lc, batch.split, w, dims, dyu))


def backbone_bwd(batch, x, full_ws, tgt_ws, dims, n_blocks, k_target, dy, boundary=None):
    """Gradients of sum(backbone(x) * dy) through the whole hybrid stack.

    The stack is n_blocks x (1 full layer + k_target target layers) ([explainer]
    §4: B blocks of 1 full + K target layers; [blog] §3.3.1).  One forward pass
    keeps every layer's input; then the layers' backward run in reverse order,
    the upstream gradient of layer l being the input gradient of layer l + 1
    (chain rule through the stack).  ``boundary`` (e.g. bf16 rounding) is
    applied to the activations between layers, as in oracle.model.backbone, and
    to the gradients handed from one layer to the next, mirroring a run that
    stores both in reduced precision.  Returns {"x": dL/dX, "full": [grads of
    each full layer], "target": [grads of each target layer]} in the layers'
    order.
    """
    from .model import full_layer, target_layer
    b = boundary or (lambda a: a)
    layers = []
    for blk in range(n_blocks):
        layers.append(("full", full_ws[blk]))
        for t in range(k_target):
            layers.append(("target", tgt_ws[blk * k_target + t]))
    inputs = []
    cur = b(np.asarray(x, np.float64))
    for l, (kind, w) in enumerate(layers):
        inputs.append(cur)
        if l + 1 < len(layers):
            cur = b(full_layer(batch, cur, w, dims) if kind == "full" else target_layer(batch, cur, w, dims))
    g = np.asarray(dy, np.float64)
    out_full, out_tgt = [], []
    for l in reversed(range(len(layers))):
        kind, w = layers[l]
        fn = full_layer_bwd if kind == "full" else target_layer_bwd
        r = fn(batch, inputs[l], w, dims, g)
        g = r.pop("x")
        if l > 0:
            g = b(g)
        (out_full if kind == "full" else out_tgt).insert(0, r)
    return {"x": g, "full": out_full, "target": out_tgt}
