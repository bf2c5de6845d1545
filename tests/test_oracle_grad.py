"""Pins of the oracle's hand-derived backward: central finite differences (fp64).

For L(theta) = sum(layer(theta) * dY) and random directions delta,
(L(theta + eps delta) - L(theta - eps delta)) / (2 eps) must equal
<grad, delta>.  Random directions touch every element, so a dropped term, a
wrong sign or a transposed operand anywhere in the backward shows up.
"""
import numpy as np
import pytest

import synth
from oracle import grad as og
from oracle import model as om_model


def _setup(rng, split, lens):
    dims = synth.Dims(12, 4, 2, 3, ln_eps=1e-3)
    b = synth.make_batch(rng, np.asarray(lens, np.int32), split)
    x = rng.standard_normal((b.total_rows, dims.d_model))
    wf = {k: v.astype(np.float64) for k, v in synth.full_weights(rng, dims, 0.4, 0.4).items()}
    wt = {k: v.astype(np.float64) for k, v in synth.target_weights(rng, dims, split, 0.4, 0.4).items()}
    dy = rng.standard_normal(x.shape)
    return b, dims, x, wf, wt, dy


def _check(loss, grads, params, rng, n_dirs=3, eps=1e-6, rtol=1e-6):
    for name, val in params.items():
        for _ in range(n_dirs):
            d = rng.standard_normal(val.shape)
            plus, minus = dict(params), dict(params)
            plus[name] = val + eps * d
            minus[name] = val - eps * d
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= rtol * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("split", [1, 4])
def test_full_layer_backward_finite_differences(split):
    rng = np.random.default_rng(20 + split)
    b, dims, x, wf, _, dy = _setup(rng, split, [[4, 3, 2], [2, 4, 1], [3, 0, 2]])
    grads = og.full_layer_bwd(b, x, wf, dims, dy)

    def loss(p):
        w = {k: p.get(k, wf[k]) for k in wf}
        return float(np.sum(om_model.full_layer(b, p["x"], w, dims) * dy))

    params = {"x": x, **wf}
    _check(loss, grads, params, rng)


@pytest.mark.parametrize("split", [1, 4])
def test_target_layer_backward_finite_differences(split):
    rng = np.random.default_rng(30 + split)
    b, dims, x, _, wt, dy = _setup(rng, split, [[4, 3, 2], [2, 4, 1], [3, 2, 0]])
    grads = og.target_layer_bwd(b, x, wt, dims, dy)

    def loss(p):
        w = {k: p.get(k, wt[k]) for k in wt}
        return float(np.sum(om_model.target_layer(b, p["x"], w, dims) * dy))

    params = {"x": x, **wt}
    _check(loss, grads, params, rng)


def test_target_backward_context_rows_get_residual_plus_kv_path():
    # zero U weights make the gate U = 0: the branch output is 0 whatever A is,
    # so no gradient reaches Q, K, V or X~ (dX = dY exactly) and dW_o = 0.
    rng = np.random.default_rng(41)
    b, dims, x, _, wt, dy = _setup(rng, 1, [[4, 3, 2]])
    w = dict(wt); w["w_u"] = np.zeros_like(wt["w_u"])
    g = og.target_layer_bwd(b, x, w, dims, dy)
    np.testing.assert_allclose(g["x"], dy, rtol=0, atol=1e-15)
    assert np.all(g["w_o"] == 0)


@pytest.mark.parametrize("split", [1, 4])
def test_backbone_backward_finite_differences(split):
    """2 blocks x (1 full + 2 target): dX and the weights of the first and last layers."""
    rng = np.random.default_rng(50 + split)
    lens = [[4, 3, 2], [2, 4, 1], [3, 0, 2]]
    dims = synth.Dims(12, 4, 2, 3, ln_eps=1e-3)
    b = synth.make_batch(rng, np.asarray(lens, np.int32), split)
    x = rng.standard_normal((b.total_rows, dims.d_model))
    n_blocks, k = 2, 2
    full = [{kk: v.astype(np.float64) for kk, v in synth.full_weights(rng, dims, 0.4, 0.4).items()}
            for _ in range(n_blocks)]
    tgt = [{kk: v.astype(np.float64) for kk, v in synth.target_weights(rng, dims, split, 0.4, 0.4).items()}
           for _ in range(n_blocks * k)]
    dy = rng.standard_normal(x.shape)
    g = og.backbone_bwd(b, x, full, tgt, dims, n_blocks, k, dy)
    assert len(g["full"]) == n_blocks and len(g["target"]) == n_blocks * k

    def loss(p):
        f = [dict(w) for w in full]
        t = [dict(w) for w in tgt]
        for kk in full[0]:
            if "f0_" + kk in p:
                f[0][kk] = p["f0_" + kk]
        for kk in tgt[-1]:
            if "tl_" + kk in p:
                t[-1][kk] = p["tl_" + kk]
        out = om_model.backbone(b, p["x"], f, t, dims, n_blocks, k)
        return float(np.sum(out * dy))

    params = {"x": x, **{"f0_" + kk: v for kk, v in full[0].items()}, **{"tl_" + kk: v for kk, v in tgt[-1].items()}}
    grads = {"x": g["x"], **{"f0_" + kk: v for kk, v in g["full"][0].items()},
             **{"tl_" + kk: v for kk, v in g["target"][-1].items()}}
    _check(loss, grads, params, rng, n_dirs=2)


def test_backbone_backward_of_one_layer_is_the_layer_backward():
    """n_blocks = 1, k_target = 0 reduces to the full layer's backward exactly."""
    rng = np.random.default_rng(61)
    b, dims, x, wf, _, dy = _setup(rng, 1, [[4, 3, 2], [2, 0, 1]])
    g = og.backbone_bwd(b, x, [wf], [], dims, 1, 0, dy)
    ref = og.full_layer_bwd(b, x, wf, dims, dy)
    np.testing.assert_array_equal(g["x"], ref["x"])
    for kk in wf:
        np.testing.assert_array_equal(g["full"][0][kk], ref[kk])
