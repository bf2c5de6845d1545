"""Pins of the V2 target-side oracle (oracle/v2.py) against definitions fixed
independently of its code: a hand-worked mixing example, involution and
permutation properties, library routines for the linear maps and SiLU, closed
forms when weights vanish, and the reduction of the V2 stack to the V1 stack."""
import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from oracle import v2


def test_token_mix_worked_example():
    # S = 2, d = 4: tokens [a0 a1 | a2 a3], [b0 b1 | b2 b3] -> [a0 a1 b0 b1], [a2 a3 b2 b3]
    x = np.array([[1., 2., 3., 4.], [5., 6., 7., 8.]])
    np.testing.assert_array_equal(v2.token_mix(x, 2), [[1., 2., 5., 6.], [3., 4., 7., 8.]])


def test_token_mix_is_an_involution_and_a_permutation_per_parent():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3 * 4, 16))
    y = v2.token_mix(x, 4)
    np.testing.assert_array_equal(v2.token_mix(y, 4), x)       # square chunk grid: mixing twice is the identity
    for p in range(3):
        np.testing.assert_array_equal(np.sort(y[4 * p:4 * p + 4].ravel()), np.sort(x[4 * p:4 * p + 4].ravel()))
    # chunk c of output token c comes from token c itself: the grid diagonal stays in place
    for c in range(4):
        np.testing.assert_array_equal(y[c, 4 * c:4 * c + 4], x[c, 4 * c:4 * c + 4])
    np.testing.assert_array_equal(v2.token_mix(x, 1), x)


def test_autosplit_is_a_linear_map_cut_into_sub_tokens():
    rng = np.random.default_rng(2)
    f = rng.standard_normal((5, 7))
    w = rng.standard_normal((3 * 6, 7))
    out = v2.autosplit(f, w, 3)
    ref = torch.nn.functional.linear(torch.from_numpy(f), torch.from_numpy(w)).numpy()   # library routine
    assert out.shape == (15, 6)
    np.testing.assert_allclose(out.reshape(5, 18), ref, rtol=1e-12, atol=1e-12)
    # permuting the weight's row blocks permutes the sub-tokens
    wp = np.concatenate([w[12:18], w[0:6], w[6:12]])
    op = v2.autosplit(f, wp, 3).reshape(5, 3, 6)
    np.testing.assert_array_equal(op[:, 1], out.reshape(5, 3, 6)[:, 0])


def test_token_ffn_against_torch_and_closed_forms():
    rng = np.random.default_rng(3)
    S, d, dff, P = 4, 8, 6, 3
    x = rng.standard_normal((P * S, d))
    w = {"ln_g": 1 + 0.1 * rng.standard_normal((3, d)), "ln_b": 0.1 * rng.standard_normal((3, d)),
         "w_gate": rng.standard_normal((S, dff, d)), "w_up": rng.standard_normal((S, dff, d)),
         "w_down": rng.standard_normal((S, d, dff))}
    out = v2.token_ffn(x, w, S, 1e-5)
    xt = torch.from_numpy(x)
    xn = torch.nn.functional.layer_norm(xt, (d,), torch.from_numpy(w["ln_g"][2]), torch.from_numpy(w["ln_b"][2]), 1e-5)
    for z in range(S):
        h = torch.nn.functional.silu(xn[z::S] @ torch.from_numpy(w["w_gate"][z]).T) * (xn[z::S] @ torch.from_numpy(w["w_up"][z]).T)
        ref = xt[z::S] + h @ torch.from_numpy(w["w_down"][z]).T
        np.testing.assert_allclose(out[z::S], ref.numpy(), rtol=1e-10, atol=1e-10)
    # zero gate: SiLU(0) = 0 kills the branch; zero down projection likewise
    for k in ("w_gate", "w_down"):
        w0 = dict(w); w0[k] = np.zeros_like(w[k])
        np.testing.assert_array_equal(v2.token_ffn(x, w0, S, 1e-5), x)


def test_mean_pool():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 5))
    np.testing.assert_allclose(v2.mean_pool(x, 3), x.reshape(2, 3, 5).mean(1))
    same = np.repeat(rng.standard_normal((2, 5)), 4, axis=0)
    np.testing.assert_allclose(v2.mean_pool(same, 4), same[::4])


def test_pooling_after_mixing_averages_each_tokens_own_chunks():
    # output token c, chunk z = input token z, chunk c; so chunk z of the pooled vector is
    # the mean over c of input token z's chunks
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 8))
    pooled = v2.mean_pool(v2.token_mix(x, 4), 4)[0]
    for z in range(4):
        np.testing.assert_allclose(pooled[2 * z:2 * z + 2], x[z].reshape(4, 2).mean(0), rtol=1e-14)


@pytest.mark.parametrize("split", [1, 4])
def test_v2_stack_reduces_to_v1_without_ffn(split):
    """Zero down projections: the FFN adds nothing; with S = 1 the mixing is the identity, so the V2
    stack is the V1 stack; with S = 4 it is the V1 stack with the T rows' chunks permuted after each
    target layer (checked against mixing applied by hand)."""
    rng = np.random.default_rng(40 + split)
    dims = synth.Dims(16, 4, 2, 4, ln_eps=1e-3)
    b = synth.make_batch(rng, np.asarray([[5, 3, 2], [3, 4, 1], [2, 0, 2]], np.int32), split)
    x = rng.standard_normal((b.total_rows, dims.d_model))
    full = [{k: v.astype(np.float64) for k, v in synth.full_weights(rng, dims, 0.3, 0.3).items()} for _ in range(2)]
    tgt = [{k: v.astype(np.float64) for k, v in synth.target_weights(rng, dims, split, 0.3, 0.3).items()}
           for _ in range(2)]
    ffn = [{"ln_g": np.ones((3, 16)), "ln_b": np.zeros((3, 16)), "w_gate": rng.standard_normal((split, 8, 16)),
            "w_up": rng.standard_normal((split, 8, 16)), "w_down": np.zeros((split, 16, 8))} for _ in range(2)]
    got = v2.backbone_v2(b, x, full, tgt, ffn, dims, 2, 1)
    if split == 1:
        np.testing.assert_allclose(got, om.backbone(b, x, full, tgt, dims, 2, 1), rtol=0, atol=1e-12)
    else:
        # by hand: V1 layers, mixing the T rows after each target layer
        ref = np.array(x, np.float64)
        tr = v2.t_rows(b)
        for blk in range(2):
            ref = om.full_layer(b, ref, full[blk], dims)
            ref = om.target_layer(b, ref, tgt[blk], dims)
            ref[tr] = v2.token_mix(ref[tr], split)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
