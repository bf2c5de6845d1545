"""Pins of the oracle's layers (CPU only).

Each test fixes a fact that a plausible slip would break: library special
cases (torch LayerNorm, SiLU), a hand-worked attention example, closed forms
when Q, K or U vanish, the GQA head-to-group map, the invariants the mask
implies, and the identity between the target layer and the T rows of the full
layer ([explainer] §4.2: the target layer is the full layer restricted to T
queries).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import mask as om
from oracle import model as om_model


def small_workload(rng, lens, split=1, dims=None, x_std=1.0, w_std=0.2, n_users=None):
    dims = dims or synth.Dims(16, 4, 2, 4)
    b = synth.make_batch(rng, np.asarray(lens, np.int32).reshape(-1, 3), split)
    x = x_std * rng.standard_normal((b.total_rows, dims.d_model))
    wf = synth.full_weights(rng, dims, w_std, w_std)
    wt = synth.target_weights(rng, dims, split, w_std, w_std)
    return b, dims, x, wf, wt


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(om_model.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-300)


def test_gln_unit_affine_matches_torch_layer_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 3 + 1
    types = rng.integers(0, 3, size=7)
    ones, zeros = np.ones((3, 33)), np.zeros((3, 33))
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (33,), eps=1e-5).numpy()
    np.testing.assert_allclose(om_model.gln(x, ones, zeros, types, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_gln_type_indexing():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 8))
    types = np.array([0, 1, 2, 2, 1, 0])
    g = rng.standard_normal((3, 8)); b = rng.standard_normal((3, 8))
    base = torch.nn.functional.layer_norm(torch.from_numpy(x), (8,), eps=1e-3).numpy()
    out = om_model.gln(x, g, b, types, 1e-3)
    for i, t in enumerate(types):
        np.testing.assert_allclose(out[i], base[i] * g[t] + b[t], rtol=1e-12, atol=1e-12)


def test_attention_hand_worked_example():
    # one head, dh = 4 (scale 1/2).  q = (2,0,0,0); keys k_j = (a_j,0,0,0) with
    # a = (2, 0, -2, 4) give scores a_j;  SiLU(2) = 2/(1+e^-2) = 1.7615941559557649,
    # SiLU(0) = 0, SiLU(-2) = -0.2384058440442351, SiLU(4) = 3.928055160151634.
    # Values v_j = e_j (one-hot over 4 columns).  The mask shows keys 0, 1, 2 to
    # row 0 (n = 3) and keys 0 and 3 to row 1 (n = 2).
    q = np.array([[2.0, 0, 0, 0], [2.0, 0, 0, 0]])
    k = np.array([[2.0, 0, 0, 0], [0.0, 0, 0, 0], [-2.0, 0, 0, 0], [4.0, 0, 0, 0]])
    v = np.eye(4)
    m = np.array([[1, 1, 1, 0], [1, 0, 0, 1]], np.uint8)
    a = om_model.masked_attention(q, k, v, m, 1, 1, 4)
    exp = np.array([[1.7615941559557649 / 3, 0.0, -0.2384058440442351 / 3, 0.0],
                    [1.7615941559557649 / 2, 0.0, 0.0, 3.928055160151634 / 2]])
    np.testing.assert_allclose(a, exp, rtol=1e-14, atol=1e-15)


def test_gqa_head_to_group_map():
    rng = np.random.default_rng(2)
    H, G, dh = 4, 2, 3
    q = rng.standard_normal((5, H * dh)); k = rng.standard_normal((6, G * dh)); v = rng.standard_normal((6, G * dh))
    v[:, dh:] = 0.0                                  # group 1 values vanish
    m = np.ones((5, 6), np.uint8)
    a = om_model.masked_attention(q, k, v, m, H, G, dh)
    assert np.all(a[:, 2 * dh:] == 0)                # heads 2, 3 use group 1 (h // r, r = 2)
    assert np.all(np.abs(a[:, :2 * dh]).sum(axis=1) > 0)
    # replicating each group r times and running as multi-head attention is the same
    k_rep = np.concatenate([k[:, (h // 2) * dh:(h // 2 + 1) * dh] for h in range(H)], axis=1)
    v_rep = np.concatenate([v[:, (h // 2) * dh:(h // 2 + 1) * dh] for h in range(H)], axis=1)
    np.testing.assert_allclose(om_model.masked_attention(q, k_rep, v_rep, m, H, H, dh), a, rtol=1e-13)


def test_attention_linear_in_v():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 8)); k = rng.standard_normal((5, 4))
    v1, v2 = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    m = (rng.random((4, 5)) < 0.6).astype(np.uint8); m[:, 0] = 1
    f = lambda v: om_model.masked_attention(q, k, v, m, 2, 1, 4)
    np.testing.assert_allclose(f(v1 + 2.5 * v2), f(v1) + 2.5 * f(v2), rtol=1e-12, atol=1e-12)


def _layer_norm_np(x, eps):
    return torch.nn.functional.layer_norm(torch.from_numpy(np.asarray(x, np.float64)), (x.shape[1],), eps=eps).numpy()


def test_full_layer_closed_form_when_queries_vanish():
    # zero Q weights -> Q = SiLU(0) = 0 -> every score 0 -> A = 0 -> GLN(A) = beta[type]
    rng = np.random.default_rng(4)
    b, dims, x, w, _ = small_workload(rng, [[5, 3, 2]])
    hd = dims.n_q_heads * dims.head_dim
    w = dict(w); w1 = w["w_uqkv"].copy(); w1[hd:2 * hd] = 0; w["w_uqkv"] = w1
    types = om.row_types(5, 3, 2, 1)
    m = om_model.user_mask(b, 0)
    out = om_model.full_layer_user(x, m, types, w, dims)
    xt = _layer_norm_np(x, dims.ln_eps) * w["ln1_g"][types] + w["ln1_b"][types]
    u = torch.nn.functional.silu(torch.from_numpy(xt @ w1[:hd].astype(np.float64).T)).numpy()
    ref = (w["ln2_b"][types] * u) @ w["w_o"].astype(np.float64).T + x
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_full_layer_zero_gate_is_identity():
    # zero U weights -> U = 0 -> the residual branch vanishes (split order [U|Q|K|V])
    rng = np.random.default_rng(5)
    b, dims, x, w, _ = small_workload(rng, [[4, 4, 3]])
    hd = dims.n_q_heads * dims.head_dim
    w = dict(w); w1 = w["w_uqkv"].copy(); w1[:hd] = 0; w["w_uqkv"] = w1
    out = om_model.full_layer(b, x, w, dims)
    np.testing.assert_array_equal(out, x)


def test_full_layer_zero_values_gives_beta_gate():
    # zero V weights -> V = 0 -> A = 0, same closed form as vanishing queries
    rng = np.random.default_rng(6)
    b, dims, x, w, _ = small_workload(rng, [[3, 2, 2]])
    hd, gd = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    w = dict(w); w1 = w["w_uqkv"].copy(); w1[2 * hd + gd:] = 0; w["w_uqkv"] = w1
    types = om.row_types(3, 2, 2, 1)
    out, parts = om_model.full_layer_user(x, om_model.user_mask(b, 0), types, w, dims, return_parts=True)
    assert np.all(parts["a"] == 0)
    np.testing.assert_allclose(parts["y"], w["ln2_b"][types] * parts["u"], rtol=1e-12, atol=1e-14)


def test_invariant_t_row_ignores_other_targets_and_later_actions():
    rng = np.random.default_rng(8)
    dims = synth.Dims(16, 4, 2, 4)
    for split in (1, 4):
        b = synth.Batch(np.array([[4, 5, 3]], np.int32), split, np.array([1, 3, 3, 8, 9], np.int32),
                        np.array([3, 9, 20], np.int32))
        x = rng.standard_normal((b.total_rows, dims.d_model))
        w = synth.full_weights(rng, dims, 0.3, 0.3)
        wt = synth.target_weights(rng, dims, split, 0.3, 0.3)
        base_f = om_model.full_layer(b, x, w, dims)
        base_t = om_model.target_layer(b, x, wt, dims)
        lc = 9
        i = lc  # first sub-token of target 0 (exposure 3: sees the action at time 1 only)
        x2 = x.copy()
        x2[lc + split:] += rng.standard_normal(x2[lc + split:].shape)      # other targets
        x2[4 + 1:4 + 5] += rng.standard_normal((4, dims.d_model))          # actions at >= 3
        for layer, base in ((om_model.full_layer, base_f), (om_model.target_layer, base_t)):
            out = layer(b, x2, w if layer is om_model.full_layer else wt, dims)
            np.testing.assert_allclose(out[i:i + split], base[i:i + split], rtol=1e-12, atol=1e-12)


def test_invariant_h_rows_ignore_r_and_t():
    rng = np.random.default_rng(9)
    b, dims, x, w, _ = small_workload(rng, [[6, 4, 3]])
    base = om_model.full_layer(b, x, w, dims)
    x2 = x.copy(); x2[6:] += rng.standard_normal(x2[6:].shape)
    np.testing.assert_allclose(om_model.full_layer(b, x2, w, dims)[:6], base[:6], rtol=1e-12, atol=1e-12)


def test_target_layer_keeps_context_rows_bit_exact():
    rng = np.random.default_rng(10)
    b, dims, x, _, wt = small_workload(rng, [[6, 4, 3], [2, 0, 1], [3, 3, 0]], split=4)
    out = om_model.target_layer(b, x, wt, dims)
    for u in range(b.n_users):
        r0 = b.row_off[u]; lc = int(b.lens[u, 0] + b.lens[u, 1])
        np.testing.assert_array_equal(out[r0:r0 + lc], x[r0:r0 + lc])


def test_target_layer_equals_full_layer_t_rows():
    rng = np.random.default_rng(12)
    b, dims, x, wf, _ = small_workload(rng, [[7, 5, 4], [3, 6, 2], [5, 0, 3]])
    hd, gd = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    w1 = wf["w_uqkv"]
    wt = {"w_u": w1[:hd], "w_q": w1[hd:2 * hd][None], "w_kv": w1[2 * hd:],
          "w_o": wf["w_o"], "ln1_g": wf["ln1_g"], "ln1_b": wf["ln1_b"], "ln2_g": wf["ln2_g"], "ln2_b": wf["ln2_b"]}
    full = om_model.full_layer(b, x, wf, dims)
    tgt = om_model.target_layer(b, x, wt, dims)
    for u in range(b.n_users):
        r0, r1 = b.row_off[u], b.row_off[u + 1]
        lc = int(b.lens[u, 0] + b.lens[u, 1])
        np.testing.assert_allclose(tgt[r0 + lc:r1], full[r0 + lc:r1], rtol=1e-12, atol=1e-12)


def test_v2_subtokens_use_their_own_q():
    rng = np.random.default_rng(13)
    dims = synth.Dims(16, 4, 2, 4)
    b = synth.Batch(np.array([[4, 3, 2]], np.int32), 4, np.array([1, 2, 3], np.int32), np.array([5, 2], np.int32))
    x = rng.standard_normal((b.total_rows, dims.d_model))
    wt = synth.target_weights(rng, dims, 4, 0.3, 0.3)
    base = om_model.target_layer(b, x, wt, dims)
    # swapping W_q[1] and W_q[2] together with the X rows of sub-tokens 1 and 2 swaps their outputs
    w2 = dict(wt); wq = wt["w_q"].copy(); wq[[1, 2]] = wq[[2, 1]]; w2["w_q"] = wq
    x2 = x.copy(); lc = 7
    for t in range(2):
        x2[[lc + 4 * t + 1, lc + 4 * t + 2]] = x2[[lc + 4 * t + 2, lc + 4 * t + 1]]
    out = om_model.target_layer(b, x2, w2, dims)
    for t in range(2):
        np.testing.assert_allclose(out[lc + 4 * t + 1], base[lc + 4 * t + 2], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out[lc + 4 * t + 2], base[lc + 4 * t + 1], rtol=1e-12, atol=1e-12)
    # identical W_q[k] and identical sub-token inputs give identical sub-token outputs
    w3 = dict(wt); w3["w_q"] = np.repeat(wt["w_q"][:1], 4, axis=0)
    x3 = x.copy()
    for t in range(2):
        x3[lc + 4 * t:lc + 4 * t + 4] = x3[lc + 4 * t]
    out3 = om_model.target_layer(b, x3, w3, dims)
    for t in range(2):
        for s in range(1, 4):
            np.testing.assert_allclose(out3[lc + 4 * t + s], out3[lc + 4 * t], rtol=1e-12, atol=1e-12)


def test_batch_is_concatenation_and_user_order_is_irrelevant():
    rng = np.random.default_rng(14)
    b, dims, x, wf, wt = small_workload(rng, [[5, 2, 2], [3, 4, 1], [6, 0, 3]], split=4)
    for layer, w in ((om_model.full_layer, wf), (om_model.target_layer, wt)):
        whole = layer(b, x, w, dims)
        perm = [2, 0, 1]
        bp = b.subset(perm)
        xp = x[b.rows_of(perm)]
        outp = layer(bp, xp, w, dims)
        np.testing.assert_allclose(outp, whole[b.rows_of(perm)], rtol=1e-13, atol=1e-13)


def test_all_history_user_is_unmasked_attention():
    # L_R = L_T = 0: every row sees every key; A = SiLU(Q K^T / sqrt(dh)) V / N, computed with torch
    rng = np.random.default_rng(15)
    b, dims, x, w, _ = small_workload(rng, [[9, 0, 0]])
    _, parts = om_model.full_layer(b, x, w, dims, return_parts=True)
    types = om.row_types(9, 0, 0, 1)
    xt = _layer_norm_np(x, dims.ln_eps) * w["ln1_g"][types] + w["ln1_b"][types]
    z = torch.nn.functional.silu(torch.from_numpy(xt @ w["w_uqkv"].astype(np.float64).T))
    hd, gd, dh = 16, 8, 4
    q = z[:, hd:2 * hd].reshape(9, 4, dh).transpose(0, 1)
    k = z[:, 2 * hd:2 * hd + gd].reshape(9, 2, dh).transpose(0, 1).repeat_interleave(2, 0)
    v = z[:, 2 * hd + gd:].reshape(9, 2, dh).transpose(0, 1).repeat_interleave(2, 0)
    a = (torch.nn.functional.silu(q @ k.transpose(1, 2) / math.sqrt(dh)) @ v) / 9
    np.testing.assert_allclose(parts["a"], a.transpose(0, 1).reshape(9, hd).numpy(), rtol=1e-12, atol=1e-14)


def test_backbone_keeps_context_rows_through_target_layers():
    rng = np.random.default_rng(16)
    b, dims, x, wf, wt = small_workload(rng, [[6, 3, 2]])
    types = om.row_types(6, 3, 2, 1)
    m = om_model.user_mask(b, 0)
    out = om_model.backbone_user(x, m, types, 9, 1, [wf], [wt, wt], dims, 1, 2)
    after_full = om_model.full_layer_user(x, m, types, wf, dims)
    np.testing.assert_array_equal(out[:9], after_full[:9])
    t1 = om_model.target_layer_user(after_full, m, types, 9, 1, wt, dims)
    np.testing.assert_allclose(out, om_model.target_layer_user(t1, m, types, 9, 1, wt, dims), rtol=1e-13)


@pytest.mark.parametrize("lens,split", [((9, 7, 4), 1), ((5, 0, 3), 3), ((12, 6, 0), 1), ((1, 1, 1), 1), ((0, 4, 2), 2)])
def test_full_layer_rows_equals_dense_full_layer(lens, split):
    """full_layer_rows (per-row masks, selected query rows) gives the rows of the dense full layer."""
    rng = np.random.default_rng(12)
    b, dims, x, wf, _ = small_workload(rng, [lens], split)
    l_h, l_r, l_t = lens
    m = om.dense_mask(l_h, l_r, l_t, split, b.ts_r, b.ts_t)
    ref = om_model.full_layer_user(x, m, om.row_types(l_h, l_r, l_t, split), wf, dims)
    rows = rng.permutation(x.shape[0])[:max(1, x.shape[0] // 2)]
    got = om_model.full_layer_rows(x, l_h, l_r, l_t, split, b.ts_r, b.ts_t, wf, dims, rows)
    np.testing.assert_allclose(got, ref[rows], rtol=1e-12, atol=1e-12)
