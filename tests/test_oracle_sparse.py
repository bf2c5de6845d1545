"""Pins of oracle.sparse (2:4 structured pruning, [explainer] §5.2.1) against
what the definition fixes: worked groups, the two-largest rule restated as a
search over all pairs, and invariants of the operation."""
import itertools

import numpy as np
import pytest

from oracle import sparse as osp


def test_worked_groups():
    w = np.array([[0.5, -2.0, 1.0, 0.1,   1.0, -1.0, 1.0, -1.0,   0.0, 0.0, 0.0, 3.0,   -4.0, 4.0, 0.25, -0.5]])
    ref = np.array([[0.0, -2.0, 1.0, 0.0,  1.0, -1.0, 0.0, 0.0,    0.0, 0.0, 0.0, 3.0,   -4.0, 4.0, 0.0, 0.0]])
    np.testing.assert_array_equal(osp.prune_24(w), ref)
    # ties go to the lower position: of [1, -1, 1, -1] positions 0 and 1 stay
    np.testing.assert_array_equal(osp.keep_mask_24(w)[0, 4:8], [True, True, False, False])
    # in an all-zero-but-one group the kept zero is the lowest position
    np.testing.assert_array_equal(osp.keep_mask_24(w)[0, 8:12], [True, False, False, True])


def _best_pair(g):
    """The definition as a search: the pair of positions with the largest magnitude sum, the
    lexicographically smallest such pair on ties."""
    best = None
    for pair in itertools.combinations(range(4), 2):
        s = abs(g[pair[0]]) + abs(g[pair[1]])
        if best is None or s > best[0]:
            best = (s, pair)
    return best[1]


@pytest.mark.parametrize("seed", [0, 1])
def test_two_largest_equals_the_best_pair(seed):
    rng = np.random.default_rng(seed)
    # small integers make ties frequent
    w = rng.integers(-3, 4, size=(6, 32)).astype(np.float64)
    keep = osp.keep_mask_24(w)
    for r in range(w.shape[0]):
        for q in range(8):
            g = w[r, 4 * q:4 * q + 4]
            pair = _best_pair(g)
            expect = np.zeros(4, bool)
            expect[list(pair)] = True
            np.testing.assert_array_equal(keep[r, 4 * q:4 * q + 4], expect, err_msg=f"row {r} group {q}: {g}")


def test_invariants():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((3, 5, 64))
    p = osp.prune_24(w)
    g, gp = w.reshape(-1, 4), p.reshape(-1, 4)
    assert np.all((gp != 0).sum(axis=1) <= 2)
    kept = gp != 0
    np.testing.assert_array_equal(gp[kept], g[kept])                    # kept values unchanged
    mags = np.abs(g)
    for row, k in zip(mags, kept):                                      # nothing dropped is larger
        if k.any() and (~k).any():
            assert row[~k].max() <= row[k].min()
    np.testing.assert_array_equal(osp.prune_24(p), p)                   # idempotent
    np.testing.assert_array_equal(osp.prune_24(-w), -p)                 # sign symmetric
    perm = rng.permutation(16)                                          # groups are independent
    wg = w.reshape(3, 5, 16, 4)[:, :, perm].reshape(w.shape)
    np.testing.assert_array_equal(osp.prune_24(wg), p.reshape(3, 5, 16, 4)[:, :, perm].reshape(w.shape))
    np.testing.assert_array_equal(p, w * osp.keep_mask_24(w))


def test_layer_weights_prune_only_the_projections():
    rng = np.random.default_rng(3)
    full = {"ln1_g": rng.standard_normal((3, 8)), "ln1_b": rng.standard_normal((3, 8)),
            "w_uqkv": rng.standard_normal((20, 8)), "ln2_g": rng.standard_normal((3, 8)),
            "ln2_b": rng.standard_normal((3, 8)), "w_o": rng.standard_normal((8, 8))}
    pf = osp.prune_full_weights(full)
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        assert pf[k] is full[k]
    for k in ("w_uqkv", "w_o"):
        np.testing.assert_array_equal(pf[k], osp.prune_24(full[k]))
    tgt = dict(full, w_u=rng.standard_normal((8, 8)), w_q=rng.standard_normal((4, 8, 8)),
               w_kv=rng.standard_normal((4, 8)))
    del tgt["w_uqkv"]
    pt = osp.prune_target_weights(tgt)
    for k in ("w_u", "w_q", "w_kv", "w_o"):
        np.testing.assert_array_equal(pt[k], osp.prune_24(tgt[k]))
