"""Pins of the oracle's mask and metadata (CPU only).

The worked 7x7 matrix of [explainer] §8.2 is the one printed example; the rest
are structural facts the rules imply, checked by brute force on many tiny
random users (ties, empty parts, V2 split 4).
"""
import os

import numpy as np
import pytest

import synth
from oracle import mask as om
from oracle import model as omodel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_3h2r2t.txt")


def _golden():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    return np.array(rows, dtype=np.uint8)


def test_mask_golden_example():
    # both exposures after both R actions, as the table implies
    m = om.dense_mask(3, 2, 2, 1, ts_r=[10, 20], ts_t=[30, 40])
    np.testing.assert_array_equal(m, _golden())
    assert np.array_equal(omodel.dense_mask_fast(3, 2, 2, 1, [10, 20], [30, 40]), _golden())


def _block_form(l_h, l_r, l_t, split):
    """The §8.2 pattern at any size when every exposure follows every R action."""
    n_t = split * l_t
    n = l_h + l_r + n_t
    m = np.zeros((n, n), np.uint8)
    m[:, :l_h] = 1                                  # H columns: everyone
    m[:l_h, l_h:] = 0                               # H rows: H only
    m[l_h:l_h + l_r, l_h:l_h + l_r] = np.tril(np.ones((l_r, l_r), np.uint8))
    m[l_h + l_r:, l_h:l_h + l_r] = 1                # T rows see all R
    m[l_h + l_r:, l_h + l_r:] = np.eye(n_t, dtype=np.uint8)
    return m


@pytest.mark.parametrize("lens,split", [((5, 4, 3), 1), ((0, 3, 2), 4), ((7, 0, 2), 4), ((2, 6, 0), 1)])
def test_mask_block_form_when_all_actions_precede_exposures(lens, split):
    l_h, l_r, l_t = lens
    ts_r = np.sort(np.arange(l_r) * 3)
    ts_t = np.full(l_t, 10_000)
    m = om.dense_mask(l_h, l_r, l_t, split, ts_r, ts_t)
    np.testing.assert_array_equal(m, _block_form(l_h, l_r, l_t, split))


def test_mask_targets_before_all_actions_see_no_r():
    m = om.dense_mask(3, 4, 2, 4, ts_r=[5, 6, 7, 8], ts_t=[5, 0])
    lc = 7
    assert m[lc:, 3:7].sum() == 0      # exposure at/below every action: no R visible (strict <)
    assert np.all(m[lc:, :3] == 1)     # H still visible


def test_mask_ties_are_strict():
    # exposure time equal to an action's time: that action is not "before" the exposure
    m = om.dense_mask(1, 3, 1, 1, ts_r=[4, 7, 7], ts_t=[7])
    np.testing.assert_array_equal(m[4, 1:4], [1, 0, 0])


def test_mask_v2_siblings_invisible_and_share_exposure():
    m = om.dense_mask(2, 3, 2, 4, ts_r=[1, 5, 9], ts_t=[6, 100])
    t0 = slice(5, 9)
    np.testing.assert_array_equal(m[t0, 5:13], np.eye(4, 8, dtype=np.uint8))
    np.testing.assert_array_equal(m[t0, 2:5], np.tile([1, 1, 0], (4, 1)))
    np.testing.assert_array_equal(m[9:13, 2:5], np.ones((4, 3), np.uint8))


def test_enumeration_equals_broadcast_form():
    rng = np.random.default_rng(123)
    for _ in range(300):
        b = synth.random_small(rng, 1, int(rng.choice([1, 4])), None)
        l_h, l_r, l_t = (int(v) for v in b.lens[0])
        a = om.dense_mask(l_h, l_r, l_t, b.split, b.ts_r, b.ts_t)
        c = omodel.dense_mask_fast(l_h, l_r, l_t, b.split, b.ts_r, b.ts_t)
        np.testing.assert_array_equal(a, c)


def test_row_meta_bruteforce_properties():
    rng = np.random.default_rng(7)
    for _ in range(400):
        b = synth.random_small(rng, 1, int(rng.choice([1, 4])), None)
        l_h, l_r, l_t = (int(v) for v in b.lens[0])
        m = om.dense_mask(l_h, l_r, l_t, b.split, b.ts_r, b.ts_t)
        p, selfv, n = om.row_meta(m, l_h, l_r)   # raises unless every context row is a prefix
        assert np.all(n >= 1)                    # every row sees at least one key
        lc = l_h + l_r
        assert np.all(p[:l_h] == l_h)
        assert np.all(p[l_h:lc] == l_h + 1 + np.arange(l_r))
        assert np.all(selfv[:lc] == 0) and np.all(selfv[lc:] == 1)
        # T rows: visible R prefix = actions strictly before the parent's exposure
        for i in range(lc, m.shape[0]):
            e = b.ts_t[(i - lc) // b.split]
            assert p[i] == l_h + int(np.sum(np.asarray(b.ts_r) < e))
        assert np.array_equal(n, p + selfv)


def test_tile_classes_shape_rule():
    rng = np.random.default_rng(11)
    for _ in range(200):
        b = synth.random_small(rng, 1, int(rng.choice([1, 4])), None, max_h=20, max_r=12, max_t=4)
        l_h, l_r, l_t = (int(v) for v in b.lens[0])
        m = om.dense_mask(l_h, l_r, l_t, b.split, b.ts_r, b.ts_t)
        for bm, bn in ((4, 4), (3, 5), (8, 2)):
            for begin in (0, l_h + l_r):
                cls = om.tile_classes(m, begin, l_h + l_r, bm, bn)
                om.tile_desc_from_classes(cls)   # raises unless full*, partial*, skip*


def test_batch_meta_concatenates_users():
    rng = np.random.default_rng(5)
    b = synth.random_small(rng, 6, 4, None)
    meta = om.batch_meta(b, 4, 4)
    assert meta["p"].shape[0] == b.total_rows
    for u in range(b.n_users):
        one = om.batch_meta(b.user(u), 4, 4)
        r0, r1 = b.row_off[u], b.row_off[u + 1]
        np.testing.assert_array_equal(meta["p"][r0:r1], one["p"])
        sel = meta["full_tiles"][:, 0] == u
        np.testing.assert_array_equal(meta["full_tiles"][sel][:, 1:], one["full_tiles"][:, 1:])


# Hand-derived block classes ([blog] §6.2: the mask is pre-scanned into an index
# of the key blocks worth computing; here "skip" = 0, "partial" = 1, "full" = 2).
# Each expectation below was worked out by hand from the matrix it names, key
# tiles covering only the context columns [0, L_H + L_R) and the last key tile
# short when L_H + L_R is not a multiple of bn.
#
# Golden user ([explainer] §8.2 matrix, tests/golden): context columns 0..4,
#   rows 0-2 see cols 0-2, row 3 cols 0-3, rows 4-6 cols 0-4.
# Second user (L_H 2, L_R 3 at times 10/20/30, two targets exposed at 25 and 5):
#   rows 0-1 see cols 0-1, row 2 cols 0-2, row 3 cols 0-3, row 4 cols 0-4,
#   row 5 (exposure 25: actions 10, 20) cols 0-3, row 6 (exposure 5) cols 0-1.
_SECOND = dict(l_h=2, l_r=3, l_t=2, ts_r=[10, 20, 30], ts_t=[25, 5])

_HAND_CLASSES = [
    # (user, begin, bm, bn, classes per query tile)
    ("golden", 0, 2, 2, [[2, 1, 0], [2, 1, 0], [2, 2, 2], [2, 2, 2]]),
    ("golden", 5, 2, 2, [[2, 2, 2]]),
    ("golden", 0, 3, 2, [[2, 1, 0], [2, 2, 1], [2, 2, 2]]),
    ("golden", 5, 3, 2, [[2, 2, 2]]),
    ("golden", 0, 7, 5, [[1]]),
    ("golden", 0, 4, 3, [[2, 1], [2, 2]]),
    ("second", 0, 2, 2, [[2, 0, 0], [2, 1, 0], [2, 2, 1], [2, 0, 0]]),
    ("second", 5, 2, 2, [[2, 1, 0]]),
    ("second", 0, 3, 2, [[2, 1, 0], [2, 2, 1], [2, 0, 0]]),
    ("second", 5, 1, 4, [[2, 0], [1, 0]]),
]


def _hand_user(which):
    if which == "golden":
        return om.dense_mask(3, 2, 2, 1, ts_r=[10, 20], ts_t=[30, 40]), 5
    s = _SECOND
    return om.dense_mask(s["l_h"], s["l_r"], s["l_t"], 1, s["ts_r"], s["ts_t"]), s["l_h"] + s["l_r"]


@pytest.mark.parametrize("which,begin,bm,bn,expect", _HAND_CLASSES)
def test_tile_classes_hand_derived(which, begin, bm, bn, expect):
    m, l_ctx = _hand_user(which)
    cls = om.tile_classes(m, begin, l_ctx, bm, bn)
    np.testing.assert_array_equal(cls, np.array(expect, np.int8))


# (leading full key tiles, one past the last non-skip key tile) per query tile,
# read off the hand-derived classes above
_HAND_DESC = {
    ("golden", 0, 2, 2): [(1, 2), (1, 2), (3, 3), (3, 3)],
    ("golden", 0, 3, 2): [(1, 2), (2, 3), (3, 3)],
    ("golden", 0, 7, 5): [(0, 1)],
    ("second", 0, 2, 2): [(1, 1), (1, 2), (2, 3), (1, 1)],
    ("second", 5, 2, 2): [(1, 2)],
    ("second", 5, 1, 4): [(1, 1), (0, 1)],
}


@pytest.mark.parametrize("key", sorted(_HAND_DESC))
def test_tile_desc_hand_derived(key):
    which, begin, bm, bn = key
    m, l_ctx = _hand_user(which)
    desc = om.tile_desc_from_classes(om.tile_classes(m, begin, l_ctx, bm, bn))
    np.testing.assert_array_equal(desc, np.array(_HAND_DESC[key], np.int32))


def test_tile_desc_worked_rows():
    # rows of classes written out directly: an all-skip row, an all-full row, a
    # row ending in partial tiles, a row with no key tiles at all
    cls = np.array([[0, 0, 0], [2, 2, 2], [2, 1, 1], [1, 0, 0]], np.int8)
    np.testing.assert_array_equal(om.tile_desc_from_classes(cls), [[0, 0], [3, 3], [1, 3], [0, 1]])
    assert om.tile_desc_from_classes(np.zeros((2, 0), np.int8)).tolist() == [[0, 0], [0, 0]]
    with pytest.raises(AssertionError):
        om.tile_desc_from_classes(np.array([[2, 0, 1]], np.int8))   # a visible tile after a skipped one


def test_batch_meta_tile_tables_hand_derived():
    # the two users above as one batch at 2 x 2 tiles: the tables are
    # (user, first row in the user, rows, leading full tiles, key-tile end)
    b = synth.Batch(np.array([[3, 2, 2], [2, 3, 2]], np.int32), 1,
                    np.array([10, 20, 10, 20, 30], np.int32), np.array([30, 40, 25, 5], np.int32))
    meta = om.batch_meta(b, 2, 2)
    np.testing.assert_array_equal(meta["full_tiles"], [
        [0, 0, 2, 1, 2], [0, 2, 2, 1, 2], [0, 4, 2, 3, 3], [0, 6, 1, 3, 3],
        [1, 0, 2, 1, 1], [1, 2, 2, 1, 2], [1, 4, 2, 2, 3], [1, 6, 1, 1, 1]])
    np.testing.assert_array_equal(meta["target_tiles"], [[0, 5, 2, 3, 3], [1, 5, 2, 1, 2]])


def test_mask_row_equals_enumerated_mask():
    """mask_row restates the rules one query at a time: row for row it equals the
    pure-Python enumeration (timestamp ties, empty parts, V2 split 3)."""
    rng = np.random.default_rng(11)
    checked = 0
    for trial in range(80):
        split = (1, 3)[trial % 2]
        l_h, l_r, l_t = (int(v) for v in rng.integers(0, 6, size=3))
        if l_h + l_r + l_t == 0:
            continue
        ts_r = np.sort(rng.integers(0, 5, size=l_r))
        ts_t = rng.integers(0, 5, size=l_t)
        m = om.dense_mask(l_h, l_r, l_t, split, ts_r, ts_t)
        for i in range(m.shape[0]):
            np.testing.assert_array_equal(om.mask_row(i, l_h, l_r, l_t, split, ts_r, ts_t), m[i])
            checked += 1
    assert checked > 300
