"""Host side of the attention work order (no GPU): the metadata layout sizes
the order arrays by the rule in tests/_order.py, and the rule's own properties
hold (every non-empty slice listed once, a user's slices together on one XCD,
last first, the XCD loads within one user's work of each other)."""
import os

import numpy as np
import pytest

import synth
from tests import _order

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from hybrid_masked_attention_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from hybrid_masked_attention_amd import build
        build.build()
    binding.lib()
    return binding


def _batches():
    rng = np.random.default_rng(11)
    yield "config1", synth.config1().batch
    yield "config2_s4", synth.config2(4).batch
    yield "config3", synth.config3(weights=False).batch
    yield "config4", synth.config4(arrays=False).batch
    dims = synth.config0().dims
    yield "random_s1", synth.random_small(rng, 37, 1, dims)
    yield "random_s4", synth.random_small(rng, 19, 4, dims)
    lens = np.array([[0, 0, 0], [5, 0, 0], [0, 0, 3], [700, 90, 0], [1, 1, 1]], np.int32)
    yield "degenerate", synth.make_batch(rng, lens, 1)


def _layout(B, batch):
    db = B.DeviceBatch(batch.lens, batch.split, batch.ts_r, batch.ts_t, device=None)
    return B.meta_layout(db)


@pytest.mark.parametrize("name,batch", list(_batches()), ids=[n for n, _ in _batches()])
def test_layout_sizes_the_orders_by_the_rule(B, name, batch):
    lay = _layout(B, batch)
    assert lay.n_full_order == len(_order.expected_order(batch.lens, batch.split, _order.FULL))
    assert lay.n_target_order == len(_order.expected_order(batch.lens, batch.split, _order.TARGET))
    assert lay.off_full_order % 256 == 0 and lay.off_target_order % 256 == 0
    assert lay.off_parent_row <= lay.off_full_order <= lay.off_target_order <= lay.off_tsort_q <= lay.total_bytes


def test_no_order_past_the_user_limit(B):
    lens = np.tile(np.array([[3, 2, 1]], np.int32), (_order.MAX_USERS + 1, 1))
    batch = synth.make_batch(np.random.default_rng(0), lens, 1)
    lay = _layout(B, batch)
    assert lay.n_full_order == 0 and lay.n_target_order == 0
    lay = _layout(B, synth.make_batch(np.random.default_rng(0), lens[:_order.MAX_USERS], 1))
    assert lay.n_full_order > 0 and lay.n_target_order > 0


@pytest.mark.parametrize("layer", [_order.FULL, _order.TARGET])
@pytest.mark.parametrize("name,batch", list(_batches()), ids=[n for n, _ in _batches()])
def test_rule_properties(name, batch, layer):
    lens = batch.lens.astype(np.int64)
    order = _order.expected_order(lens, batch.split, layer)
    if len(order) == 0:
        assert batch.n_users == 0 or not _order.balanced(lens, batch.split, layer)
        return
    ns = _order.slices(lens, batch.split, layer)
    tiles = (ns + 1) // 2
    first = np.concatenate([[0], np.cumsum(tiles)[:-1]])
    owner = np.repeat(np.arange(len(lens)), 2 * tiles)
    listed = order[order >= 0]
    # every non-empty slice exactly once
    want = np.concatenate([2 * first[u] + np.arange(ns[u]) for u in range(len(lens))]) if len(lens) else []
    assert sorted(listed.tolist()) == sorted(np.asarray(want).tolist())
    work = _order.user_work(lens, batch.split, layer)
    loads = []
    for x in range(8):
        col = order[x::8]
        k = int(np.sum(col >= 0))
        assert np.all(col[:k] >= 0) and np.all(col[k:] == -1)      # the list, then padding
        users = owner[col[:k]]
        # a user's slices are consecutive, last first
        for u in np.unique(users):
            pos = np.nonzero(users == u)[0]
            assert np.all(np.diff(pos) == 1)
            assert np.all(np.diff(col[:k][pos]) == -1)
        # users in non-increasing work order
        seq = [users[0]] + [users[i] for i in range(1, len(users)) if users[i] != users[i - 1]] if k else []
        assert all(work[a] >= work[b] for a, b in zip(seq, seq[1:]))
        loads.append(int(sum(work[u] for u in seq)))
    if len(lens) >= 8:
        assert max(loads) - min(loads) <= int(work.max())


def test_unbalanced_dealing_keeps_the_plain_order(B):
    """A few users, or one user far longer than the rest, would put most of the work on one or
    two XCDs: such batches get no order (the kernels' XCD-contiguous order spreads the long user's
    slices over all of them); the benchmarked configurations keep theirs."""
    rng = np.random.default_rng(5)
    lopsided = np.array([[37, 20, 3], [200000, 61992, 8]], np.int32)
    few = np.array([[1000, 200, 20]] * 4, np.int32)
    one_long = np.concatenate([np.array([[3000, 500, 40]], np.int32), np.tile([[40, 10, 2]], (60, 1)).astype(np.int32)])
    for lens in (lopsided, few, one_long):
        batch = synth.make_batch(rng, lens, 1)
        lay = _layout(B, batch)
        assert lay.n_full_order == 0 and lay.n_target_order == 0, lens[:3]
        assert not _order.balanced(lens, 1, _order.FULL)
    for batch in (synth.config1().batch, synth.config3(weights=False).batch, synth.config4(arrays=False).batch):
        lay = _layout(B, batch)
        assert lay.n_full_order > 0 and lay.n_target_order > 0
