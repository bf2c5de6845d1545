"""Debug entry points on the GPU.

mtfm_mask_dense rebuilds one user's dense visibility matrix from the
metadata alone; it must equal the oracle's enumeration of the mask rules
element for element (the metadata claims the visible context is a prefix
plus the T row's own column).  mtfm_validate_batch must flag planted
violations of the data-level contracts and nothing else.
"""
import numpy as np
import pytest

import synth
from oracle import mask as omask

pytestmark = pytest.mark.gpu


def _user_ts(batch, u):
    ro = np.concatenate([[0], np.cumsum(batch.lens[:, 1])])
    to = np.concatenate([[0], np.cumsum(batch.lens[:, 2])])
    return batch.ts_r[ro[u]:ro[u + 1]], batch.ts_t[to[u]:to[u + 1]]


@pytest.mark.parametrize("split", [1, 4])
def test_mask_dense_equals_the_oracle_mask(split):
    """Random small users with empty sections and timestamp ties, and two users near tile edges."""
    from hybrid_masked_attention_amd import binding as B
    rng = np.random.default_rng(60 + split)
    dims = synth.Dims(16, 2, 1, 8)
    small = synth.random_small(rng, 12, split, dims, allow_empty=True)
    edge = synth.make_batch(rng, np.asarray([[63, 1, 17], [64, 65, 2]], np.int32), split)
    for batch in (small, edge):
        db = B.DeviceBatch.from_synth(batch)
        meta = B.mask_build(db)
        for u in range(batch.n_users):
            lh, lr, lt = (int(v) for v in batch.lens[u])
            ts_r, ts_t = _user_ts(batch, u)
            ref = omask.dense_mask_fast(lh, lr, lt, split, ts_r, ts_t)
            got = B.mask_dense(db, meta, u).cpu().numpy()
            np.testing.assert_array_equal(got, ref, err_msg=f"user {u} lens {(lh, lr, lt)}")


def test_validate_batch_flags_planted_violations():
    import torch
    from hybrid_masked_attention_amd import binding as B
    rng = np.random.default_rng(64)
    lens = np.asarray([[5, 4, 2], [3, 0, 1], [0, 6, 3], [7, 5, 0]], np.int32)
    batch = synth.make_batch(rng, lens, 1)
    assert B.validate_batch(B.DeviceBatch.from_synth(batch)) == 0

    # action times out of order inside user 2 (its R segment starts after users 0 and 1: 4 + 0)
    ts = batch.ts_r.copy()
    ts[4], ts[5] = ts[5] + 1, ts[4]
    bad = synth.Batch(lens, 1, ts, batch.ts_t)
    assert B.validate_batch(B.DeviceBatch.from_synth(bad)) == B.BAD_ACTION_ORDER

    # a drop from one user's last action to the next user's first is allowed
    ts = batch.ts_r.copy()
    ts[:4] += 1000
    ok = synth.Batch(lens, 1, ts, batch.ts_t)
    assert B.validate_batch(B.DeviceBatch.from_synth(ok)) == 0

    # device lengths that differ from the host lengths: two users swapped (same totals),
    # then one length changed
    for dev in ([[3, 0, 1], [5, 4, 2], [0, 6, 3], [7, 5, 0]], [[5, 4, 2], [3, 0, 1], [0, 7, 3], [7, 5, 0]]):
        db = B.DeviceBatch.from_synth(batch)
        db.lens_d.copy_(torch.as_tensor(np.asarray(dev, np.int32)))
        assert B.validate_batch(db) & B.BAD_LENGTHS

    # an empty batch has nothing to violate
    empty = synth.Batch(np.zeros((0, 3), np.int32), 1, np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert B.validate_batch(B.DeviceBatch.from_synth(empty)) == 0
