"""The benchmark's tile-padding figure: pairs the attention kernel computes over visible pairs.

bench.computed_pairs walks a layer's tile list the way the bf16 attention kernel does (32-row
slices, 64-key tiles from the user's aligned first row up to the slice's largest visible prefix,
both 32-key blocks of the tiles below the slice's smallest prefix, the blocks some row sees in the
others, 32 x 32 pairs per block, one pair per T row's self term).  Expected counts below are worked
by hand for users small enough to count.
"""
import numpy as np

import bench


def _tiles(rows_per_tile, urow0=0):
    """Full-layer tile descriptors of one user starting at packed row urow0."""
    out, r0 = [], 0
    for nr in rows_per_tile:
        out.append((0, r0, nr, 0, 0, urow0 + r0, urow0 + r0, urow0))
        r0 += nr
    return np.array(out, np.int32)


def test_history_only_user_of_whole_tiles_wastes_nothing():
    # 128 H rows, each seeing the 128 H keys: 4 slices x 2 key tiles x 2 blocks x 1024 pairs
    p = n = np.full(128, 128)
    assert bench.computed_pairs(_tiles([64, 64]), p, n) == (16384, 16384)


def test_ragged_history_computes_whole_blocks():
    # 100 H rows seeing 100 keys: slices of 32, 32, 32 and 4 rows, each over 2 key tiles of 2 blocks
    p = n = np.full(100, 100)
    assert bench.computed_pairs(_tiles([64, 36]), p, n) == (4 * 4 * 1024, 100 * 100)


def test_target_rows_add_their_self_term():
    # 64 H rows, then 2 T rows that see the 64 H keys and themselves (p = 64, n = 65)
    p = np.array([64] * 64 + [64, 64])
    n = np.array([64] * 64 + [65, 65])
    # H tile: 2 slices x 2 blocks; T tile: one slice of 2 rows x 2 blocks + 2 self terms
    assert bench.computed_pairs(_tiles([64, 2]), p, n) == (2 * 2048 + 2048 + 2, 64 * 64 + 2 * 65)


def test_causal_rows_in_a_cut_tile():
    # 32 H rows (p = 32) then 32 causal R rows (R row j sees 32 + j + 1 keys).  The H slice runs
    # its only tile unmasked (keys 32..63 load as zeros, one wasted block); the R slice's tile is
    # cut (prefixes 33..64), and each of its two blocks is seen by some row.
    p = n = np.array([32] * 32 + [33 + j for j in range(32)])
    assert bench.computed_pairs(_tiles([64]), p, n) == (2048 + 2048, 32 * 32 + sum(33 + j for j in range(32)))


def test_blocks_no_row_sees_are_skipped():
    # a user whose first row is packed row 40: its key tiles start at the aligned row 0 (the rows
    # before 40 are an earlier user's and load as zeros).  Rows: 24 H (p = 24) then 8 R rows
    # (p = 25..32); one slice of 32 rows, prefixes 24..32, keys [40, 72).
    p = n = np.concatenate([np.zeros(40, int), [24] * 24, [25 + j for j in range(8)]])
    tiles = _tiles([32], urow0=40)
    # kz = 72 -> tiles starting at rows 0 and 64; smallest prefix 24 -> kf = 64 -> tile 0 unmasked
    # (2 blocks), tile 1 cut: lo = 0, lim_hi = 8 -> block 0 seen, block 1 (keys 96..127) skipped
    assert bench.computed_pairs(tiles, p, n) == (3 * 1024, 24 * 24 + sum(25 + j for j in range(8)))
