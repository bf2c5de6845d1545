"""Expected attention work order, rebuilt in Python from its rule.

The attention grids take their 32-row query slices in an order that balances
the GPU's 8 XCDs: users ranked by estimated work (largest first, ties by
index), dealt to the XCDs in a boustrophedon 0..7, 7..0, ..., every XCD's
users in rank order and each user's slices last first.  Entry 8 k + x of the
order is the slice id (2 tile + half) that XCD x takes k-th, -1 past the end
of its list; the array holds 8 x the longest list.  Batches of more than 2048
users have no order (the kernels keep the XCD-contiguous one), nor have those
whose dealing would give some XCD more than 1.25 x the mean work (a few users,
or one far longer than the rest: that user's slices would all sit on one XCD).

This is scheduling, not the method's arithmetic: any order that lists every
non-empty slice once gives the same attention output, which the parity tests
check.  These helpers pin what the library builds against the rule.
"""
import numpy as np

MAX_USERS = 2048
FULL, TARGET = 0, 1


def slices(lens, split, layer):
    lens = np.asarray(lens, np.int64)
    rows = split * lens[:, 2] + (lens[:, 0] + lens[:, 1] if layer == FULL else 0)
    return (rows + 31) // 32


def user_work(lens, split, layer):
    """Key tiles each slice can visit (a bound from the lengths) plus one, summed per user."""
    out = []
    for lh, lr, lt in np.asarray(lens, np.int64):
        ctx = lh + lr
        if layer == TARGET:
            out.append(((split * lt + 31) // 32) * ((ctx + 63) // 64 + 1))
            continue
        rows = ctx + split * lt
        w = 0
        for k in range((rows + 31) // 32):
            last = min(32 * k + 32, rows) - 1
            vis = lh if last < lh else (last + 1 if last < ctx else ctx)   # visible keys of the slice's last row
            w += (vis + 63) // 64 + 1
        out.append(w)
    return np.asarray(out, np.int64)


def xcd_of_rank(r):
    return 7 - r % 8 if (r // 8) % 2 else r % 8


def xcd_loads(lens, split, layer):
    """Work the dealing gives each XCD."""
    lens = np.asarray(lens, np.int64).reshape(-1, 3)
    work = user_work(lens, split, layer)
    loads = np.zeros(8, np.int64)
    for r, u in enumerate(sorted(range(len(lens)), key=lambda u: (-work[u], u))):
        loads[xcd_of_rank(r)] += work[u]
    return loads


def balanced(lens, split, layer):
    loads = xcd_loads(lens, split, layer)
    return 4 * 8 * int(loads.max()) <= 5 * int(loads.sum())


def expected_order(lens, split, layer):
    lens = np.asarray(lens, np.int64).reshape(-1, 3)
    n = len(lens)
    if n == 0 or n > MAX_USERS or not balanced(lens, split, layer):
        return np.zeros(0, np.int32)
    work = user_work(lens, split, layer)
    ns = slices(lens, split, layer)
    tiles = (ns + 1) // 2                                   # 64-row query tiles of each user
    first = np.concatenate([[0], np.cumsum(tiles)[:-1]])
    ranked = sorted(range(n), key=lambda u: (-work[u], u))
    lists = [[] for _ in range(8)]
    for r, u in enumerate(ranked):
        lists[xcd_of_rank(r)].extend(2 * first[u] + k for k in reversed(range(ns[u])))
    m = max(len(x) for x in lists)
    out = np.full(8 * m, -1, np.int32)
    for x, lst in enumerate(lists):
        out[x:8 * len(lst):8] = lst
    return out
