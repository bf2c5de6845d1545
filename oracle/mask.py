"""Dynamic H/R/T visibility mask, by literal enumeration of the pages' rules.

Row i is the query token, column j the key token; M[i, j] = 1 means i sees j
([blog] §3.2: each row lists what the current token can see).  Rows and
columns of one user are ordered H, R, T ([explainer] §2.1.3, X = (H; R; T)).

Rules ([explainer] §4.1.1 and its worked 7x7 matrix in §8.2; [blog] §3.2;
[digest] paragraph on the dynamic mask), with the readings taken where the
pages leave room:
  * H keys are visible to every query (T queries included, whatever the
    exposure time: H carries no timestamps).
  * H queries see all H keys and nothing else (the §8.2 matrix: H-to-H is all
    ones, H/R-to-T and H-to-R are zero).
  * R queries see all H keys and R keys up to and including themselves by
    position: the standard causal mask of [blog] §3.2 and the lower triangle,
    diagonal included, of the §8.2 matrix.
  * T queries see an R key iff that action's timestamp is strictly earlier
    than the target's exposure time ([blog] §3.2: actions that happened before
    this exposure).
  * T queries see themselves and no other T token ([blog] §3.2; §8.2 diagonal).
    With V2 sub-tokens ([blog] §3.3.2) each sub-token is a T row carrying its
    parent's exposure time; siblings stay invisible to one another.
"""
from __future__ import annotations

import numpy as np

H_TYPE, R_TYPE, T_TYPE = 0, 1, 2


def _kind(i: int, l_h: int, l_r: int) -> int:
    if i < l_h:
        return H_TYPE
    if i < l_h + l_r:
        return R_TYPE
    return T_TYPE


def visible(i: int, j: int, l_h: int, l_r: int, split: int, ts_r, ts_t) -> bool:
    """Does query token i see key token j?  (one user; positions in H, R, T order)"""
    qi, kj = _kind(i, l_h, l_r), _kind(j, l_h, l_r)
    if qi == H_TYPE:
        return kj == H_TYPE
    if qi == R_TYPE:
        if kj == H_TYPE:
            return True
        if kj == R_TYPE:
            return (j - l_h) <= (i - l_h)
        return False
    # T query: its parent target and that target's exposure time
    parent = (i - l_h - l_r) // split
    e_t = int(ts_t[parent])
    if kj == H_TYPE:
        return True
    if kj == R_TYPE:
        return int(ts_r[j - l_h]) < e_t
    return i == j


def dense_mask(l_h: int, l_r: int, l_t: int, split: int, ts_r, ts_t) -> np.ndarray:
    """The user's N x N mask, N = L_H + L_R + split * L_T, by enumerating (i, j)."""
    n = l_h + l_r + split * l_t
    m = np.zeros((n, n), dtype=np.uint8)
    for i in range(n):
        for j in range(n):
            m[i, j] = 1 if visible(i, j, l_h, l_r, split, ts_r, ts_t) else 0
    return m


def dense_mask_fast(l_h, l_r, l_t, split, ts_r, ts_t):
    """The same rules as dense_mask, written with numpy broadcasting.

    Used for users too long for the pure-Python enumeration; the tests check
    that both forms agree element for element.
    """
    n = l_h + l_r + split * l_t
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    lc = l_h + l_r
    qh, qr, qt = i < l_h, (i >= l_h) & (i < lc), i >= lc
    kh, kr, kt = j < l_h, (j >= l_h) & (j < lc), j >= lc
    m = np.zeros((n, n), bool)
    m |= qh & kh
    m |= qr & kh
    m |= qr & kr & (j <= i)
    m |= qt & kh
    if l_r > 0 and l_t > 0:
        ts_r = np.asarray(ts_r, np.int64)
        ts_t = np.asarray(ts_t, np.int64)
        parent = np.clip((np.arange(n) - lc) // split, 0, l_t - 1)
        e = ts_t[parent][:, None]
        tr = ts_r[np.clip(np.arange(n) - l_h, 0, l_r - 1)][None, :]
        m |= qt & kr & (tr < e)
    m |= qt & kt & (i == j)
    return m.astype(np.uint8)



def mask_row(i: int, l_h: int, l_r: int, l_t: int, split: int, ts_r, ts_t) -> np.ndarray:
    """Row i of the user's mask (the keys query token i sees), 0/1 of length N.

    The rules of `visible` for one query against every key at once, for users
    too long to hold the N x N matrix.
    """
    n = l_h + l_r + split * l_t
    lc = l_h + l_r
    row = np.zeros(n, bool)
    kind = _kind(i, l_h, l_r)
    row[:l_h] = True                            # every query sees every H key
    if kind == R_TYPE:
        row[l_h:i + 1] = True                   # R keys up to and including itself
    elif kind == T_TYPE:
        e_t = int(ts_t[(i - lc) // split])      # the parent target's exposure time
        if l_r:
            row[l_h:lc] = np.asarray(ts_r, np.int64) < e_t
        row[i] = True                           # itself, the only T key it sees
    return row.astype(np.uint8)


def row_types(l_h: int, l_r: int, l_t: int, split: int) -> np.ndarray:
    n = l_h + l_r + split * l_t
    return np.array([_kind(i, l_h, l_r) for i in range(n)], dtype=np.uint8)


def row_meta(m: np.ndarray, l_h: int, l_r: int):
    """Per-row metadata of one user's mask, read off the dense matrix.

    p[i]    = 1 + the last visible context column (H or R), 0 if none;
    selfv[i] = 1 for a T row that sees itself (the only T key it can see);
    n[i]    = number of visible keys (the 1/n normaliser).
    Raises if a row's visible context is not exactly the prefix [0, p[i]).
    """
    lc = l_h + l_r
    rows = m.shape[0]
    p = np.zeros(rows, np.int32)
    selfv = np.zeros(rows, np.int32)
    for i in range(rows):
        vis = np.nonzero(m[i, :lc])[0]
        p[i] = (vis.max() + 1) if vis.size else 0
        if not np.array_equal(m[i, :p[i]], np.ones(p[i], np.uint8)):
            raise AssertionError(f"row {i}: visible context is not a prefix")
        if i >= lc:
            tvis = np.nonzero(m[i, lc:])[0] + lc
            if not (tvis.size == 0 or (tvis.size == 1 and tvis[0] == i)):
                raise AssertionError(f"row {i}: a T row sees another T row")
            selfv[i] = int(m[i, i])
    n = m.sum(axis=1).astype(np.int32)
    return p, selfv, n


def tile_classes(m: np.ndarray, row_begin: int, l_ctx: int, bm: int, bn: int) -> np.ndarray:
    """Brute-force class of every (query tile, key tile) block of one user's mask.

    Query tiles cover rows [row_begin, N) in steps of bm (the last may be short);
    key tiles cover the context columns [0, l_ctx) in steps of bn.  Only
    in-range elements count.  Classes: 0 = all zero (skip), 2 = all one (full),
    1 = mixed (partial).  T columns are not tiled: a T row's only T key is
    itself, carried by the self flag.
    """
    rows = m.shape[0]
    nq = -(-(rows - row_begin) // bm) if rows > row_begin else 0
    nk = -(-l_ctx // bn) if l_ctx > 0 else 0
    out = np.zeros((nq, nk), np.int8)
    for a in range(nq):
        r0, r1 = row_begin + a * bm, min(row_begin + (a + 1) * bm, rows)
        for b in range(nk):
            c0, c1 = b * bn, min((b + 1) * bn, l_ctx)
            blk = m[r0:r1, c0:c1]
            out[a, b] = 0 if blk.sum() == 0 else (2 if blk.all() else 1)
    return out


def tile_desc_from_classes(cls: np.ndarray):
    """(leading full tiles, 1 + last non-skip tile) per query tile.

    Raises unless every row of classes reads full*, partial*, skip*, which is
    what per-row visible prefixes imply.
    """
    out = []
    for row in cls:
        nfull = 0
        while nfull < len(row) and row[nfull] == 2:
            nfull += 1
        nz = np.nonzero(row)[0]
        end = int(nz.max() + 1) if nz.size else 0
        if not (np.all(row[nfull:end] == 1) and np.all(row[end:] == 0)):
            raise AssertionError(f"tile row {row} is not full*, partial*, skip*")
        out.append((nfull, end))
    return np.array(out, dtype=np.int32).reshape(-1, 2)


def batch_meta(batch, bm: int = 64, bn: int = 64, fast: bool = False):
    """Mask metadata of a whole jagged batch, user by user.

    ``fast`` builds each mask with the broadcast form (checked equal to the
    enumeration by the tests) for users too long for Python loops.
    Returns a dict with per-row p, self, n, row_type (over all packed rows),
    and the full-layer and target-layer tile tables, each row
    (user, first row within the user, rows in tile, leading full key tiles,
    key-tile end), users in order and tiles in order within a user.
    """
    ps, ss, ns, ts = [], [], [], []
    full_tiles, tgt_tiles = [], []
    ro, to = batch.r_off, batch.t_off
    for u in range(batch.n_users):
        l_h, l_r, l_t = (int(v) for v in batch.lens[u])
        ts_r = batch.ts_r[ro[u]:ro[u + 1]]
        ts_t = batch.ts_t[to[u]:to[u + 1]]
        m = (dense_mask_fast if fast else dense_mask)(l_h, l_r, l_t, batch.split, ts_r, ts_t)
        p, selfv, n = row_meta(m, l_h, l_r)
        ps.append(p); ss.append(selfv); ns.append(n)
        ts.append(row_types(l_h, l_r, l_t, batch.split))
        lc, rows = l_h + l_r, m.shape[0]
        for begin, table in ((0, full_tiles), (lc, tgt_tiles)):
            cls = tile_classes(m, begin, lc, bm, bn)
            desc = tile_desc_from_classes(cls)
            for a in range(cls.shape[0]):
                r0 = begin + a * bm
                table.append((u, r0, min(bm, rows - r0), desc[a, 0], desc[a, 1]))
    cat = lambda xs, dt: np.concatenate(xs).astype(dt) if xs else np.zeros(0, dt)
    return {"p": cat(ps, np.int32), "self": cat(ss, np.int32), "n": cat(ns, np.int32),
            "row_type": cat(ts, np.uint8),
            "full_tiles": np.array(full_tiles, np.int32).reshape(-1, 5),
            "target_tiles": np.array(tgt_tiles, np.int32).reshape(-1, 5)}
