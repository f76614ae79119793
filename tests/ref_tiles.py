"""Reference tile lists of one head, vectorised over all queries.

The definition is the oracle's (token voting with threshold one): key tile Kb
is listed for query tile Qa iff some query i in Qa retains some key j in Kb.
`oracle.query_tile_row` walks it one query at a time, which takes seconds per
hundred tiles at the video shapes; this module evaluates the same definition
for every query at once, so that full-size plans can be compared row by row.
It is a test helper, pinned against `oracle.csr` on random small grids in
tests/test_ref_tiles.py, and shares nothing with the HIP library.

For the disk (L2) and Manhattan (L1) masks, a query (t, h, w) retains in frame
tk (|tk - t| = delta active) the keys of row h + dh whose columns lie within
the half-width of that row: isqrt(R2 - dh^2) for the disk, R - |dh| for L1.
Each such (query, frame, row) interval covers a run of key-tile columns.  For
the 1-D window, the retained keys form the raster interval [n - rho, n + rho],
which is cut into one column interval per key row it touches.  The runs are
accumulated in a difference array over key-tile columns per (query tile, key
tile row).
"""
import numpy as np

import oracle as O


def _isqrt(x):
    """Exact integer square root of a non-negative int64 array."""
    r = np.floor(np.sqrt(x.astype(np.float64))).astype(np.int64)
    r -= (r * r > x)
    r += ((r + 1) * (r + 1) <= x)
    return r


def _table_rows(lv, R2, p, N):
    if p["radius_override"] >= 0:
        return np.broadcast_to(R2[0], (N, R2.shape[1]))
    return R2[np.asarray(lv, dtype=np.int64) - O.level_range(p)[0]]


def tile_hits(lv, R2, T, H, W, p, th=8, tw=8):
    """Boolean [n_qtiles, n_ktiles]: True where the key tile is listed."""
    N = T * H * W
    n = np.arange(N, dtype=np.int64)
    t, h, w = n // (H * W), (n // W) % H, n % W
    nh, nw = -(-H // th), -(-W // tw)
    nq = T * nh * nw
    nkr = T * nh  # key tile rows (frame, tile row)
    qt = (t * nh + h // th) * nw + w // tw
    rows = _table_rows(lv, R2, p, N)
    size = nq * nkr * (nw + 1)
    diff = np.zeros(size, dtype=np.int64)

    starts, ends = [], []

    def add(sel, qtile, tk, hk, c_lo, c_hi):
        """Mark key columns c_lo..c_hi (inclusive, token columns) of row hk of
        frame tk for the selected queries."""
        if not np.any(sel):
            return
        qtile, tk, hk, c_lo, c_hi = qtile[sel], tk[sel], hk[sel], c_lo[sel], c_hi[sel]
        base = (qtile * nkr + tk * nh + hk // th) * (nw + 1)
        starts.append(base + c_lo // tw)
        ends.append(base + c_hi // tw + 1)

    def flush():
        nonlocal diff
        if starts:
            diff += np.bincount(np.concatenate(starts), minlength=size)
            diff -= np.bincount(np.concatenate(ends), minlength=size)
        starts.clear()
        ends.clear()

    gen = p.get("generator", 0)
    if gen == O.GEN_WINDOW_1D:
        rho = rows[:, 0].astype(np.int64)
        lo = np.maximum(0, n - rho)
        hi = np.minimum(N - 1, n + rho)
        r_lo, r_hi = lo // W, hi // W
        for step in range(int((r_hi - r_lo).max()) + 1):
            r = r_lo + step
            sel = r <= r_hi
            c_lo = np.maximum(lo - r * W, 0)
            c_hi = np.minimum(hi - r * W, W - 1)
            add(sel, qt, r // H, r % H, c_lo, c_hi)
            if step % 16 == 15:
                flush()
    else:
        l1 = gen == O.GEN_MANHATTAN
        for delta in range(T):
            lim = rows[:, delta].astype(np.int64)
            act = lim >= 0
            if not np.any(act):
                continue
            reach = np.where(act, lim if l1 else _isqrt(np.maximum(lim, 0)), -1)
            rmax = int(reach.max())
            for sign in ((1,) if delta == 0 else (1, -1)):
                tk = t + sign * delta
                ok_t = act & (tk >= 0) & (tk < T)
                for dh in range(-rmax, rmax + 1):
                    hk = h + dh
                    if l1:
                        half = lim - abs(dh)
                    else:
                        rem = lim - dh * dh
                        half = np.where(rem >= 0, _isqrt(np.maximum(rem, 0)), -1)
                    sel = ok_t & (hk >= 0) & (hk < H) & (half >= 0)
                    add(sel, qt, np.clip(tk, 0, T - 1), np.clip(hk, 0, H - 1),
                        np.maximum(0, w - half), np.minimum(W - 1, w + half))
                flush()
    flush()
    runs = np.cumsum(diff.reshape(nq, nkr, nw + 1), axis=2)[:, :, :nw] > 0
    return runs.reshape(nq, nkr * nw)


def csr(lv, R2, T, H, W, p, th=8, tw=8):
    """(row_ptr, col_idx) of one head, rows in query-tile order, columns ascending."""
    hits = tile_hits(lv, R2, T, H, W, p, th, tw)
    counts = hits.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    col_idx = np.nonzero(hits)[1].astype(np.int64)
    return row_ptr, col_idx


def edge_queries(T, H, W, rng, th=8, tw=8):
    """One random query of every tile on the border of every frame (first and
    last tile row and tile column, ragged ones included)."""
    nh, nw = -(-H // th), -(-W // tw)
    out = []
    for t in range(T):
        for r in range(nh):
            for c in range(nw):
                if r in (0, nh - 1) or c in (0, nw - 1):
                    h0, w0 = r * th, c * tw
                    hh = h0 + int(rng.integers(min(th, H - h0)))
                    ww = w0 + int(rng.integers(min(tw, W - w0)))
                    out.append((t * H + hh) * W + ww)
    return np.array(out, dtype=np.int64)


def query_sample(T, H, W, n_total, rng):
    """At least `n_total` distinct queries: every frame-border tile once, the
    grid's first and last token, and random queries for the rest."""
    N = T * H * W
    base = np.concatenate([edge_queries(T, H, W, rng), [0, N - 1]])
    base = np.unique(base)
    extra = max(0, n_total - len(base))
    rest = np.setdiff1d(np.arange(N), base)
    pick = rng.choice(rest, size=min(extra, len(rest)), replace=False) if extra else np.zeros(0, np.int64)
    return np.sort(np.concatenate([base, pick]).astype(np.int64))
