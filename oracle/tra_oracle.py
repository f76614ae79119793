"""Plain, slow fp64 reference of the Token Radius Attention (TRA) hot path.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Shares no code with the
HIP library; its only common dependency is the seeded input generator.

Sources.  The method is described by the page "Token Radius Attention for
Efficient Video Generation" (a French summary, section 2 "Méthodologie":
Intuition I, Intuition II and "Le Pipeline TRA") and by its English TL;DR page.
The pages fix the shape of the method but no constants and no closed form for
the radius; every step below states the reading it takes.  The generic
fixed-radius blog post ("Token Radius Attention视频生成里被忽略但值得关注的高效
注意力思路", sections 4.1, 5.1-5.2 and 9) is used for the attention scale, the
token order and "mask with -inf before softmax".

Steps (all in fp64 unless stated):
  1  geometry      token n = (t*H + h)*W + w; pool blocks and tiles are
                   rectangles inside one frame, ragged at the bottom/right edge.
  2  pool_keys     Kbar_b = round_once_to_input_dtype(mean_{j in b} k_j).
  3  entropy       z_ib = q_i.Kbar_b/sqrt(d);
                   H_i = ln sum_b |b| e^{z_ib} - sum_b |b| e^{z_ib} z_ib / sum_b |b| e^{z_ib}
                   (entropy of the softmax over all N keys with every key
                   replaced by its pooled key).
  4  levels        k_i = clamp(floor(q_lv*(a*H_i + c)), k_lo, k_hi)
                   (log-linear budget ln B = a*H + c; Intuition I's analytic
                   map B ~ tau*exp(H) with a = 1, c = ln tau).
  5  radius table  S = sum_{delta=-(T-1)}^{T-1} phi^(2|delta|); r0^2 = e^{k/q_lv}/(pi*S);
                   R2[k][delta] = floor(r0^2 * phi^(2 delta)); frame delta >= 1 is
                   active iff R2 >= 1 (inactive entries are stored as -1).
                   (Intuition II: budget -> radius, phi(delta) = exp(-gamma*delta).)
  6  mask          retained(i,j) iff R2[k_i][|t_i-t_j|] >= 0 and
                   (h_i-h_j)^2 + (w_i-w_j)^2 <= R2[k_i][|t_i-t_j|].
  7  CSR           key tile Kb is listed for query tile Qa iff some (i in Qa,
                   j in Kb) is retained ("token voting" with threshold one).
  8  output        O_i = sum_{j retained} softmax_j(q_i.k_j/sqrt(d)) v_j.
"""
import math
from fractions import Fraction

import numpy as np

__all__ = [
    "Geometry", "pool_keys", "entropy", "explicit_softmax_entropy", "level_range", "levels",
    "frame_sum", "radius_table", "table_margin", "retained_keys", "retained_count",
    "retained_counts", "dense_mask", "query_tile_row", "csr", "attention_rows",
    "dense_attention", "dense_entropy", "excused_queries", "round_to_dtype", "plan", "ENTROPY_EXCUSE",
    "GEN_ENTROPY_DISK", "GEN_MANHATTAN", "GEN_RADIAL", "GEN_WINDOW_1D", "radial_band", "tile_votes", "csr_vote",
    "listed_keys", "attention_rows_listed",
]

ENTROPY_EXCUSE = 1e-5  # queries this close (nats) to a level boundary may differ


# ----------------------------------------------------------------------------
# Step 1: geometry
# ----------------------------------------------------------------------------
class Geometry:
    """Partition of each T x H x W frame stack into bh x bw rectangles.

    Rectangle id = (t*nbh + h//bh)*nbw + w//bw; the last row/column of
    rectangles in a frame is ragged when bh (bw) does not divide H (W).
    """

    def __init__(self, T, H, W, bh, bw):
        self.T, self.H, self.W, self.bh, self.bw = T, H, W, bh, bw
        self.nbh = -(-H // bh)
        self.nbw = -(-W // bw)
        self.per_frame = self.nbh * self.nbw
        self.count = T * self.per_frame

    def coords(self):
        n = np.arange(self.T * self.H * self.W)
        return n // (self.H * self.W), (n // self.W) % self.H, n % self.W

    def block_of_tokens(self):
        t, h, w = self.coords()
        return (t * self.nbh + h // self.bh) * self.nbw + w // self.bw

    def block_sizes(self):
        rows = np.minimum(self.bh, self.H - np.arange(self.nbh) * self.bh)
        cols = np.minimum(self.bw, self.W - np.arange(self.nbw) * self.bw)
        per_frame = (rows[:, None] * cols[None, :]).reshape(-1)
        return np.tile(per_frame, self.T)

    def rect(self, b):
        """(t, h0, h1, w0, w1) with half-open row/column ranges of rectangle b."""
        t, rem = divmod(int(b), self.per_frame)
        r, c = divmod(rem, self.nbw)
        return t, r * self.bh, min(self.H, (r + 1) * self.bh), c * self.bw, min(self.W, (c + 1) * self.bw)

    def tokens(self, b):
        t, h0, h1, w0, w1 = self.rect(b)
        hh, ww = np.meshgrid(np.arange(h0, h1), np.arange(w0, w1), indexing="ij")
        return ((t * self.H + hh) * self.W + ww).reshape(-1)


# ----------------------------------------------------------------------------
# Step 2: pooled keys, rounded once to the input dtype
# ----------------------------------------------------------------------------
_SIGBITS = {"bf16": 8, "fp32": 24}


def _lowest_bit_exponent(x):
    """Exponent of the lowest set bit of each nonzero float64 (huge for zeros)."""
    m, e = np.frexp(np.abs(x))
    ints = np.ldexp(m, 53).astype(np.int64)  # exact: 53-bit significand as an integer
    low = ints & -ints
    tz = np.where(ints > 0, np.log2(np.maximum(low, 1)).round().astype(np.int64), 0)
    return np.where(x != 0, e - 53 + tz, np.iinfo(np.int64).max // 4)


def round_to_dtype(num, den, dtype):
    """Round the exact rational num/den (num: exact float64 array, den: positive
    ints) to the nearest value of `dtype` (round half to even), in one step.

    The float64 quotient q = num/den is correctly rounded.  Rounding q instead of
    the rational can only go wrong when q lands exactly on a midpoint between two
    dtype values (a representable float64); those entries are re-decided in
    exact rational arithmetic.
    """
    num = np.asarray(num, dtype=np.float64)
    den = np.broadcast_to(np.asarray(den, dtype=np.float64), num.shape)
    sb = _SIGBITS[dtype]
    q = num / den
    a = np.abs(q)
    m, e = np.frexp(a)
    scaled = np.ldexp(m, sb)  # in [2^(sb-1), 2^sb): exact scaling by a power of two
    lo = np.floor(scaled)
    frac = scaled - lo
    up = (frac > 0.5) | ((frac == 0.5) & (np.fmod(lo, 2) == 1))
    res = np.ldexp(lo + up, e - sb)
    mid = np.argwhere((frac == 0.5) & (a != 0))
    for idx in map(tuple, mid):
        exact = abs(Fraction(float(num[idx])) / Fraction(int(den[idx])))
        midpoint = Fraction(float(lo[idx]) + 0.5) * Fraction(2) ** int(e[idx] - sb)
        if exact > midpoint:
            res[idx] = math.ldexp(lo[idx] + 1, int(e[idx] - sb))
        elif exact < midpoint:
            res[idx] = math.ldexp(lo[idx], int(e[idx] - sb))
    if dtype == "bf16":
        assert np.all((a == 0) | (a >= 2.0 ** -126)), "bf16 subnormal mean: outside the oracle's domain"
    return np.copysign(res, q)


def pool_keys(k, geom: Geometry, dtype):
    """Mean of the keys of each pool block, rounded once to the input dtype.

    k: [N, d] float64 holding the input values exactly.  The per-block sum is
    exact: it is taken in float64 only where every partial sum is provably an
    integer multiple of 2^L below 2^(L+53) (L = lowest set bit over the block),
    and with math.fsum otherwise.  Returns [n_blocks, d] float64 (dtype values).
    """
    k = np.asarray(k, dtype=np.float64)
    blk = geom.block_of_tokens()
    order = np.argsort(blk, kind="stable")
    sizes = geom.block_sizes()
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    ks = k[order]
    sums = np.add.reduceat(ks, starts, axis=0)
    abssum = np.add.reduceat(np.abs(ks), starts, axis=0)
    low = np.minimum.reduceat(_lowest_bit_exponent(ks), starts, axis=0)
    exact = abssum < np.ldexp(1.0, np.clip(low + 53, -1000, 1000).astype(np.int64))
    for b, dim in np.argwhere(~exact):
        sums[b, dim] = math.fsum(ks[starts[b]:starts[b] + sizes[b], dim])
    return round_to_dtype(sums, sizes[:, None], dtype)


# ----------------------------------------------------------------------------
# Step 3: per-query entropy over pooled keys
# ----------------------------------------------------------------------------
def entropy(q, kbar, sizes):
    """H_i of softmax over all keys with each key replaced by its pool block mean.

    q: [n, d], kbar: [nb, d], sizes: [nb] block sizes |b|.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    z = (q @ np.asarray(kbar, dtype=np.float64).T) / math.sqrt(d)
    m = z.max(axis=1, keepdims=True)
    w = sizes[None, :] * np.exp(z - m)
    A = w.sum(axis=1)
    return np.log(A) + m[:, 0] - (w * z).sum(axis=1) / A


def explicit_softmax_entropy(q, kbar, geom: Geometry):
    """Shannon entropy -sum_j p_j ln p_j of the length-N softmax of q against the
    block-replaced keys (an independent computation used to pin `entropy`)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(kbar, dtype=np.float64)[geom.block_of_tokens()]
    s = (q @ keys.T) / math.sqrt(q.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(p > 0, -p * np.log(p), 0.0)
    return terms.sum(axis=1)


# ----------------------------------------------------------------------------
# Step 4: budget levels
# ----------------------------------------------------------------------------
def level_range(p):
    """(k_lo, k_hi): the budget clamp [B_min, B_max] expressed as level indices."""
    q = p["levels_per_nat"]
    k_lo = math.ceil(q * math.log(p["budget_min"]))
    k_hi = math.floor(q * math.log(p["budget_max"]))
    assert k_lo <= k_hi, "empty budget range"
    return k_lo, k_hi


def levels(H, p):
    """k_i = clamp(floor(q_lv*(a*H_i + c)), k_lo, k_hi); -1 for every query when a
    fixed radius overrides the entropy budget."""
    H = np.asarray(H, dtype=np.float64)
    if p["radius_override"] >= 0:
        return np.full(H.shape, -1, dtype=np.int64)
    k_lo, k_hi = level_range(p)
    k = np.floor(p["levels_per_nat"] * (p["a"] * H + p["c"])).astype(np.int64)
    return np.clip(k, k_lo, k_hi)


def excused_queries(H, p, tol=ENTROPY_EXCUSE):
    """Indices of queries whose entropy lies within `tol` of a level boundary that
    can change the clamped level (boundaries k/q_lv for k_lo < k <= k_hi)."""
    if p["radius_override"] >= 0:
        return np.zeros(0, dtype=np.int64)
    k_lo, k_hi = level_range(p)
    if k_hi <= k_lo:
        return np.zeros(0, dtype=np.int64)  # a single level: no boundary changes it
    H = np.asarray(H, dtype=np.float64)
    L = p["levels_per_nat"] * (p["a"] * H + p["c"])
    nearest = np.clip(np.round(L), k_lo + 1, k_hi)
    Hb = (nearest / p["levels_per_nat"] - p["c"]) / p["a"]
    return np.nonzero(np.abs(H - Hb) < tol)[0]


# ----------------------------------------------------------------------------
# Step 5: radius table
# ----------------------------------------------------------------------------
def frame_sum(decay, T):
    """S = sum over delta in [-(T-1), T-1] of decay^(2|delta|)."""
    return sum(decay ** (2 * abs(dl)) for dl in range(-(T - 1), T))


GEN_ENTROPY_DISK, GEN_MANHATTAN, GEN_RADIAL, GEN_WINDOW_1D = 0, 1, 2, 3


def _generator(p):
    return p.get("generator", GEN_ENTROPY_DISK)


def _l1(p):
    """True when the mask measures distance with the L1 norm (Manhattan)."""
    return _generator(p) == GEN_MANHATTAN


def _window(p):
    """True for the 1-D ablation: distance along the raster token order."""
    return _generator(p) == GEN_WINDOW_1D


def radial_band(delta):
    """Octave band of a frame distance: 0 for delta = 0, then 1, 2, 2, 3, 3, 3,
    3, 4, ... (band b >= 1 holds the 2^(b-1) distances 2^(b-1) .. 2^b - 1)."""
    return 0 if delta == 0 else delta.bit_length()


def _r0_squared(p, T):
    if p["radius_override"] >= 0:
        return [p["radius_override"] ** 2]
    k_lo, k_hi = level_range(p)
    S = frame_sum(p["decay"], T)
    return [math.exp(k / p["levels_per_nat"]) / (math.pi * S) for k in range(k_lo, k_hi + 1)]


def radius_table(p, T):
    """int64 [n_levels, T]: R2[k - k_lo][delta], -1 where frame delta is inactive.

    Row 0 is the only row when a fixed radius override is set (level -1).
    Alternative generators (static, radius r = radius_override):
      Manhattan  the L1 ball |dt| + |dh| + |dw| <= r of the fixed-radius post
                 (section 5.2): frame delta holds the 2D L1 disk of radius
                 floor(r) - delta, inactive below 0 (the entry is an L1 radius);
      Radial     the static mask whose spatial window shrinks with temporal
                 distance: in octave band b (radial_band) the disk area halves
                 per band, R2 = floor(r^2 / 2^b), active while R2 >= 1."""
    if _generator(p) == GEN_MANHATTAN:
        assert p["radius_override"] >= 0, "the Manhattan generator needs a fixed radius"
        R = math.floor(p["radius_override"])
        return np.array([[R - dl if R - dl >= 0 else -1 for dl in range(T)]], dtype=np.int64)
    if _window(p):
        # 1-D ablation ([TRA] section 4: the radius mask replaced by a 1-D
        # distance): query i keeps the keys j with |n_i - n_j| <= rho along the
        # raster order, rho = floor((B - 1)/2) so that the window of 2 rho + 1
        # tokens holds the quantised budget B (or floor(radius_override) when
        # set).  The same rho stands in every column (frame distances play no
        # part of their own).
        if p["radius_override"] >= 0:
            rhos = [math.floor(p["radius_override"])]
        else:
            k_lo, k_hi = level_range(p)
            rhos = [math.floor((math.exp(k / p["levels_per_nat"]) - 1.0) / 2.0) for k in range(k_lo, k_hi + 1)]
        return np.array([[r] * T for r in rhos], dtype=np.int64)
    if _generator(p) == GEN_RADIAL:
        assert p["radius_override"] >= 0, "the Radial generator needs a fixed radius"
        r0sq = p["radius_override"] ** 2
        row = []
        for delta in range(T):
            v = math.floor(r0sq / 2 ** radial_band(delta))
            row.append(v if (delta == 0 or v >= 1) else -1)
        return np.array([row], dtype=np.int64)
    rows = []
    for r0sq in _r0_squared(p, T):
        row = []
        for delta in range(T):
            v = math.floor(r0sq * p["decay"] ** (2 * delta))
            row.append(v if (delta == 0 or v >= 1) else -1)
        rows.append(row)
    return np.array(rows, dtype=np.int64)


def table_margin(p, T):
    """Smallest relative distance of an unrounded table entry to an integer that
    the floor could fall on (an ambiguity check: floors of values this close to
    an integer could legitimately differ between two float64 evaluations)."""
    worst = math.inf
    for r0sq in _r0_squared(p, T):
        for delta in range(T):
            x = r0sq * p["decay"] ** (2 * delta)
            if x >= 0.5 and x != round(x):
                worst = min(worst, abs(x - round(x)) / x)
    return worst


# ----------------------------------------------------------------------------
# Step 6: the per-token radius mask
# ----------------------------------------------------------------------------
def _row(level, R2, p):
    return R2[0] if p["radius_override"] >= 0 else R2[level - level_range(p)[0]]


def _reach(lim, p):
    """Largest |h_i - h_j| with a retained key in a frame whose entry is lim >= 0."""
    return lim if _l1(p) else math.isqrt(lim)


def _half_width(lim, dh, p):
    """Half-width of the retained columns at row offset dh (-1: none)."""
    if _l1(p):
        return lim - abs(dh) if lim - abs(dh) >= 0 else -1
    rem = lim - dh * dh
    return math.isqrt(rem) if rem >= 0 else -1


def retained_keys(i, level, R2, T, H, W, p):
    """Sorted key indices retained by query i (disk enumeration per frame)."""
    t, h, w = i // (H * W), (i // W) % H, i % W
    r2row = _row(level, R2, p)
    if _window(p):
        rho = int(r2row[0])
        return np.arange(max(0, i - rho), min(T * H * W - 1, i + rho) + 1, dtype=np.int64)
    out = []
    for tk in range(T):
        lim = r2row[abs(tk - t)]
        if lim < 0:
            continue
        for hk in range(H):
            a = _half_width(lim, hk - h, p)
            if a < 0:
                continue
            for wk in range(max(0, w - a), min(W - 1, w + a) + 1):
                out.append((tk * H + hk) * W + wk)
    return np.array(out, dtype=np.int64)


def retained_count(i, level, R2, T, H, W, p):
    t, h, w = i // (H * W), (i // W) % H, i % W
    r2row = _row(level, R2, p)
    if _window(p):
        rho = int(r2row[0])
        return min(T * H * W - 1, i + rho) - max(0, i - rho) + 1
    n = 0
    for tk in range(T):
        lim = r2row[abs(tk - t)]
        if lim < 0:
            continue
        reach = _reach(lim, p)
        for hk in range(max(0, h - reach), min(H - 1, h + reach) + 1):
            a = _half_width(lim, hk - h, p)
            n += min(W - 1, w + a) - max(0, w - a) + 1
    return n


def retained_counts(lv, R2, T, H, W, p):
    """Vectorised retained-key count of every query (same definition as
    `retained_count`, used for densities at full size)."""
    N = T * H * W
    n = np.arange(N)
    t, h, w = n // (H * W), (n // W) % H, n % W
    rows = R2[np.zeros(N, dtype=np.int64)] if p["radius_override"] >= 0 else R2[lv - level_range(p)[0]]
    if _window(p):
        rho = rows[:, 0]
        return np.minimum(N - 1, n + rho) - np.maximum(0, n - rho) + 1
    total = np.zeros(N, dtype=np.int64)
    for tk in range(T):
        lim = rows[np.arange(N), np.abs(tk - t)]
        for hk in range(H):
            if _l1(p):
                a = lim - np.abs(hk - h)
                ok = a >= 0
            else:
                rem = lim - (hk - h) ** 2
                ok = rem >= 0
                a = np.floor(np.sqrt(np.maximum(rem, 0))).astype(np.int64)
                a -= (a * a > rem)  # exact integer square root
                a += ((a + 1) * (a + 1) <= rem)
            cnt = np.minimum(W - 1, w + a) - np.maximum(0, w - a) + 1
            total += np.where(ok, cnt, 0)
    return total


def dense_mask(lv, R2, T, H, W, p):
    """N x N boolean mask by brute force over every (query, key) pair."""
    N = T * H * W
    n = np.arange(N)
    t, h, w = n // (H * W), (n // W) % H, n % W
    rows = R2[np.zeros(N, dtype=np.int64)] if p["radius_override"] >= 0 else R2[lv - level_range(p)[0]]
    dt = np.abs(t[:, None] - t[None, :])
    lim = np.take_along_axis(rows, dt, axis=1)
    if _window(p):
        return np.abs(n[:, None] - n[None, :]) <= rows[:, :1]
    if _l1(p):
        d = np.abs(h[:, None] - h[None, :]) + np.abs(w[:, None] - w[None, :])
    else:
        d = (h[:, None] - h[None, :]) ** 2 + (w[:, None] - w[None, :]) ** 2
    return (lim >= 0) & (d <= lim)


# ----------------------------------------------------------------------------
# Step 7: block-sparse structure
# ----------------------------------------------------------------------------
def query_tile_row(a, lv, R2, tiles: Geometry, p):
    """Sorted key tile ids listed for query tile a (any retained pair votes)."""
    T, H, W = tiles.T, tiles.H, tiles.W
    hit = set()
    if _window(p):
        key_tile = tiles.block_of_tokens()
        for i in tiles.tokens(a):
            hit.update(np.unique(key_tile[retained_keys(int(i), int(lv[i]), R2, T, H, W, p)]).tolist())
        return np.array(sorted(hit), dtype=np.int64)
    for i in tiles.tokens(a):
        t, h, w = i // (H * W), (i // W) % H, i % W
        r2row = _row(lv[i], R2, p)
        for tk in range(T):
            lim = r2row[abs(tk - t)]
            if lim < 0:
                continue
            reach = _reach(lim, p)
            for hk in range(max(0, h - reach), min(H - 1, h + reach) + 1):
                half = _half_width(lim, hk - h, p)
                c0 = max(0, w - half) // tiles.bw
                c1 = min(W - 1, w + half) // tiles.bw
                base = (tk * tiles.nbh + hk // tiles.bh) * tiles.nbw
                hit.update(range(base + c0, base + c1 + 1))
    return np.array(sorted(hit), dtype=np.int64)


def csr(lv, R2, tiles: Geometry, p):
    """(row_ptr, col_idx) over all query tiles of one head, rows in tile-id order."""
    rows = [query_tile_row(a, lv, R2, tiles, p) for a in range(tiles.count)]
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64)
    col_idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return row_ptr, col_idx


# ----------------------------------------------------------------------------
# Token voting with a threshold; block-only masks
# ----------------------------------------------------------------------------
def tile_votes(a, lv, R2, tiles: Geometry, p):
    """{key tile id: number of retained pairs (i, j) with i in query tile a and j
    in that key tile}: the votes of [TRA]'s token voting (section 2, "Exécution
    Efficace"), which turns token masks into block masks."""
    key_tile = tiles.block_of_tokens()
    votes = {}
    for i in tiles.tokens(a):
        keys = retained_keys(int(i), int(lv[i]), R2, tiles.T, tiles.H, tiles.W, p)
        for b, n in zip(*np.unique(key_tile[keys], return_counts=True)):
            votes[int(b)] = votes.get(int(b), 0) + int(n)
    return votes


def csr_vote(lv, R2, tiles: Geometry, p, theta):
    """(row_ptr, col_idx): key tile b is listed for query tile a iff it holds at
    least `theta` votes (theta = 1 gives `csr`)."""
    rows = []
    for a in range(tiles.count):
        votes = tile_votes(a, lv, R2, tiles, p)
        rows.append(np.array(sorted(b for b, n in votes.items() if n >= theta), dtype=np.int64))
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64)
    col_idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return row_ptr, col_idx


def listed_keys(i, tiles: Geometry, row_ptr, col_idx):
    """Sorted key indices of every tile listed for query i's tile."""
    a = int(tiles.block_of_tokens()[i])
    toks = [tiles.tokens(b) for b in col_idx[row_ptr[a]:row_ptr[a + 1]]]
    return np.sort(np.concatenate(toks)) if toks else np.zeros(0, dtype=np.int64)


def attention_rows_listed(q, k, v, rows, lv, R2, tiles: Geometry, p, row_ptr, col_idx, block_only):
    """O_i over the keys of the tiles listed for i's tile: all of them (block-only
    mask, the block-sparse execution of the pages) or only those i retains
    (exact mask restricted to the listed tiles).  A query left with no key (its
    tiles all fell below the vote threshold) gets O_i = 0."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    out = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    for slot, i in enumerate(rows):
        keys = listed_keys(int(i), tiles, row_ptr, col_idx)
        if not block_only:
            keys = np.intersect1d(keys, retained_keys(int(i), int(lv[i]), R2, tiles.T, tiles.H, tiles.W, p))
        if len(keys) == 0:
            continue
        s = (np.asarray(k[keys], dtype=np.float64) @ q[i]) / math.sqrt(d)
        e = np.exp(s - s.max())
        out[slot] = (e / e.sum()) @ np.asarray(v[keys], dtype=np.float64)
    return out


# ----------------------------------------------------------------------------
# Step 8: masked softmax attention
# ----------------------------------------------------------------------------
def attention_rows(q, k, v, rows, lv, R2, T, H, W, p):
    """O_i for the listed query indices, fp64 (softmax over retained keys only)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    out = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    for slot, i in enumerate(rows):
        keys = retained_keys(int(i), int(lv[i]), R2, T, H, W, p)
        s = (np.asarray(k[keys], dtype=np.float64) @ q[i]) / math.sqrt(d)
        e = np.exp(s - s.max())
        out[slot] = (e / e.sum()) @ np.asarray(v[keys], dtype=np.float64)
    return out


def dense_attention(q, k, v, mask=None):
    """softmax(q k^T / sqrt(d)) v in fp64, optionally with a boolean mask."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = (q @ k.T) / math.sqrt(q.shape[1])
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ v


# ----------------------------------------------------------------------------
# Warm-up variant: the entropy measured on a dense pass
# ----------------------------------------------------------------------------
def dense_entropy(q, k):
    """Entropy of each query's full softmax over all N keys, fp64:
    H_i = -sum_j p_ij ln p_ij with p_i = softmax_j(q_i.k_j/sqrt(d)).

    The summary page's pipeline ("Le Pipeline TRA", entropy-to-budget step)
    takes the entropy during dense warm-up steps, on the full attention rather
    than on pooled keys; levels, radii and tile lists then follow the same
    steps 4-7 as the pooled estimate.
    """
    q, k = (np.asarray(x, dtype=np.float64) for x in (q, k))
    s = (q @ k.T) / math.sqrt(q.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(p > 0, -p * np.log(p), 0.0)
    return terms.sum(axis=1)


# ----------------------------------------------------------------------------
# Steps 1-7 for one (batch, head) slice
# ----------------------------------------------------------------------------
def plan(q, k, cfg, want_csr=True):
    """Pooled keys, entropies, levels, radius table and (optionally) CSR for one
    [N, d] head.  `cfg` is a workloads.Workload."""
    p = cfg.params()
    pools = Geometry(cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w)
    kbar = pool_keys(k, pools, cfg.dtype)
    H = entropy(q, kbar, pools.block_sizes())
    lv = levels(H, p)
    R2 = radius_table(p, cfg.T)
    out = {"kbar": kbar, "H": H, "levels": lv, "R2": R2, "params": p}
    if want_csr:
        tiles = Geometry(cfg.T, cfg.H, cfg.W, cfg.tile_h, cfg.tile_w)
        out["row_ptr"], out["col_idx"] = csr(lv, R2, tiles, p)
    return out
