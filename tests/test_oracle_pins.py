"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle against a closed form, a textbook count, a library
routine or a brute-force enumeration computed differently, so that a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails here.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from workloads import small_workload, CONFIGS, positional_features


def _p(**kw):
    base = dict(a=1.0, c=0.0, budget_min=16.0, budget_max=2048.0, decay=0.5,
                levels_per_nat=8, pool_h=8, pool_w=8, tile_h=8, tile_w=8, radius_override=-1.0)
    base.update(kw)
    return base


# ---------------------------------------------------------------------------
# Rounding of the pooled mean: brute force over bf16 bit patterns
# ---------------------------------------------------------------------------
def _bf16_values_around(x):
    """All bf16 values adjacent to x, as exact Fractions, by enumerating bit patterns."""
    f32 = np.array([x], dtype=np.float32).view(np.uint32)[0]
    top = int(f32 >> 16)
    out = []
    for b in range(max(0, top - 2), min(0xFFFF, top + 3)):
        v = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        if np.isfinite(v):
            out.append((b, Fraction(float(v))))
    return out


def _nearest_bf16(exact: Fraction):
    sign = -1 if exact < 0 else 1
    cands = _bf16_values_around(float(abs(exact)))
    best = min(cands, key=lambda bv: (abs(bv[1] - abs(exact)), bv[0] & 1))
    return sign * best[1]


def test_round_to_bf16_matches_bit_pattern_search():
    rng = np.random.default_rng(1)
    nums = (rng.standard_normal(3000) * 4.0).astype(np.float64)
    dens = rng.integers(1, 300, size=3000)
    got = O.round_to_dtype(nums, dens, "bf16")
    for x, n, g in zip(nums, dens, got):
        assert Fraction(float(g)) == _nearest_bf16(Fraction(float(x)) / int(n))


def test_round_to_bf16_ties_and_near_ties():
    """Exact midpoints between two bf16 values round to the even pattern; the
    nearest float64 numerators on either side round away from the midpoint."""
    checked = 0
    for den in (1, 3, 7, 64, 208, 224, 255, 256):
        for top in range(128, 256, 5):
            mid = Fraction(2 * top + 1, 2 * 128) * Fraction(2) ** int(top % 7 - 3)
            num = float(mid * den)
            if Fraction(num) != mid * den:
                continue
            for x in (num, np.nextafter(num, np.inf), np.nextafter(num, -np.inf)):
                for sgn in (1.0, -1.0):
                    got = O.round_to_dtype(np.array([sgn * x]), np.array([den]), "bf16")[0]
                    assert Fraction(float(got)) == _nearest_bf16(Fraction(float(sgn * x)) / den)
                    checked += 1
    assert checked > 100


def test_pool_keys_exact_mean_bf16_ragged():
    cfg = small_workload(T=2, H=11, W=13, heads=1, head_dim=16, dtype="bf16", pool_h=4, pool_w=5)
    rng = np.random.default_rng(3)
    k32 = torch.from_numpy(rng.standard_normal((cfg.N, 16)).astype(np.float32)).to(torch.bfloat16)
    k = k32.double().numpy()
    geom = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w)
    kbar = O.pool_keys(k, geom, "bf16")
    for b in range(geom.count):
        toks = geom.tokens(b)
        for dim in range(16):
            exact = sum(Fraction(float(k[j, dim])) for j in toks) / len(toks)
            assert Fraction(float(kbar[b, dim])) == _nearest_bf16(exact)


def test_pool_keys_fp32_power_of_two_blocks_are_plain_means():
    """For 8x8 blocks the exact mean is a power-of-two scaling of an exact sum;
    numpy's fp32 conversion of the (exactly representable) fp64 mean is then the
    single correctly rounded result."""
    rng = np.random.default_rng(4)
    T, H, W = 2, 16, 16
    k = rng.standard_normal((T * H * W, 8)).astype(np.float32).astype(np.float64)
    geom = O.Geometry(T, H, W, 8, 8)
    kbar = O.pool_keys(k, geom, "fp32")
    for b in range(geom.count):
        s = math.fsum  # exact sums
        toks = geom.tokens(b)
        for dim in range(8):
            exact_mean = s(k[toks, dim]) / 64.0  # exact: fsum is correctly rounded, /64 exact
            assert kbar[b, dim] == np.float64(np.float32(exact_mean))


def test_geometry_block_sizes_cover_grid():
    g = O.Geometry(3, 45, 80, 16, 16)
    sizes = g.block_sizes()
    assert sizes.sum() == 3 * 45 * 80
    assert set(np.unique(sizes)) == {256, 208}
    blk = g.block_of_tokens()
    assert np.array_equal(np.bincount(blk, minlength=g.count), sizes)


# ---------------------------------------------------------------------------
# Entropy
# ---------------------------------------------------------------------------
def test_entropy_all_keys_equal_is_log_n():
    T, H, W, d = 2, 9, 10, 16
    geom = O.Geometry(T, H, W, 4, 4)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((7, d)) * 3.0
    kbar = np.tile(rng.standard_normal((1, d)), (geom.count, 1))
    Hq = O.entropy(q, kbar, geom.block_sizes())
    assert np.allclose(Hq, math.log(T * H * W), atol=1e-12, rtol=0)


def test_entropy_equals_explicit_softmax_entropy_ragged():
    T, H, W, d = 2, 11, 13, 16
    geom = O.Geometry(T, H, W, 4, 5)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((20, d)) * rng.uniform(0.2, 6.0, size=(20, 1))
    kbar = rng.standard_normal((geom.count, d))
    Hq = O.entropy(q, kbar, geom.block_sizes())
    ref = O.explicit_softmax_entropy(q, kbar, geom)
    assert np.max(np.abs(Hq - ref)) < 1e-11


def test_entropy_two_point_closed_form():
    """Two blocks of sizes n1, n2 with scores z1, z2: H = ln Z - (n1 e^z1 z1 + n2 e^z2 z2)/Z
    evaluated from the binary-entropy form H = h(p) + p ln n1 + (1-p) ln n2."""
    d = 4
    geom = O.Geometry(1, 1, 5, 1, 3)  # blocks of 3 and 2 tokens
    kbar = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    q = np.array([[0.7, -1.3, 0, 0]]) * math.sqrt(d)
    z1, z2 = 0.7, -1.3
    w1, w2 = 3 * math.exp(z1), 2 * math.exp(z2)
    p = w1 / (w1 + w2)
    expected = -p * math.log(p) - (1 - p) * math.log(1 - p) + p * math.log(3) + (1 - p) * math.log(2)
    assert abs(O.entropy(q, kbar, geom.block_sizes())[0] - expected) < 1e-13


def test_entropy_bounds_on_generated_inputs():
    from workloads import make_inputs
    cfg = CONFIGS["tiny"]
    q, k, _ = make_inputs(cfg, heads=[0])
    geom = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w)
    kbar = O.pool_keys(k[0, 0].double().numpy(), geom, cfg.dtype)
    Hq = O.entropy(q[0, 0].double().numpy(), kbar, geom.block_sizes())
    assert np.all(Hq <= math.log(cfg.N) + 1e-12)
    assert np.all(Hq >= math.log(geom.block_sizes().min()) - 1e-12)


# ---------------------------------------------------------------------------
# Dense (warm-up) entropy
# ---------------------------------------------------------------------------
def test_dense_entropy_matches_scipy():
    from scipy.special import softmax
    from scipy.stats import entropy as scipy_entropy
    rng = np.random.default_rng(21)
    d = 32
    q = rng.standard_normal((9, d)) * rng.uniform(0.2, 8.0, size=(9, 1))
    k = rng.standard_normal((150, d))
    ref = scipy_entropy(softmax(q @ k.T / math.sqrt(d), axis=1), axis=1)
    assert np.max(np.abs(O.dense_entropy(q, k) - ref)) < 1e-11


def test_dense_entropy_is_pooled_entropy_with_one_token_blocks():
    """With 1x1 pool blocks the pooled-key entropy (log-sum-exp form) is the
    dense entropy (-sum p ln p form)."""
    T, H, W, d = 2, 5, 7, 16
    geom = O.Geometry(T, H, W, 1, 1)
    rng = np.random.default_rng(22)
    q = rng.standard_normal((11, d)) * 4.0
    k = rng.standard_normal((T * H * W, d)).astype(np.float32).astype(np.float64)
    kbar = O.pool_keys(k, geom, "fp32")
    assert np.array_equal(kbar, k)
    assert np.max(np.abs(O.dense_entropy(q, k) - O.entropy(q, kbar, geom.block_sizes()))) < 1e-11


def test_dense_entropy_closed_forms():
    d, n1, n2 = 8, 13, 29
    rng = np.random.default_rng(23)
    q = rng.standard_normal((4, d)) * 2.0
    same = np.tile(rng.standard_normal((1, d)), (n1 + n2, 1))
    assert np.allclose(O.dense_entropy(q, same), math.log(n1 + n2), atol=1e-12, rtol=0)
    # n1 copies of key a and n2 of key b: H = h(p) + p ln n1 + (1-p) ln n2, where
    # p is the total probability of the a copies.
    ka, kb = rng.standard_normal(d), rng.standard_normal(d)
    keys = np.vstack([np.tile(ka, (n1, 1)), np.tile(kb, (n2, 1))])
    za, zb = q @ ka / math.sqrt(d), q @ kb / math.sqrt(d)
    pa = n1 * np.exp(za) / (n1 * np.exp(za) + n2 * np.exp(zb))
    expected = -pa * np.log(pa) - (1 - pa) * np.log(1 - pa) + pa * math.log(n1) + (1 - pa) * math.log(n2)
    assert np.max(np.abs(O.dense_entropy(q, keys) - expected)) < 1e-12


# ---------------------------------------------------------------------------
# Levels
# ---------------------------------------------------------------------------
def test_levels_by_search():
    p = _p(a=0.9, c=-0.4, budget_min=20.0, budget_max=900.0, levels_per_nat=8)
    rng = np.random.default_rng(7)
    Hs = np.concatenate([rng.uniform(0, 10, 500), np.arange(0, 80) / 8.0 / 0.9 + 0.4 / 0.9])
    got = O.levels(Hs, p)
    for H, k in zip(Hs, got):
        # largest integer k with k <= 8*(a*H + c), by linear search, then the clamp
        L = 8 * (0.9 * H - 0.4)
        kk = -1000
        while kk + 1 <= L:
            kk += 1
        lo = next(j for j in range(-100, 200) if math.exp(j / 8) >= 20.0)
        hi = max(j for j in range(-100, 200) if math.exp(j / 8) <= 900.0)
        assert k == min(max(kk, lo), hi)


def test_excused_queries_window():
    p = _p()
    k_lo, k_hi = O.level_range(p)
    Hb = (k_lo + 5) / 8.0
    Hs = np.array([Hb - 2e-5, Hb - 5e-6, Hb, Hb + 5e-6, Hb + 2e-5, (k_lo - 3) / 8.0, (k_hi + 3) / 8.0])
    assert list(O.excused_queries(Hs, p)) == [1, 2, 3]
    single = _p(budget_min=1.0, budget_max=1.0)  # one level: nothing can move it
    assert len(O.excused_queries(np.array([0.0, 1e-7]), single)) == 0


# ---------------------------------------------------------------------------
# Radius table and mask
# ---------------------------------------------------------------------------
# Lattice points x^2 + y^2 <= n for n = 0..10 (Gauss circle problem).
GAUSS = [1, 5, 9, 9, 13, 21, 21, 21, 25, 29, 37]


@pytest.mark.parametrize("n", range(11))
def test_gauss_circle_counts_single_frame(n):
    p = _p(radius_override=math.sqrt(n) if n else 0.0, decay=1.0)
    T, H, W = 1, 15, 15
    R2 = O.radius_table(p, T)
    i = (0 * H + 7) * W + 7
    assert len(O.retained_keys(i, -1, R2, T, H, W, p)) == GAUSS[n]
    assert O.retained_count(i, -1, R2, T, H, W, p) == GAUSS[n]


def test_gauss_circle_counts_across_frames():
    """Interior query, decay 1/2: frame delta retains N_disk(floor(r0^2/4^delta))
    keys in each of the (1 or 2) frames at that distance."""
    p = _p(radius_override=3.0, decay=0.5)  # r0^2 = 9 -> 9, 2, 0(inactive)
    T, H, W = 5, 13, 13
    R2 = O.radius_table(p, T)
    assert list(R2[0]) == [9, 2, -1, -1, -1]
    i = (2 * H + 6) * W + 6  # middle frame: two frames at delta = 1
    assert O.retained_count(i, -1, R2, T, H, W, p) == 29 + 2 * 9
    i0 = (0 * H + 6) * W + 6  # first frame: one neighbour frame
    assert O.retained_count(i0, -1, R2, T, H, W, p) == 29 + 9


def test_radius_table_decay_one_is_uniform_high_precision():
    """With decay 1 every frame shares the budget equally: R2 = floor(e^{k/q}/(pi (2T-1)))
    for every delta, evaluated here in 50-digit decimal arithmetic."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    pi = Decimal("3.14159265358979323846264338327950288419716939937510")
    T = 6
    p = _p(decay=1.0, budget_min=16.0, budget_max=5000.0)
    R2 = O.radius_table(p, T)
    k_lo, k_hi = O.level_range(p)
    for row, k in enumerate(range(k_lo, k_hi + 1)):
        val = int((Decimal(k) / 8).exp() / (pi * (2 * T - 1)))
        assert R2[row][0] == val
        assert all(x == (val if val >= 1 else -1) for x in R2[row][1:])


def test_radius_conserves_budget_single_frame():
    """T = 1: the disk holds the budget, so an interior query's retained count is
    the quantised budget up to the Gauss-circle error (|N - pi r^2| < 2 pi r + 5)."""
    p = _p(budget_min=16.0, budget_max=3000.0)
    T, H, W = 1, 81, 81
    R2 = O.radius_table(p, T)
    k_lo, k_hi = O.level_range(p)
    i = 40 * W + 40
    for row, k in enumerate(range(k_lo, k_hi + 1)):
        B = math.exp(k / 8)
        cnt = O.retained_count(i, k, R2, T, H, W, p)
        assert abs(cnt - B) < 2 * math.pi * math.sqrt(B / math.pi) + 5


def test_radius_conserves_budget_across_frames():
    """Interior query in the middle of a long clip: retained keys summed over
    frames approximate the quantised budget (the budget is spread over the
    frames' disks, not given to each)."""
    p = _p(budget_min=16.0, budget_max=20000.0, decay=0.7)
    T, H, W = 31, 121, 121
    R2 = O.radius_table(p, T)
    k_lo, k_hi = O.level_range(p)
    k = k_hi
    B = math.exp(k / 8)
    i = (15 * H + 60) * W + 60
    cnt = O.retained_count(i, k, R2, T, H, W, p)
    assert abs(cnt - B) / B < 0.06


def test_config_tables_are_unambiguous():
    for cfg in CONFIGS.values():
        assert O.table_margin(cfg.params(), cfg.T) > 1e-9


def _random_levels(rng, N, p):
    k_lo, k_hi = O.level_range(p)
    return rng.integers(k_lo, k_hi + 1, size=N)


@pytest.mark.parametrize("seed", range(6))
def test_disk_enumeration_matches_dense_mask(seed):
    rng = np.random.default_rng(100 + seed)
    T, H, W = int(rng.integers(1, 5)), int(rng.integers(1, 10)), int(rng.integers(1, 10))
    p = _p(budget_min=2.0, budget_max=400.0, decay=float(rng.uniform(0.3, 1.0)))
    R2 = O.radius_table(p, T)
    lv = _random_levels(rng, T * H * W, p)
    mask = O.dense_mask(lv, R2, T, H, W, p)
    for i in range(T * H * W):
        keys = O.retained_keys(i, lv[i], R2, T, H, W, p)
        assert np.array_equal(keys, np.nonzero(mask[i])[0])
        assert O.retained_count(i, lv[i], R2, T, H, W, p) == mask[i].sum()
        assert mask[i, i]
    assert np.array_equal(O.retained_counts(lv, R2, T, H, W, p), mask.sum(axis=1))


@pytest.mark.parametrize("seed", range(4))
def test_csr_coverage_and_minimality(seed):
    rng = np.random.default_rng(200 + seed)
    T, H, W = int(rng.integers(1, 4)), int(rng.integers(3, 20)), int(rng.integers(3, 20))
    p = _p(budget_min=2.0, budget_max=300.0, decay=float(rng.uniform(0.3, 1.0)),
           tile_h=int(rng.choice([2, 3, 8])), tile_w=int(rng.choice([2, 5, 8])))
    R2 = O.radius_table(p, T)
    lv = _random_levels(rng, T * H * W, p)
    mask = O.dense_mask(lv, R2, T, H, W, p)
    tiles = O.Geometry(T, H, W, p["tile_h"], p["tile_w"])
    blk = tiles.block_of_tokens()
    hit = np.zeros((tiles.count, tiles.count), dtype=bool)
    qi, kj = np.nonzero(mask)
    hit[blk[qi], blk[kj]] = True
    row_ptr, col_idx = O.csr(lv, R2, tiles, p)
    for a in range(tiles.count):
        assert np.array_equal(col_idx[row_ptr[a]:row_ptr[a + 1]], np.nonzero(hit[a])[0])


# ---------------------------------------------------------------------------
# Alternative generators: fixed Manhattan radius, Radial static mask
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("R", range(5))
def test_manhattan_counts_are_octahedral_numbers(R):
    """Interior query: the 3D L1 ball of radius R holds the centred octahedral
    number (2R+1)(2R^2+2R+3)/3 of lattice points; frame delta holds the
    centred square number 2m^2+2m+1, m = R - delta."""
    p = _p(radius_override=R + 0.5, generator=O.GEN_MANHATTAN)
    T, H, W = 2 * R + 3, 2 * R + 5, 2 * R + 7
    R2 = O.radius_table(p, T)
    i = ((T // 2) * H + H // 2) * W + W // 2
    expected = (2 * R + 1) * (2 * R * R + 2 * R + 3) // 3
    assert O.retained_count(i, -1, R2, T, H, W, p) == expected
    keys = O.retained_keys(i, -1, R2, T, H, W, p)
    assert len(keys) == expected
    t = keys // (H * W)
    for delta in range(R + 1):
        m = R - delta
        assert np.sum(t == T // 2 + delta) == 2 * m * m + 2 * m + 1
    assert np.sum(np.abs(t - T // 2) > R) == 0


def test_radial_table_bands():
    """Octave bands 0 | 1 | 2-3 | 4-7 | 8-15 | 16-31 and a disk area halving per band."""
    p = _p(radius_override=8.0, generator=O.GEN_RADIAL)
    R2 = O.radius_table(p, 20)
    assert list(R2[0]) == [64, 32, 16, 16] + [8] * 4 + [4] * 8 + [2] * 4
    assert [O.radial_band(d) for d in range(9)] == [0, 1, 2, 2, 3, 3, 3, 3, 4]
    # Each band b >= 1 spends the same total area r0^2/2 (2^(b-1) frames of r0^2/2^b):
    # the O(n log n) budget of a static mask that shrinks with temporal distance.
    q = _p(radius_override=16.0, generator=O.GEN_RADIAL)
    row = O.radius_table(q, 128)[0]
    for b in range(1, 8):
        assert sum(row[2 ** (b - 1):2 ** b]) == 128
    tiny = O.radius_table(_p(radius_override=2.0, generator=O.GEN_RADIAL), 6)[0]
    assert list(tiny) == [4, 2, 1, 1, -1, -1]  # 4/8 < 1: inactive from band 3 on


@pytest.mark.parametrize("gen,seed", [(g, s) for g in (1, 2) for s in range(2)])
def test_generator_masks_enumeration_and_csr(gen, seed):
    rng = np.random.default_rng(300 + seed)
    T, H, W = int(rng.integers(1, 5)), int(rng.integers(3, 14)), int(rng.integers(3, 14))
    p = _p(radius_override=float(rng.uniform(0.0, 6.0)), generator=gen, tile_h=int(rng.choice([2, 3, 8])),
           tile_w=int(rng.choice([2, 5, 8])))
    R2 = O.radius_table(p, T)
    lv = np.full(T * H * W, -1)
    mask = O.dense_mask(lv, R2, T, H, W, p)
    n = np.arange(T * H * W)
    t, h, w = n // (H * W), (n // W) % H, n % W
    if gen == O.GEN_MANHATTAN:  # the ball itself, straight from the coordinates
        ref = (np.abs(t[:, None] - t[None, :]) + np.abs(h[:, None] - h[None, :]) + np.abs(w[:, None] - w[None, :])
               <= math.floor(p["radius_override"]))
        assert np.array_equal(mask, ref)
    for i in range(T * H * W):
        assert np.array_equal(O.retained_keys(i, -1, R2, T, H, W, p), np.nonzero(mask[i])[0])
        assert O.retained_count(i, -1, R2, T, H, W, p) == mask[i].sum()
    assert np.array_equal(O.retained_counts(lv, R2, T, H, W, p), mask.sum(axis=1))
    tiles = O.Geometry(T, H, W, p["tile_h"], p["tile_w"])
    blk = tiles.block_of_tokens()
    hit = np.zeros((tiles.count, tiles.count), dtype=bool)
    qi, kj = np.nonzero(mask)
    hit[blk[qi], blk[kj]] = True
    row_ptr, col_idx = O.csr(lv, R2, tiles, p)
    for a in range(tiles.count):
        assert np.array_equal(col_idx[row_ptr[a]:row_ptr[a + 1]], np.nonzero(hit[a])[0])


def test_window_1d_table_holds_the_budget():
    """Each level's window of 2 rho + 1 tokens is the largest odd window within
    the quantised budget B = e^(k/q): 2 rho + 1 <= B < 2 rho + 3."""
    p = _p(generator=O.GEN_WINDOW_1D)
    R2 = O.radius_table(p, 3)
    k_lo, k_hi = O.level_range(p)
    assert R2.shape == (k_hi - k_lo + 1, 3)
    for r, k in enumerate(range(k_lo, k_hi + 1)):
        B = math.exp(k / p["levels_per_nat"])
        rho = int(R2[r, 0])
        assert np.all(R2[r] == rho)
        assert 2 * rho + 1 <= B < 2 * rho + 3
    assert list(O.radius_table(_p(generator=O.GEN_WINDOW_1D, radius_override=7.9), 2)[0]) == [7, 7]


@pytest.mark.parametrize("seed", range(3))
def test_window_1d_masks_enumeration_and_csr(seed):
    rng = np.random.default_rng(500 + seed)
    T, H, W = int(rng.integers(1, 4)), int(rng.integers(2, 12)), int(rng.integers(2, 12))
    p = _p(budget_min=2.0, budget_max=300.0, generator=O.GEN_WINDOW_1D,
           tile_h=int(rng.choice([2, 3, 8])), tile_w=int(rng.choice([2, 5, 8])))
    R2 = O.radius_table(p, T)
    lv = _random_levels(rng, T * H * W, p)
    mask = O.dense_mask(lv, R2, T, H, W, p)
    # the window straight from coordinates
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    n = ((t * H + h) * W + w).reshape(-1)
    rho = R2[lv - O.level_range(p)[0], 0]
    assert np.array_equal(mask, np.abs(n[:, None] - n[None, :]) <= rho[:, None])
    for i in range(T * H * W):
        assert np.array_equal(O.retained_keys(i, lv[i], R2, T, H, W, p), np.nonzero(mask[i])[0])
        assert O.retained_count(i, lv[i], R2, T, H, W, p) == mask[i].sum()
    assert np.array_equal(O.retained_counts(lv, R2, T, H, W, p), mask.sum(axis=1))
    tiles = O.Geometry(T, H, W, p["tile_h"], p["tile_w"])
    blk = tiles.block_of_tokens()
    hit = np.zeros((tiles.count, tiles.count), dtype=bool)
    qi, kj = np.nonzero(mask)
    hit[blk[qi], blk[kj]] = True
    row_ptr, col_idx = O.csr(lv, R2, tiles, p)
    for a in range(tiles.count):
        assert np.array_equal(col_idx[row_ptr[a]:row_ptr[a + 1]], np.nonzero(hit[a])[0])


# ---------------------------------------------------------------------------
# Token voting with a threshold; block-only masks
# ---------------------------------------------------------------------------
def _vote_case(seed):
    rng = np.random.default_rng(400 + seed)
    T, H, W = int(rng.integers(1, 4)), int(rng.integers(3, 17)), int(rng.integers(3, 17))
    p = _p(budget_min=2.0, budget_max=300.0, decay=float(rng.uniform(0.3, 1.0)),
           tile_h=int(rng.choice([2, 3, 4])), tile_w=int(rng.choice([2, 5, 4])))
    R2 = O.radius_table(p, T)
    lv = _random_levels(rng, T * H * W, p)
    return T, H, W, p, R2, lv, O.Geometry(T, H, W, p["tile_h"], p["tile_w"])


@pytest.mark.parametrize("seed", range(3))
def test_tile_votes_match_brute_force_mask(seed):
    T, H, W, p, R2, lv, tiles = _vote_case(seed)
    mask = O.dense_mask(lv, R2, T, H, W, p)
    blk = tiles.block_of_tokens()
    counts = np.zeros((tiles.count, tiles.count), dtype=np.int64)
    qi, kj = np.nonzero(mask)
    np.add.at(counts, (blk[qi], blk[kj]), 1)
    for a in range(tiles.count):
        votes = O.tile_votes(a, lv, R2, tiles, p)
        assert votes == {int(b): int(counts[a, b]) for b in np.nonzero(counts[a])[0]}
    rp1, ci1 = O.csr_vote(lv, R2, tiles, p, 1)
    rp, ci = O.csr(lv, R2, tiles, p)
    assert np.array_equal(rp1, rp) and np.array_equal(ci1, ci)
    for theta in (2, 5, 17):
        rpt, cit = O.csr_vote(lv, R2, tiles, p, theta)
        for a in range(tiles.count):
            assert np.array_equal(cit[rpt[a]:rpt[a + 1]], np.nonzero(counts[a] >= theta)[0])


def test_listed_attention_matches_library_sdpa():
    T, H, W, p, R2, lv, tiles = _vote_case(7)
    rng = np.random.default_rng(17)
    d = 16
    N = T * H * W
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    mask = O.dense_mask(lv, R2, T, H, W, p)
    blk = tiles.block_of_tokens()
    rp, ci = O.csr_vote(lv, R2, tiles, p, 3)
    listed = np.zeros((tiles.count, tiles.count), dtype=bool)
    for a in range(tiles.count):
        listed[a, ci[rp[a]:rp[a + 1]]] = True
    block_mask = listed[blk[:, None], blk[None, :]]
    rows = np.nonzero(block_mask.any(axis=1) & (mask & block_mask).any(axis=1))[0]
    got_b = O.attention_rows_listed(q, k, v, rows, lv, R2, tiles, p, rp, ci, True)
    assert np.max(np.abs(got_b - _sdpa(q, k, v, block_mask)[rows])) < 1e-12
    got_x = O.attention_rows_listed(q, k, v, rows, lv, R2, tiles, p, rp, ci, False)
    assert np.max(np.abs(got_x - _sdpa(q, k, v, mask & block_mask)[rows])) < 1e-12
    # With threshold 1 the exact mask loses nothing to the tile lists.
    rp1, ci1 = O.csr(lv, R2, tiles, p)
    allr = np.arange(N)
    assert np.max(np.abs(O.attention_rows_listed(q, k, v, allr, lv, R2, tiles, p, rp1, ci1, False)
                         - O.attention_rows(q, k, v, allr, lv, R2, T, H, W, p))) < 1e-12


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def _sdpa(q, k, v, mask=None):
    import torch.nn.functional as F
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)[0, 0].numpy()


def test_dense_limit_matches_library_sdpa():
    T, H, W, d = 3, 5, 6, 16
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((T * H * W, d)) for _ in range(3))
    p = _p(radius_override=math.hypot(H - 1, W - 1) + 0.01, decay=1.0)
    R2 = O.radius_table(p, T)
    lv = np.full(T * H * W, -1)
    out = O.attention_rows(q, k, v, np.arange(T * H * W), lv, R2, T, H, W, p)
    assert np.max(np.abs(out - _sdpa(q, k, v))) < 1e-12
    assert np.max(np.abs(out - O.dense_attention(q, k, v))) < 1e-12


def test_radius_zero_returns_own_value():
    T, H, W, d = 2, 4, 5, 8
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((T * H * W, d)) for _ in range(3))
    p = _p(radius_override=0.0)
    R2 = O.radius_table(p, T)
    out = O.attention_rows(q, k, v, np.arange(T * H * W), np.full(T * H * W, -1), R2, T, H, W, p)
    assert np.array_equal(out, v)


@pytest.mark.parametrize("seed", range(3))
def test_masked_attention_matches_library_sdpa(seed):
    rng = np.random.default_rng(300 + seed)
    T, H, W, d = 3, 7, 9, 16
    p = _p(budget_min=2.0, budget_max=200.0, decay=0.6)
    R2 = O.radius_table(p, T)
    lv = _random_levels(rng, T * H * W, p)
    q, k, v = (rng.standard_normal((T * H * W, d)) * 2 for _ in range(3))
    mask = O.dense_mask(lv, R2, T, H, W, p)
    out = O.attention_rows(q, k, v, np.arange(T * H * W), lv, R2, T, H, W, p)
    assert np.max(np.abs(out - _sdpa(q, k, v, mask))) < 1e-12
    # convexity: every output channel lies within the retained values' range
    for i in range(T * H * W):
        vv = v[mask[i]]
        assert np.all(out[i] <= vv.max(axis=0) + 1e-12) and np.all(out[i] >= vv.min(axis=0) - 1e-12)


# ---------------------------------------------------------------------------
# Generator
# ---------------------------------------------------------------------------
def test_positional_feature_norm():
    P = positional_features(3, 4, 5, 64)
    assert P.shape == (60, 64)
    assert np.allclose((P ** 2).sum(axis=1), 32.0)  # one sin^2 + cos^2 = 1 per frequency


def test_generator_is_deterministic_and_head_local():
    from workloads import make_inputs
    cfg = small_workload(T=2, H=5, W=6, heads=3, head_dim=64)
    q1, k1, v1 = make_inputs(cfg)
    q2, _, _ = make_inputs(cfg, heads=[1])
    assert q1.dtype == torch.bfloat16 and q1.shape == (1, 3, 60, 64)
    assert torch.equal(q1[:, 1:2], q2)
    q3, _, _ = make_inputs(cfg)
    assert torch.equal(q1, q3)
