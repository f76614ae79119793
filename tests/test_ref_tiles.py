"""The vectorised reference tile lists (tests/ref_tiles.py) against the
oracle's query-by-query definition (`oracle.csr`), on random small grids with
ragged edges, mixed budget levels and every generator."""
import numpy as np
import pytest

import oracle as O
from workloads import small_workload

import ref_tiles


def _levels(cfg, rng):
    p = cfg.params()
    if p["radius_override"] >= 0:
        return np.full(cfg.N, -1, dtype=np.int64)
    k_lo, k_hi = O.level_range(p)
    return rng.integers(k_lo, k_hi + 1, size=cfg.N)


CASES = [
    # (T, H, W, extra workload fields)
    (3, 13, 21, dict(c=-0.5, budget_max=819.0)),
    (4, 17, 9, dict(c=-1.0, budget_max=600.0, decay=0.7)),
    (2, 8, 8, dict(budget_max=128.0)),
    (5, 11, 26, dict(c=0.5, budget_max=1430.0, decay=0.35)),
    (1, 30, 37, dict(budget_max=1110.0)),
    (3, 13, 21, dict(radius_override=6.5)),
    (3, 13, 21, dict(radius_override=7.0, generator=1)),
    (4, 13, 21, dict(radius_override=13.0, generator=2)),
    (4, 13, 21, dict(c=-2.0, budget_max=600.0, generator=3)),
    (4, 13, 21, dict(radius_override=40.0, generator=3)),
    (2, 3, 5, dict(radius_override=0.0)),
    (1, 1, 1, dict(budget_min=1.0, budget_max=1.0)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_reference_tile_lists_match_oracle(case):
    T, H, W, extra = CASES[case]
    cfg = small_workload(T=T, H=H, W=W, heads=1, **extra)
    p = cfg.params()
    rng = np.random.default_rng(100 + case)
    lv = _levels(cfg, rng)
    R2 = O.radius_table(p, T)
    tiles = O.Geometry(T, H, W, 8, 8)
    rp_o, ci_o = O.csr(lv, R2, tiles, p)
    rp_r, ci_r = ref_tiles.csr(lv, R2, T, H, W, p)
    assert np.array_equal(rp_o, rp_r)
    assert np.array_equal(ci_o, ci_r)


def test_query_sample_covers_every_border_tile():
    T, H, W = 3, 13, 21
    rng = np.random.default_rng(0)
    qs = ref_tiles.query_sample(T, H, W, 100, rng)
    assert len(qs) >= 100 and len(np.unique(qs)) == len(qs)
    tiles = O.Geometry(T, H, W, 8, 8)
    hit = set(tiles.block_of_tokens()[qs].tolist())
    for t in range(T):
        for r in range(tiles.nbh):
            for c in range(tiles.nbw):
                if r in (0, tiles.nbh - 1) or c in (0, tiles.nbw - 1):
                    assert (t * tiles.nbh + r) * tiles.nbw + c in hit
    assert 0 in qs and T * H * W - 1 in qs
