"""GPU parity of the HIP path against the fp64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import sparse_self_attention_amd as tra
from workloads import CONFIGS, make_inputs, perturb, small_workload

from oracle import runner

import ref_tiles
from parity_util import (check_csr_properties, check_group_lists, check_head, check_key_sets, check_levels,
                         check_listed, gpu_run)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_tiny_workload_full_parity(gpu):
    cfg = CONFIGS["tiny"]
    _say("case: tiny fp32", cfg)
    run = gpu_run(cfg, gpu)
    for h in range(cfg.heads):
        m = check_head(cfg, run, 0, h)
        _say("head", h, {k: v for k, v in m.items() if k not in ("excused", "level_mismatch")},
             "excused", len(m["excused"]), "mismatch", len(m["level_mismatch"]))
        assert m["o_max_abs"] < 1e-4  # fp32 path


@pytest.mark.parametrize("shape", [(3, 13, 21, 128), (2, 17, 9, 64), (4, 8, 8, 128), (1, 30, 37, 128)])
def test_small_bf16_full_parity(gpu, shape):
    T, H, W, d = shape
    cfg = small_workload(T=T, H=H, W=W, heads=2, head_dim=d, c=-0.5, budget_max=float(T * H * W))
    _say("case: small bf16", shape)
    run = gpu_run(cfg, gpu)
    check_csr_properties(cfg, run)
    for h in range(cfg.heads):
        check_group_lists(cfg, run, h)
        m = check_head(cfg, run, 0, h)
        _say("head", h, m["o_max_abs"], m["o_mean_abs"], m.get("entropy_max_abs_err"),
             "excused", len(m.get("excused", [])))


def test_small_fp32_d128_parity(gpu):
    cfg = small_workload(T=2, H=11, W=19, heads=1, head_dim=128, dtype="fp32", budget_max=418.0)
    _say("case: small fp32 d128")
    run = gpu_run(cfg, gpu)
    m = check_head(cfg, run, 0, 0)
    assert m["o_max_abs"] < 1e-4


@pytest.mark.parametrize("kw", [dict(generator=1, radius_override=5.0), dict(generator=2, radius_override=6.0),
                                dict(generator=3, c=-2.0, budget_max=300.0)])
def test_small_fp32_d128_generators(gpu, kw):
    """The fp32 kernel at d = 128 (four waves per query tile) with the
    Manhattan, Radial and 1-D window masks: every output against the oracle."""
    cfg = small_workload(T=3, H=11, W=19, heads=1, head_dim=128, dtype="fp32", **kw)
    _say("case: small fp32 d128", kw)
    run = gpu_run(cfg, gpu)
    m = check_head(cfg, run, 0, 0)
    assert m["o_max_abs"] < 1e-4


def test_batch_of_two(gpu):
    cfg = small_workload(T=2, H=9, W=12, heads=2, batch=2, c=-0.25, budget_max=216.0)
    _say("case: batch 2")
    run = gpu_run(cfg, gpu)
    for b in range(2):
        for h in range(2):
            check_head(cfg, run, b, h)


def test_degenerate_grids(gpu):
    for (T, H, W) in [(1, 1, 1), (1, 1, 5), (2, 3, 2), (1, 7, 1)]:
        cfg = small_workload(T=T, H=H, W=W, heads=1, head_dim=64, pool_h=2, pool_w=2,
                             budget_min=1.0, budget_max=max(1.0, float(T * H * W)))
        _say("case: degenerate", (T, H, W))
        run = gpu_run(cfg, gpu)
        check_head(cfg, run, 0, 0)


def test_radius_zero_returns_own_value(gpu):
    cfg = small_workload(T=3, H=10, W=12, heads=2, radius_override=0.0)
    _say("case: radius 0")
    run = gpu_run(cfg, gpu)
    assert torch.equal(run["o"], run["v"])
    for h in range(2):
        check_head(cfg, run, 0, h)


def test_dense_limit_matches_dense_attention(gpu):
    T, H, W = 2, 9, 11
    cfg = small_workload(T=T, H=H, W=W, heads=1, radius_override=math.hypot(H - 1, W - 1) + 0.01,
                         decay=1.0)
    _say("case: dense limit")
    run = gpu_run(cfg, gpu)
    assert run["plan"].info()["nnz"] == (T * 2 * 2) ** 2  # every tile pair listed
    q, k, v = (run[x][0, 0].double().cpu().numpy() for x in "qkv")
    ref = O.dense_attention(q, k, v)
    err = np.abs(run["o"][0, 0].double().cpu().numpy() - ref)
    _say("dense", err.max(), err.mean())
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_stats_match_oracle_counts(gpu):
    cfg = small_workload(T=3, H=13, W=21, heads=2, c=-0.5, budget_max=819.0)
    run = gpu_run(cfg, gpu)
    retained, listed = run["plan"].stats()
    exp = run["export"]
    R2 = O.radius_table(cfg.params(), cfg.T)
    ref = sum(int(O.retained_counts(exp["levels"][bh].astype(np.int64), R2, cfg.T, cfg.H, cfg.W,
                                    cfg.params()).sum()) for bh in range(cfg.heads))
    assert retained == ref
    tiles = O.Geometry(cfg.T, cfg.H, cfg.W, 8, 8)
    sizes = tiles.block_sizes()
    rp, ci = exp["row_ptr"], exp["col_idx"]
    ref_listed = sum(int(sizes[r % tiles.count]) * int(sizes[ci[e]])
                     for r in range(len(rp) - 1) for e in range(rp[r], rp[r + 1]))
    assert listed == ref_listed


def test_rebuild_equals_create(gpu):
    cfg = small_workload(T=3, H=13, W=21, heads=2, c=-0.5, budget_max=819.0)
    q, k, v = make_inputs(cfg, device=gpu)
    p1 = tra.plan(q, k, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
    q2, k2 = perturb(q, 2, 0, rel=0.5), perturb(k, 2, 1, rel=0.5)
    p1.rebuild(q2, k2)
    p2 = tra.plan(q2, k2, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
    e1, e2 = p1.export(), p2.export()
    for key in ("levels", "row_ptr", "col_idx", "kbar"):
        assert np.array_equal(e1[key], e2[key]), key


def test_plan_mismatch_rejected(gpu):
    cfg = small_workload(T=2, H=8, W=8, heads=1)
    q, k, v = make_inputs(cfg, device=gpu)
    plan = tra.plan(q, k, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
    q2 = torch.zeros((1, 2, cfg.N, 128), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(tra.TraError) as ei:
        tra.attention(q2, q2, q2, plan)
    assert ei.value.name == "TRA_ERR_PLAN_MISMATCH"


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times.  Every
# head runs on the GPU and, per workload:
#   - pooled keys and levels of every head against the oracle's (the oracle
#     runs per head in a pool of worker processes);
#   - every tile list of two heads against the vectorised reference lists;
#   - O of at least 2,000 queries of those two heads (one query in every tile
#     on the border of every frame, the rest random) against the oracle.
# ---------------------------------------------------------------------------
FULL_QUERIES = 2000


def check_full_size(cfg, run, pool, heads_o=None, rng_seed=11):
    exp = run["export"]
    check_csr_properties(cfg, run)
    assert torch.isfinite(run["o"].float()).all()
    excused = 0
    if cfg.radius_override < 0:
        plans = runner.head_plans(pool, cfg, run["q"], run["k"], range(cfg.heads))
        for h in range(cfg.heads):
            m = check_levels(cfg, exp, h, plans[h])
            excused += len(m["excused"])
        _say(cfg.name, "levels of all", cfg.heads, "heads equal outside", excused, "excused queries",
             f"({excused / (cfg.heads * cfg.N):.2e} of all)")
        assert excused <= 1e-3 * cfg.heads * cfg.N
    else:
        plans = {}
    rng = np.random.default_rng(rng_seed)
    for h in (heads_o if heads_o is not None else (0, cfg.heads - 1)):
        qs = ref_tiles.query_sample(cfg.T, cfg.H, cfg.W, FULL_QUERIES, rng)
        m = check_head(cfg, run, 0, h, query_sample=qs, oracle_plan=plans.get(h), tile_lists="reference",
                       pool=pool)
        _say(cfg.name, "head", h, "tile rows", m["tile_rows_compared"], "queries", m["queries_compared"],
             "H err", m.get("entropy_max_abs_err"), "O", m["o_max_abs"], m["o_mean_abs"],
             "excused", m.get("excused", [])[:20], "mismatched", m.get("level_mismatch", []))
    return excused


@pytest.mark.parametrize("name", ["wan21_1p3b_480p", "wan21_14b_720p", "hunyuan_720p", "long_video_2x"])
def test_full_size_workload(gpu, oracle_pool, name):
    cfg = CONFIGS[name]
    _say("case: full size", name)
    run = gpu_run(cfg, gpu)
    check_full_size(cfg, run, oracle_pool)
    retained, listed = run["plan"].stats()
    _say(name, "density", retained / (cfg.heads * cfg.N ** 2), "tile efficiency", retained / listed)


def test_plan_reuse_path(gpu, oracle_pool):
    """Plan from call 1 reused for calls 2..4 with 1% perturbed Q and K: O of
    2,000+ queries of two heads per call against the oracle under the plan."""
    cfg = CONFIGS["wan21_14b_720p"]
    _say("case: reuse path")
    q, k, v = make_inputs(cfg, device=gpu)
    plan = tra.plan(q, k, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
    exp = plan.export()
    rng = np.random.default_rng(12)
    R2 = O.radius_table(cfg.params(), cfg.T)
    for call in range(2, 5):
        qc, kc = perturb(q, call, 0), perturb(k, call, 1)
        o = tra.attention(qc, kc, v, plan)
        torch.cuda.synchronize()
        for h in (int(rng.integers(cfg.heads // 2)), int(cfg.heads // 2 + rng.integers(cfg.heads // 2))):
            qs = ref_tiles.query_sample(cfg.T, cfg.H, cfg.W, FULL_QUERIES, rng)
            done, ref, _, _, _ = runner.attention_rows(oracle_pool, cfg, qc[0, h], kc[0, h], v[0, h], qs,
                                                       exp["levels"][h].astype(np.int64), R2)
            err = np.abs(o[0, h].double().cpu().numpy()[qs] - ref)
            _say("call", call, "head", h, "queries", len(qs), err.max(), err.mean())
            assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_plan_drift(gpu):
    """Drift of a plan against new (Q, K): zero for its own inputs; for perturbed
    inputs, the same count as a fresh plan's levels give, and the oracle's count
    up to queries that sit within the excuse band of a level boundary."""
    cfg = small_workload(T=3, H=13, W=21, heads=2, c=-0.5, budget_max=819.0)
    q, k, v = make_inputs(cfg, device=gpu)
    plan = tra.plan(q, k, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
    assert plan.drift(q, k) == 0
    q2, k2 = perturb(q, 3, 0, rel=0.2), perturb(k, 3, 1, rel=0.2)
    n = plan.drift(q2, k2)
    lv1 = plan.export()["levels"].astype(np.int64)
    lv2 = tra.plan(q2, k2, grid=(cfg.T, cfg.H, cfg.W), **cfg.params()).export()["levels"].astype(np.int64)
    assert n == int((lv1 != lv2).sum())
    p = cfg.params()
    pools = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w)
    ref, slack = 0, 0
    for h in range(cfg.heads):
        lv_o, exc = [], set()
        for qq, kk in ((q, k), (q2, k2)):
            qh, kh = qq[0, h].double().cpu().numpy(), kk[0, h].double().cpu().numpy()
            Hh = O.entropy(qh, O.pool_keys(kh, pools, cfg.dtype), pools.block_sizes())
            lv_o.append(O.levels(Hh, p))
            exc |= set(O.excused_queries(Hh, p).tolist())
        ref += int((lv_o[0] != lv_o[1]).sum())
        slack += len(exc)
    _say("drift", n, "oracle", ref, "excused", slack, "of", cfg.heads * cfg.N)
    assert n > 0
    assert abs(n - ref) <= slack


# ---------------------------------------------------------------------------
# Alternative plan generators on the same kernels
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gen,r,dtype", [(1, 5.0, "bf16"), (1, 11.0, "bf16"), (2, 6.0, "bf16"), (2, 13.0, "bf16"),
                                         (1, 4.0, "fp32"), (2, 5.0, "fp32"), (3, -1.0, "bf16"), (3, 40.0, "bf16"),
                                         (3, -1.0, "fp32")])
def test_generator_small_full_parity(gpu, gen, r, dtype):
    extra = dict(c=-2.0, budget_max=600.0) if gen == 3 else {}  # 1-D windows of a few rows
    cfg = small_workload(T=4, H=13, W=21, heads=2, radius_override=r, generator=gen, dtype=dtype,
                         head_dim=128 if dtype == "bf16" else 64, **extra)
    _say("case: generator", gen, "radius", r, dtype)
    run = gpu_run(cfg, gpu)
    R2 = O.radius_table(cfg.params(), cfg.T)
    for h in range(cfg.heads):
        if dtype == "bf16":
            check_group_lists(cfg, run, h)
        m = check_head(cfg, run, 0, h)
        _say("head", h, "O", m["o_max_abs"], m["o_mean_abs"])
    retained, listed = run["plan"].stats()
    exp = run["export"]
    assert retained == sum(int(O.retained_counts(exp["levels"][h].astype(np.int64), R2, cfg.T, cfg.H, cfg.W,
                                                 cfg.params()).sum()) for h in range(cfg.heads))


@pytest.mark.parametrize("gen,r", [(1, 24.0), (2, 40.0), (3, -1.0)])
def test_generator_full_size(gpu, oracle_pool, gen, r):
    base = CONFIGS["wan21_14b_720p"]
    from dataclasses import replace
    cfg = replace(base, radius_override=r, generator=gen)
    _say("case: generator full size", gen, r)
    run = gpu_run(cfg, gpu)
    check_full_size(cfg, run, oracle_pool, rng_seed=41)
    retained, listed = run["plan"].stats()
    _say("density", retained / (cfg.heads * cfg.N ** 2), "tile efficiency", retained / listed)


# ---------------------------------------------------------------------------
# Token voting with a threshold; block-only masks
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("theta,block,dtype,d", [(4, 0, "bf16", 128), (40, 0, "bf16", 128), (1, 1, "bf16", 128),
                                                 (8, 1, "bf16", 128), (300, 1, "bf16", 128), (6, 0, "fp32", 64),
                                                 (1, 1, "fp32", 64), (20, 1, "fp32", 64), (6, 0, "fp32", 128),
                                                 (20, 1, "fp32", 128)])
def test_vote_threshold_and_block_mask_small(gpu, theta, block, dtype, d):
    cfg = small_workload(T=3, H=13, W=21, heads=2, c=-0.5, budget_max=819.0, vote_threshold=theta,
                         block_mask=block, dtype=dtype, head_dim=d)
    _say("case: votes", theta, "block", block, dtype, "d", d)
    run = gpu_run(cfg, gpu)
    for h in range(cfg.heads):
        err = check_listed(cfg, run, h, bool(block))
        _say("head", h, "O", err.max(), err.mean())
    retained, listed = run["plan"].stats()
    p = cfg.params()
    R2 = O.radius_table(p, cfg.T)
    tiles = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.tile_h, cfg.tile_w)
    if block:
        assert retained == listed
    else:
        ref = 0
        for h in range(cfg.heads):
            lv = run["export"]["levels"][h].astype(np.int64)
            for a in range(tiles.count):
                ref += sum(n for n in O.tile_votes(a, lv, R2, tiles, p).values() if n >= theta)
        assert retained == ref


@pytest.mark.parametrize("theta,block", [(64, 1), (256, 0)])
def test_vote_threshold_full_size_sampled(gpu, theta, block):
    from dataclasses import replace
    cfg = replace(CONFIGS["wan21_14b_720p"], vote_threshold=theta, block_mask=block)
    _say("case: votes full size", theta, block)
    run = gpu_run(cfg, gpu)
    check_csr_properties(cfg, run)
    rng = np.random.default_rng(51)
    tiles = O.Geometry(cfg.T, cfg.H, cfg.W, 8, 8)
    for h in (0, cfg.heads - 1):
        ts = np.concatenate([rng.choice(tiles.count, size=6, replace=False), [0, tiles.count - 1]])
        qs = np.concatenate([rng.choice(cfg.N, size=16, replace=False), [0, cfg.N - 1]])
        err = check_listed(cfg, run, h, bool(block), tile_sample=ts, query_sample=qs)
        _say("head", h, "O", err.max(), err.mean())
    retained, listed = run["plan"].stats()
    _say("pairs", retained, "listed", listed, "density", retained / (cfg.heads * cfg.N ** 2))


# ---------------------------------------------------------------------------
# Exact key sets.  With Q = 0 every retained key weighs the same, so row n of
# O is the mean of V over the keys query n retains.  V encodes each key j in
# two 64-wide one-hot blocks, e_(j % 64) + e_(64 + j // 64) (N <= 4096), so
# O[n] * |S_n| is the integer histogram of the key set's residues and 64-blocks
# (every count <= 64).  The probabilities are exactly 1 and their sums exact,
# so the only rounding is the bf16 output's (8-bit significand, relative error
# <= 2^-8): O[n] * |S_n| stays within 64 * 2^-8 = 0.25 of each count and
# rint() recovers it exactly.  A missing, extra or displaced key changes two
# counts by one.  A second V encodes the keys through a random permutation,
# so that two different key sets with equal histograms under one encoding are
# told apart by the other.
# ---------------------------------------------------------------------------
KEYSET_CASES = [
    # (T, H, W, generator, radius): static radii up to production size (the
    # 30 x 45 frame is ragged in both directions: 4 x 6 tiles, the last of each
    # row and column cut)
    (4, 13, 21, 0, 4.5), (3, 30, 45, 0, 12.5), (3, 30, 45, 0, 40.0),
    (4, 13, 21, 1, 5.0), (3, 30, 45, 1, 24.0),
    (4, 13, 21, 2, 7.0), (3, 30, 45, 2, 40.0),
    (4, 13, 21, 3, 3.0), (4, 13, 21, 3, 9.0), (3, 30, 45, 3, 50.0), (3, 30, 45, 3, 700.0),
]


@pytest.mark.parametrize("case", KEYSET_CASES)
def test_key_sets_exact(gpu, case):
    """Every query's key set, exactly, for fixed radii of every generator."""
    T, H, W, gen, r = case
    cfg = small_workload(T=T, H=H, W=W, heads=1, radius_override=r, generator=gen)
    _say("case: key sets", case)
    q = torch.zeros((1, 1, cfg.N, 128), dtype=torch.bfloat16, device=gpu)
    plan = tra.plan(q, q, grid=(T, H, W), **cfg.params())
    lv = np.full(cfg.N, -1, dtype=np.int64)
    largest, worst = check_key_sets(cfg, plan, lv, gpu, seed=5)
    _say("largest key set", largest, "worst distance from an integer count", worst)


@pytest.mark.parametrize("T,H,W,gen", [(3, 30, 45, 0), (4, 13, 21, 0), (3, 30, 45, 3)])
def test_key_sets_exact_mixed_levels(gpu, T, H, W, gen):
    """Every query's key set, exactly, when neighbouring queries hold unrelated
    budget levels (each query tile then mixes small and large disks).  The
    plan takes its levels from chosen per-query entropies, spread over the
    whole budget range [16, N]."""
    N = T * H * W
    cfg = small_workload(T=T, H=H, W=W, heads=1, generator=gen, budget_min=16.0, budget_max=float(N),
                         c=0.0, decay=0.5)
    p = cfg.params()
    rng = np.random.default_rng(7 + gen)
    Hq = rng.uniform(math.log(16.0) - 0.5, math.log(N) + 0.5, size=N).astype(np.float32)
    _say("case: key sets, mixed levels", (T, H, W), "generator", gen)
    ent = torch.from_numpy(Hq).reshape(1, 1, N).to(gpu)
    plan = tra.plan_from_entropy(ent, grid=(T, H, W), head_dim=128, dtype=torch.bfloat16, **p)
    lv = plan.export()["levels"][0].astype(np.int64)
    assert np.array_equal(lv, O.levels(Hq.astype(np.float64), p))
    k_lo, k_hi = O.level_range(p)
    assert len(np.unique(lv)) > (k_hi - k_lo) // 2  # many distinct levels
    largest, worst = check_key_sets(cfg, plan, lv, gpu, seed=9)
    _say("levels", k_lo, "..", k_hi, "largest key set", largest, "worst distance from an integer count", worst)
