"""Query regrouping by level (the `regroup` plan option, bf16): the attention
kernel deals each 2 x 2 group's queries to its waves in level order instead of
as spatial half tiles.  The retained keys and the tile lists do not change, so
everything is held to the same oracle as the spatial layout: exact key sets
when neighbouring queries hold unrelated levels, full parity on small ragged
grids of every generator, and the Wan2.1-14B shape at full size (sampled)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import ref_tiles
import sparse_self_attention_amd as tra
from parity_util import check_head, check_key_sets, gpu_run
from workloads import CONFIGS, small_workload

pytestmark = pytest.mark.gpu

FULL_QUERIES = 2000


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("T,H,W,gen", [(3, 30, 45, 0), (4, 13, 21, 0), (3, 30, 45, 3)])
def test_regroup_key_sets_exact_mixed_levels(gpu, T, H, W, gen):
    """Each query's key set, exactly, with levels spread over the whole budget
    range, so that every group's level order is far from its raster order."""
    N = T * H * W
    cfg = small_workload(T=T, H=H, W=W, heads=1, generator=gen, budget_min=16.0, budget_max=float(N),
                         c=0.0, decay=0.5, regroup=1)
    p = cfg.params()
    rng = np.random.default_rng(17 + gen)
    Hq = rng.uniform(math.log(16.0) - 0.5, math.log(N) + 0.5, size=N).astype(np.float32)
    _say("case: regrouped key sets", (T, H, W), "generator", gen)
    ent = torch.from_numpy(Hq).reshape(1, 1, N).to(gpu)
    plan = tra.plan_from_entropy(ent, grid=(T, H, W), head_dim=128, dtype=torch.bfloat16, **p)
    lv = plan.export()["levels"][0].astype(np.int64)
    assert np.array_equal(lv, O.levels(Hq.astype(np.float64), p))
    largest, worst = check_key_sets(cfg, plan, lv, gpu, seed=19)
    _say("largest key set", largest, "worst distance from an integer count", worst)


@pytest.mark.parametrize("kw", [
    dict(T=3, H=13, W=21),
    dict(T=2, H=17, W=9, head_dim=64),
    dict(T=4, H=8, W=8),
    dict(T=4, H=13, W=21, generator=1, radius_override=5.0),
    dict(T=4, H=13, W=21, generator=2, radius_override=7.0),
    dict(T=4, H=13, W=21, generator=3, c=-2.0, budget_max=600.0),
])
def test_regroup_small_full_parity(gpu, kw):
    """Every output against the oracle; the same pair counts, levels and tile
    lists as the spatial layout, and outputs within rounding of it."""
    kw = dict(kw)
    base = dict(heads=2, c=-0.5, budget_max=float(kw["T"] * kw["H"] * kw["W"]))
    base.update(kw)
    cfg = small_workload(regroup=1, **base)
    _say("case: regroup small", kw)
    run = gpu_run(cfg, gpu)
    spatial = tra.plan(run["q"], run["k"], grid=(cfg.T, cfg.H, cfg.W), **dict(cfg.params(), regroup=0))
    o_sp = tra.attention(run["q"], run["k"], run["v"], spatial)
    torch.cuda.synchronize()
    e_sp = spatial.export()
    for key in ("levels", "row_ptr", "col_idx"):
        assert np.array_equal(run["export"][key], e_sp[key]), key
    assert run["plan"].stats() == spatial.stats()
    _check_order(cfg, run["plan"])
    for h in range(cfg.heads):
        m = check_head(cfg, run, 0, h)
        _say("head", h, "O", m["o_max_abs"], m["o_mean_abs"])
    d = (run["o"].float() - o_sp.float()).abs()
    _say("against the spatial layout", float(d.max()), float(d.mean()))
    # Each query's online softmax does not depend on the other queries of its
    # wave (a reference move leaves the lanes it does not raise unchanged, and
    # a block a query keeps no key of adds exact zeros), so the outputs are
    # the spatial layout's bit for bit.
    assert torch.equal(run["o"], o_sp)


def _check_order(cfg, plan):
    """The exported order is, for every group, its slots sorted by (level,
    slot) with the positions outside the grid last, computed here from the
    exported levels."""
    perm = plan.export_regroup()
    lv = plan.export()["levels"].astype(np.int64).reshape(-1, cfg.T, cfg.H, cfg.W)
    ngh, ngw = -(-cfg.H // 16), -(-cfg.W // 16)
    assert perm.shape == (lv.shape[0] * cfg.T * ngh * ngw, 256)
    slot = np.arange(256)
    g = 0
    for bh in range(lv.shape[0]):
        for t in range(cfg.T):
            for gr in range(ngh):
                for gc in range(ngw):
                    h, w = 16 * gr + slot // 16, 16 * gc + slot % 16
                    inside = (h < cfg.H) & (w < cfg.W)
                    key = np.full(256, 1 << 20, dtype=np.int64)
                    key[inside] = lv[bh, t, h[inside], w[inside]] + 32768
                    want = np.lexsort((slot, key))
                    assert np.array_equal(perm[g], want), f"group {g}"
                    g += 1


def test_regroup_follows_rebuild_and_import(gpu):
    """A rebuild on other inputs re-sorts every group; an imported plan holds
    the same order and attends bit for bit like the exported one."""
    from workloads import make_inputs, perturb
    cfg = small_workload(T=3, H=30, W=45, heads=2, c=-0.5, budget_max=4050.0, regroup=1)
    _say("case: regroup rebuild and import")
    q, k, v = make_inputs(cfg, device=gpu)
    grid = (cfg.T, cfg.H, cfg.W)
    plan = tra.plan(q, k, grid=grid, **cfg.params())
    first = plan.export_regroup()
    q2, k2 = perturb(q, 2, 0, rel=0.5), perturb(k, 2, 1, rel=0.5)
    plan.rebuild(q2, k2)
    _check_order(cfg, plan)
    fresh = tra.plan(q2, k2, grid=grid, **cfg.params())
    assert np.array_equal(plan.export_regroup(), fresh.export_regroup())
    saved = plan.export()
    back = tra.import_plan(saved, 1, cfg.heads, grid, cfg.head_dim, device=gpu, **cfg.params())
    assert np.array_equal(back.export_regroup(), plan.export_regroup())
    o1, o2 = tra.attention(q2, k2, v, plan), tra.attention(q2, k2, v, back)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    _say("groups re-sorted by the rebuild:", int(np.sum(np.any(first != plan.export_regroup(), axis=1))),
         "of", len(first))


def test_regroup_rejected_with_block_masks(gpu):
    cfg = small_workload(T=3, H=13, W=21, heads=1, regroup=1, block_mask=1)
    q = torch.zeros((1, 1, cfg.N, 128), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(tra.TraError):
        tra.plan(q, q, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())


def test_regroup_full_size(gpu, oracle_pool):
    """Wan2.1-14B 720p regrouped: the levels and every tile list of two heads
    against the oracle, and O of 2,000+ queries of each of those heads."""
    cfg = CONFIGS["wan21_14b_720p"].with_(regroup=1)
    _say("case: regroup full size")
    run = gpu_run(cfg, gpu)
    perm = run["plan"].export_regroup()
    assert all(np.array_equal(np.sort(row), np.arange(256)) for row in perm[:: max(1, len(perm) // 500)])
    rng = np.random.default_rng(23)
    for h in (0, cfg.heads - 1):
        qs = ref_tiles.query_sample(cfg.T, cfg.H, cfg.W, FULL_QUERIES, rng)
        m = check_head(cfg, run, 0, h, query_sample=qs, tile_lists="reference", pool=oracle_pool)
        _say("head", h, "queries", m["queries_compared"], "O", m["o_max_abs"], m["o_mean_abs"])
