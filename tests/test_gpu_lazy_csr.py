"""bf16 plans build only their group lists; the CSR is completed on the first
export, stats or info call after each build.  These tests check that the
completed CSR always belongs to the latest build, also when the build ran on
another stream than the call that completes it."""
import numpy as np
import pytest
import torch

import sparse_self_attention_amd as tra
from workloads import make_inputs, perturb, small_workload

pytestmark = pytest.mark.gpu


def _csr(plan):
    e = plan.export()
    return e["levels"], e["row_ptr"], e["col_idx"]


@pytest.mark.parametrize("kw", [dict(), dict(generator=3, radius_override=30.0), dict(generator=1, radius_override=6.0)])
def test_csr_follows_the_latest_build(gpu, kw):
    cfg = small_workload(T=3, H=13, W=21, heads=2, **kw)
    print("case: lazy csr", kw, flush=True)
    grid = (cfg.T, cfg.H, cfg.W)
    q, k, v = make_inputs(cfg, device=gpu)
    q2, k2 = perturb(q, 2, 0, rel=0.5), perturb(k, 2, 1, rel=0.5)
    plan = tra.plan(q, k, grid=grid, **cfg.params())
    first = _csr(plan)
    stats1 = plan.stats()
    plan.rebuild(q2, k2)
    fresh = tra.plan(q2, k2, grid=grid, **cfg.params())
    # info first (completes the CSR on the null stream), then export and stats
    assert plan.info()["nnz"] == fresh.info()["nnz"]
    for a, b in zip(_csr(plan), _csr(fresh)):
        assert np.array_equal(a, b)
    assert plan.stats() == fresh.stats()
    # and back: the rebuild from the first inputs gives the first CSR again
    plan.rebuild(q, k)
    for a, b in zip(_csr(plan), first):
        assert np.array_equal(a, b)
    assert plan.stats() == stats1


def test_csr_completed_on_another_stream(gpu):
    """Build on a side stream, complete the CSR from the default stream."""
    cfg = small_workload(T=4, H=17, W=23, heads=2)
    grid = (cfg.T, cfg.H, cfg.W)
    q, k, v = make_inputs(cfg, device=gpu)
    ref = tra.plan(q, k, grid=grid, **cfg.params())
    want = _csr(ref)
    side = torch.cuda.Stream(device=gpu)  # default priority
    side.wait_stream(torch.cuda.current_stream(gpu))  # the inputs are written on the default stream
    with torch.cuda.stream(side):
        plan = tra.plan(q, k, grid=grid, **cfg.params())
        q2 = perturb(q, 3, 0, rel=0.5)
        plan.rebuild(q2, k)
        plan.rebuild(q, k)
    # no synchronisation here: export orders itself after the side stream's build
    got = tra.Plan.export(plan)
    for key, w in zip(("levels", "row_ptr", "col_idx"), want):
        assert np.array_equal(got[key], w), key
    torch.cuda.synchronize()
    o1 = tra.attention(q, k, v, ref)
    o2 = tra.attention(q, k, v, plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_reuse_step_in_a_graph(gpu):
    """A bf16 plan rebuild has no host round trip, so the reuse step (rebuild +
    attention calls) can be captured in a graph.  Every replay, with eager
    work in between, must match the eager step bit for bit."""
    cfg = small_workload(T=3, H=13, W=21, heads=2)
    grid = (cfg.T, cfg.H, cfg.W)
    q, k, v = make_inputs(cfg, device=gpu)
    q2, k2 = perturb(q, 2, 0, rel=0.3), perturb(k, 2, 1, rel=0.3)
    plan = tra.plan(q, k, grid=grid, **cfg.params())
    o1, o2 = torch.empty_like(q), torch.empty_like(q)

    def step(qa, ka):
        plan.rebuild(qa, ka)
        tra.attention(q2, k2, v, plan, out=o1)
        tra.attention(q, k, v, plan, out=o2)

    step(q, k)
    torch.cuda.synchronize()
    want = (o1.clone(), o2.clone())
    side = torch.cuda.Stream(device=gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(side):  # warm-up on the capture stream
        step(q, k)
    torch.cuda.current_stream(gpu).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q, k)
    for rep in range(3):
        o1.zero_()
        o2.zero_()
        step(q2, k2)  # eager work with other inputs between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, want[0]) and torch.equal(o2, want[1]), f"replay {rep}"
        e = plan.export()  # the CSR completed after a replay is the replayed build's
        ref = tra.plan(q, k, grid=grid, **cfg.params()).export()
        assert np.array_equal(e["col_idx"], ref["col_idx"]) and np.array_equal(e["levels"], ref["levels"])


@pytest.mark.parametrize("kw", [dict(), dict(vote_threshold=4), dict(dtype="fp32", head_dim=64), dict(regroup=1)])
def test_host_copies_follow_a_build_on_another_stream(gpu, kw):
    """Every call that copies plan data to the host orders itself after the
    plan's latest build, also when that build ran on another stream and the
    caller does not synchronise: levels, pooled keys, CSR, group lists, the
    regroup order and the pair counts equal a plan built from those inputs."""
    cfg = small_workload(T=3, H=13, W=21, heads=2, **kw)
    grid = (cfg.T, cfg.H, cfg.W)
    print("case: host copies after a side-stream build", kw, flush=True)
    q, k, v = make_inputs(cfg, device=gpu)
    q2, k2 = perturb(q, 2, 0, rel=0.5), perturb(k, 2, 1, rel=0.5)
    plan = tra.plan(q, k, grid=grid, **cfg.params())
    want = tra.plan(q2, k2, grid=grid, **cfg.params())
    e_want, s_want = want.export(), want.stats()
    g_want = want.export_groups() if cfg.dtype == "bf16" else None
    r_want = want.export_regroup() if cfg.regroup else None
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=gpu)  # default priority
    side.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(side):
        plan.rebuild(q2, k2)
    # no synchronisation: each host copy below orders itself after the rebuild
    if cfg.regroup:
        assert np.array_equal(tra.Plan.export_regroup(plan), r_want)
    if g_want is not None:
        for a, b in zip(tra.Plan.export_groups(plan), g_want):
            assert np.array_equal(a, b)
    got = tra.Plan.export(plan)
    for key in ("levels", "kbar", "row_ptr", "col_idx"):
        assert np.array_equal(got[key], e_want[key]), key
    assert tra.Plan.stats(plan) == s_want
    torch.cuda.synchronize()
