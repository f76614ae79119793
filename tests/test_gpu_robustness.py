"""Error paths of the library on the GPU, forced from the host: injected
allocation and launch failures (TRA_FAULT) at every allocation and launch of a
plan build, a plan whose rebuild failed, and stats/drift calls that allocate
nothing per call.  No kernel faults: an injected launch failure means the
kernel is never launched."""
import numpy as np
import pytest
import torch

import sparse_self_attention_amd as tra
from workloads import make_inputs, perturb, small_workload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture
def case(gpu):
    cfg = small_workload(T=3, H=13, W=21, heads=2, c=-0.5, budget_max=819.0)
    q, k, v = make_inputs(cfg, device=gpu)
    return cfg, q, k, v


def _count_until_clean(make, kind):
    """Injects a failure at the 1st, 2nd, ... allocation or launch of make()
    until a run completes without reaching the injection point; every injected
    run must raise TraError with the distinct status and leave nothing."""
    n = 1
    while True:
        import os
        os.environ["TRA_FAULT"] = f"{kind}:{n}"
        try:
            obj = make()
        except tra.TraError as e:
            assert e.name == ("TRA_ERR_OOM" if kind == "alloc" else "TRA_ERR_HIP"), e
            n += 1
            continue
        finally:
            del os.environ["TRA_FAULT"]
        return n - 1, obj


@pytest.mark.parametrize("kind", ["alloc", "launch"])
def test_injected_failures_in_plan_create(case, kind):
    cfg, q, k, v = case
    grid = (cfg.T, cfg.H, cfg.W)
    ref = tra.plan(q, k, grid=grid, **cfg.params())
    b = ref.export()
    o_ref = tra.attention(q, k, v, ref)
    free = []
    for rnd in range(3):
        failed, plan = _count_until_clean(lambda: tra.plan(q, k, grid=grid, **cfg.params()), kind)
        if rnd == 0:
            _say(kind, "failures injected and reported:", failed)
            # (a bf16 build launches pooling, entropy, and runs with the group lists)
            assert failed >= (10 if kind == "alloc" else 3)
            a = plan.export()
            for key in ("levels", "row_ptr", "col_idx"):
                assert np.array_equal(a[key], b[key])
            assert torch.equal(tra.attention(q, k, v, plan), o_ref)
        plan.destroy()
        torch.cuda.synchronize()
        free.append(torch.cuda.mem_get_info()[0])
    _say("free device memory after each round of injected failures:", free)
    # Failed creates release what they allocated: after the first round (the
    # runtime's allocator may keep blocks it grew), free memory holds steady.
    assert free[2] >= free[1] - (4 << 20)


def test_failed_rebuild_invalidates_the_plan(case):
    import os
    cfg, q, k, v = case
    grid = (cfg.T, cfg.H, cfg.W)
    plan = tra.plan(q, k, grid=grid, **cfg.params())
    o_ref = tra.attention(q, k, v, plan)
    q2, k2 = perturb(q, 2, 0, rel=0.3), perturb(k, 2, 1, rel=0.3)
    for at in (1, 2, 3):  # of the rebuild's three launches (pooling, entropy, runs with the group lists)
        os.environ["TRA_FAULT"] = f"launch:{at}"
        try:
            with pytest.raises(tra.TraError) as ei:
                plan.rebuild(q2, k2)
            assert ei.value.name == "TRA_ERR_HIP"
        finally:
            del os.environ["TRA_FAULT"]
        for call in (lambda: tra.attention(q, k, v, plan), plan.export, plan.stats,
                     lambda: plan.drift(q, k), plan.export_groups):
            with pytest.raises(tra.TraError) as ei:
                call()
            assert ei.value.name == "TRA_ERR_PLAN_INVALID"
    plan.rebuild(q, k)  # a successful rebuild makes it usable again
    assert torch.equal(tra.attention(q, k, v, plan), o_ref)


def test_stats_and_drift_reuse_plan_scratch(case):
    cfg, q, k, v = case
    grid = (cfg.T, cfg.H, cfg.W)
    plan = tra.plan(q, k, grid=grid, **cfg.params())
    s1 = plan.stats()
    q2, k2 = perturb(q, 3, 0, rel=0.2), perturb(k, 3, 1, rel=0.2)
    d1 = plan.drift(q2, k2)
    assert plan.drift(q, k) == 0
    for _ in range(3):
        assert plan.stats() == s1
        assert plan.drift(q2, k2) == d1
    lv1 = plan.export()["levels"].astype(np.int64)
    lv2 = tra.plan(q2, k2, grid=grid, **cfg.params()).export()["levels"].astype(np.int64)
    assert d1 == int((lv1 != lv2).sum()) and d1 > 0
