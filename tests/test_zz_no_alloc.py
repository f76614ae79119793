"""tra_plan_drift_noalloc (static scratch, no allocation) against
tra_plan_drift (the plan's scratch), through the C ABI, on two calls in a row,
the second on a smaller plan; and the size limit."""
import pytest
import torch

import sparse_self_attention_amd as tra
from workloads import make_inputs, perturb, small_workload

pytestmark = pytest.mark.gpu


def test_drift_noalloc_matches_drift(gpu):
    assert tra.drift_noalloc_max_bytes() == 32 << 20
    for cfg in (small_workload(T=4, H=30, W=45, heads=3, c=-0.5, budget_max=5400.0),
                small_workload(T=2, H=13, W=21, heads=2, c=-0.5, budget_max=546.0)):
        q, k, v = make_inputs(cfg, device=gpu)
        plan = tra.plan(q, k, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
        assert plan.drift_noalloc(q, k) == 0 == plan.drift(q, k)
        for rel in (0.05, 0.3):
            q2, k2 = perturb(q, 4, 0, rel=rel), perturb(k, 4, 1, rel=rel)
            a = plan.drift_noalloc(q2, k2)
            b = plan.drift(q2, k2)
            print(cfg.name, "rel", rel, "drift", a, b, flush=True)
            assert a == b and a > 0
        assert plan.drift_noalloc(q, k) == 0


def test_drift_noalloc_rejects_plans_beyond_its_scratch(gpu):
    # 320 heads x 65,536 queries: the levels alone take 40 MiB
    cfg = small_workload(T=4, H=128, W=128, heads=320, head_dim=64, c=-3.0, budget_max=512.0)
    g = torch.Generator(device=gpu).manual_seed(3)
    q = torch.randn((1, cfg.heads, cfg.N, 64), generator=g, device=gpu).to(torch.bfloat16)
    k = torch.randn((1, cfg.heads, cfg.N, 64), generator=g, device=gpu).to(torch.bfloat16)
    plan = tra.plan(q, k, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
    with pytest.raises(tra.TraError) as ei:
        plan.drift_noalloc(q, k)
    assert ei.value.name == "TRA_ERR_SHAPE"
    assert "static buffer" in str(ei.value)
    assert plan.drift(q, k) == 0  # the plan's own scratch still works
