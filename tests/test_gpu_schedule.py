"""GPU checks of the reuse schedule across denoising steps (dense warm-up,
re-plan from exact entropies, sparse reuse, refresh and drift tracking),
step by step against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_self_attention_amd as tra
from workloads import make_inputs, perturb, small_workload

from parity_util import MAX_ABS, MEAN_ABS

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _np(x, h):
    return x[0, h].double().cpu().numpy()


def test_schedule_modes_and_outputs(gpu):
    cfg = small_workload(T=3, H=13, W=21, heads=2, c=-0.5, budget_max=819.0)
    p = cfg.params()
    grid = (cfg.T, cfg.H, cfg.W)
    q0, k0, v = make_inputs(cfg, device=gpu)
    sched = tra.Schedule(q0, grid, warmup_steps=2, refresh_every=2, **p)
    assert sched.plan() is None
    expected = ["dense", "dense_replan", "sparse", "sparse", "dense_replan", "sparse"]
    R2 = O.radius_table(p, cfg.T)
    plan_levels = None
    for step, mode in enumerate(expected):
        q, k = perturb(q0, step + 2, 0, rel=0.1), perturb(k0, step + 2, 1, rel=0.1)
        o, info = sched.step(q, k, v)
        torch.cuda.synchronize()
        _say("step", step, info)
        assert info["step"] == step and info["mode"] == mode and info["drift"] == -1
        for h in range(cfg.heads):
            qh, kh, vh = _np(q, h), _np(k, h), _np(v, h)
            if mode.startswith("dense"):
                ref = O.dense_attention(qh, kh, vh)
            else:
                ref = O.attention_rows(qh, kh, vh, np.arange(cfg.N), plan_levels[h], R2, cfg.T, cfg.H, cfg.W, p)
            err = np.abs(_np(o, h) - ref)
            assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (step, h, err.max(), err.mean())
        if mode == "dense_replan":
            exp = sched.plan().export()
            plan_levels = exp["levels"].astype(np.int64)
            for h in range(cfg.heads):
                H_ref = O.dense_entropy(_np(q, h), _np(k, h))
                bad = np.nonzero(plan_levels[h] != O.levels(H_ref, p))[0]
                assert set(bad.tolist()) <= set(O.excused_queries(H_ref, p).tolist())
    sched.destroy()


def test_schedule_drift_triggers_refresh(gpu):
    cfg = small_workload(T=3, H=13, W=21, heads=2, c=-0.5, budget_max=819.0)
    p = cfg.params()
    grid = (cfg.T, cfg.H, cfg.W)
    qa, ka, v = make_inputs(cfg, device=gpu)
    qb, kb = perturb(qa, 9, 0, rel=1.0), perturb(ka, 9, 1, rel=1.0)  # far from A
    sched = tra.Schedule(qa, grid, warmup_steps=1, refresh_every=0, drift_threshold=0.01, **p)
    steps = [(qa, ka, "dense_replan"), (qa, ka, "sparse"), (qb, kb, "sparse"), (qb, kb, "dense_replan"),
             (qb, kb, "sparse")]
    pools = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w)

    def pooled(q, k, h):
        Hh = O.entropy(_np(q, h), O.pool_keys(_np(k, h), pools, cfg.dtype), pools.block_sizes())
        return O.levels(Hh, p), set(O.excused_queries(Hh, p).tolist())

    for step, (q, k, mode) in enumerate(steps):
        _, info = sched.step(q, k, v)
        torch.cuda.synchronize()
        _say("step", step, info)
        assert info["mode"] == mode
        if mode == "sparse":
            ref_q, ref_k = (qa, ka) if step < 3 else (qb, kb)
            ref, slack = 0, 0
            for h in range(cfg.heads):
                l0, e0 = pooled(ref_q, ref_k, h)
                l1, e1 = pooled(q, k, h)
                ref += int((l0 != l1).sum())
                slack += len(e0 | e1)
            assert abs(info["drift"] - ref) <= slack
            if step in (1, 4):
                assert info["drift"] == 0
            else:
                assert info["drift"] > 0.01 * cfg.heads * cfg.N
        else:
            assert info["drift"] == -1
    sched.destroy()
