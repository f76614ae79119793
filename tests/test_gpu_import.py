"""Checkpoint / resume of a plan (tra_plan_import): a plan exported and
imported with the same shape and params holds the same levels, tile lists and
group lists, and attends bit for bit like the original."""
import numpy as np
import pytest
import torch

import sparse_self_attention_amd as tra
from workloads import CONFIGS, make_inputs, small_workload

pytestmark = pytest.mark.gpu

_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _round_trip(cfg, gpu):
    print(f"case: import {cfg.name} gen={cfg.generator} r={cfg.radius_override} theta={cfg.vote_threshold}",
          flush=True)
    q, k, v = make_inputs(cfg, device=gpu)
    grid = (cfg.T, cfg.H, cfg.W)
    p1 = tra.plan(q, k, grid=grid, **cfg.params())
    e1 = p1.export()
    p2 = tra.import_plan(e1, q.shape[0], q.shape[1], grid, cfg.head_dim, dtype=_DT[cfg.dtype], device=gpu,
                         **cfg.params())
    e2 = p2.export()
    for key in ("levels", "entropy", "r2", "row_ptr", "col_idx", "kbar"):
        assert np.array_equal(e1[key], e2[key]), key
    if cfg.dtype == "bf16":
        for a, b in zip(p1.export_groups(), p2.export_groups()):  # gptr, glen, glist
            assert np.array_equal(a, b)
    o1 = tra.attention(q, k, v, p1)
    o2 = tra.attention(q, k, v, p2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert p1.stats() == p2.stats()
    return e1


@pytest.mark.parametrize("kw", [
    dict(T=3, H=13, W=21),
    dict(T=2, H=17, W=9, head_dim=64),
    dict(T=3, H=13, W=21, dtype="fp32"),
    dict(T=4, H=13, W=21, generator=1, radius_override=5.0),
    dict(T=4, H=13, W=21, generator=3, radius_override=40.0),
    dict(T=3, H=13, W=21, vote_threshold=6),
])
def test_import_round_trip_small(gpu, kw):
    _round_trip(small_workload(**kw), gpu)


def test_import_round_trip_full_size(gpu):
    """Wan2.1-14B 720p (40 heads, 75,600 tokens each)."""
    _round_trip(CONFIGS["wan21_14b_720p"], gpu)


def test_import_levels_only(gpu):
    """Without entropies and pooled keys the import still rebuilds the same
    tile lists; the stored entropies and pooled keys are zero."""
    cfg = small_workload(T=3, H=13, W=21)
    q, k, v = make_inputs(cfg, device=gpu)
    grid = (cfg.T, cfg.H, cfg.W)
    p1 = tra.plan(q, k, grid=grid, **cfg.params())
    e1 = p1.export()
    p2 = tra.import_plan({"levels": e1["levels"]}, q.shape[0], q.shape[1], grid, cfg.head_dim, device=gpu,
                         **cfg.params())
    e2 = p2.export()
    assert np.array_equal(e1["row_ptr"], e2["row_ptr"]) and np.array_equal(e1["col_idx"], e2["col_idx"])
    assert not e2["entropy"].any() and not e2["kbar"].any()
    assert torch.equal(tra.attention(q, k, v, p1), tra.attention(q, k, v, p2))
