"""Attention groups of 3 x 2 query tiles (the `group_rows` plan option, bf16).

The attention kernel's unit of work is a group of query tiles of one frame that
loads each key tile of its merged list once.  With three query-tile rows per
group a workgroup has 12 waves, three per SIMD.  A query's online softmax sees
the same 32-key blocks in the same order whatever group holds it (key tiles no
tile of its wave lists are skipped), so the outputs equal those of 2 x 2 groups
bit for bit.  Checked here on small ragged grids of every generator and plan
variant: the group lists against the union of their members' CSR rows, the
outputs against 2 x 2 groups and against the oracle; and the automatic
choice."""
import numpy as np
import pytest
import torch

import sparse_self_attention_amd as tra
from parity_util import check_group_lists, check_head, check_listed, gpu_run
from workloads import small_workload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("kw", [
    dict(T=3, H=13, W=21),                      # two tile rows: the second group row is empty
    dict(T=2, H=17, W=9, head_dim=64),          # three ragged tile rows, one ragged tile column
    dict(T=4, H=8, W=8),                        # a single query tile per frame
    dict(T=3, H=45, W=40),                      # six tile rows, the last one ragged
    dict(T=2, H=40, W=37),                      # five tile rows, four tile columns (the last ragged)
    dict(T=4, H=13, W=21, generator=1, radius_override=5.0),
    dict(T=4, H=13, W=21, generator=2, radius_override=7.0),
    dict(T=4, H=25, W=21, generator=3, c=-2.0, budget_max=600.0),
    dict(T=4, H=25, W=21, vote_threshold=4),
    dict(T=4, H=25, W=21, block_mask=1),
])
def test_group_rows_small_parity(gpu, kw):
    kw = dict(kw)
    base = dict(heads=2, c=-0.5, budget_max=float(kw["T"] * kw["H"] * kw["W"]))
    base.update(kw)
    cfg = small_workload(group_rows=3, **base)
    _say("case: 3 x 2 groups", kw)
    run = gpu_run(cfg, gpu)
    assert run["plan"].info()["group_rows"] == 3
    two = tra.plan(run["q"], run["k"], grid=(cfg.T, cfg.H, cfg.W), **dict(cfg.params(), group_rows=2))
    assert two.info()["group_rows"] == 2
    o2 = tra.attention(run["q"], run["k"], run["v"], two)
    torch.cuda.synchronize()
    e2 = two.export()
    for key in ("levels", "row_ptr", "col_idx"):
        assert np.array_equal(run["export"][key], e2[key]), key
    assert run["plan"].stats() == two.stats()
    n = sum(check_group_lists(cfg, run, bh) for bh in range(cfg.heads))
    _say("groups checked", n)
    assert torch.equal(run["o"], o2), float((run["o"].float() - o2.float()).abs().max())
    for h in range(cfg.heads):
        if cfg.vote_threshold > 1 or cfg.block_mask:
            err = check_listed(cfg, run, h, bool(cfg.block_mask))
            _say("head", h, "O", err.max(), err.mean())
        else:
            m = check_head(cfg, run, 0, h)
            _say("head", h, "O", m["o_max_abs"], m["o_mean_abs"])


@pytest.mark.parametrize("H,extra,want", [
    (45, {}, 3),                                  # 6 tile rows: two full groups of 3
    (17, {}, 3),                                  # 3 tile rows
    (40, {}, 3),                                  # 5 tile rows: one empty row either way
    (30, {}, 2),                                  # 4 tile rows: groups of 3 would leave 2 empty
    (13, {}, 2),                                  # 2 tile rows
    (45, dict(regroup=1), 2),                     # regrouping orders 2 x 2 groups
    (45, dict(generator=3), 2),                   # the 1-D window keeps 2 x 2 groups
    (45, dict(group_rows=2), 2),
    (30, dict(group_rows=3), 3),
])
def test_group_rows_choice(gpu, H, extra, want):
    T, W = 2, 24
    N = T * H * W
    p = small_workload(T=T, H=H, W=W, heads=1, budget_max=float(N), **extra).params()
    _say("case: group rows", H, extra)
    ent = torch.full((1, 1, N), 3.0, dtype=torch.float32, device=gpu)
    plan = tra.plan_from_entropy(ent, grid=(T, H, W), head_dim=128, dtype=torch.bfloat16, **p)
    assert plan.info()["group_rows"] == want
    gptr, _, _ = plan.export_groups()
    nh, nw = -(-H // 8), -(-W // 8)
    assert len(gptr) == T * -(-nh // want) * -(-nw // 2)
