"""Pooled-key entropy on inputs built to move the softmax reference.

The bf16 entropy kernel walks the pooled keys in 32-key chunks and keeps a
running reference (the largest score seen).  Here every query's scores rise
with the key frame (a new maximum in every chunk), fall with it (the maximum
in the first chunk), or spread over a very wide range.  The grid is ragged in
both directions, so chunks of one weight, chunks of mixed weights and a padded
last chunk all occur.  Levels, pooled keys, tile lists and O are compared with
the oracle as in the other parity tests, and the entropy itself within 2e-5
nat."""
import numpy as np
import pytest
import torch

from parity_util import check_head, gpu_run
from workloads import small_workload

pytestmark = pytest.mark.gpu


def _inputs(cfg, pattern, device):
    g = torch.Generator().manual_seed({"rising": 11, "falling": 12, "wide": 13}[pattern])
    T, N, d = cfg.T, cfg.T * cfg.H * cfg.W, cfg.head_dim
    u = torch.randn(d, generator=g)
    frame = torch.arange(N) // (cfg.H * cfg.W)
    if pattern == "rising":
        a = 0.2 + 0.4 * frame.float()
        s = torch.full((N, 1), 1.0)
    elif pattern == "falling":
        a = 0.2 + 0.4 * (T - 1 - frame).float()
        s = torch.full((N, 1), 1.0)
    else:
        a = 4.0 * torch.rand(N, generator=g) - 2.0
        s = torch.exp(3.0 * torch.rand((N, 1), generator=g))  # scores up to ~20x the others
    shape = (1, cfg.heads, N, d)
    k = a[:, None] * u + 0.3 * torch.randn(shape, generator=g)
    q = s * u + 0.3 * torch.randn(shape, generator=g)
    v = torch.randn(shape, generator=g)
    dt = torch.bfloat16
    return tuple(x.to(dt).to(device).contiguous() for x in (q, k, v))


@pytest.mark.parametrize("pattern", ["rising", "falling", "wide"])
def test_entropy_reference_moves(gpu, pattern):
    # 8 frames of 21 x 37 with 8 x 8 pools: 15 pooled keys per frame, 8 of
    # them full; 120 in all, four chunks, the last one padded.
    cfg = small_workload(T=8, H=21, W=37, heads=2, c=-0.5, budget_max=float(8 * 21 * 37))
    print("case: entropy stress", pattern, flush=True)
    run = gpu_run(cfg, gpu, inputs=_inputs(cfg, pattern, gpu))
    for h in range(cfg.heads):
        queries = np.random.default_rng(h).choice(cfg.N, 400, replace=False)
        m = check_head(cfg, run, 0, h, query_sample=queries, tile_lists="reference")
        print("head", h, "entropy err", m["entropy_max_abs_err"], "excused", len(m["excused"]),
              "mismatch", len(m["level_mismatch"]), flush=True)
        assert m["entropy_max_abs_err"] < 2e-5
