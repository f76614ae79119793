"""Seeded synthetic Q/K/V shaped like video-DiT latent attention inputs.

Recipe (per head, independent draws):
  P(t,h,w) in R^d  : 3-axis sinusoidal position feature; axis widths d/4 (t),
                     3d/8 (h), 3d/8 (w); for an axis of width m and coordinate x
                     the block is [sin(w_0 x)..sin(w_{m/2-1} x), cos(w_0 x)..],
                     w_j = 10000^(-2j/m).  Blocks are concatenated [t | h | w].
  s_i              : log-uniform in [s_lo, s_hi] (per query: varies the entropy)
  Q = s * (P + 0.3 n_Q),  K = P + 0.3 n_K,  V ~ N(0, 1)
All arithmetic is float32 on the chosen device, then rounded once to the
workload dtype (bf16 by round-to-nearest-even).  The random stream is torch's
seeded generator on that device, so a given (seed, head, device type) always
yields the same tensors; CPU and GPU streams differ, which is fine because every
comparison feeds the same materialised tensors to both sides.
"""
import math

import numpy as np
import torch

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def positional_features(T: int, H: int, W: int, d: int) -> np.ndarray:
    """[T*H*W, d] float64 sinusoidal features, token order n = (t*H + h)*W + w."""
    assert d % 8 == 0, "head_dim must be a multiple of 8"
    widths = (d // 4, 3 * d // 8, 3 * d // 8)
    coords = np.stack(np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij"), -1)
    coords = coords.reshape(-1, 3).astype(np.float64)
    blocks = []
    for axis, m in enumerate(widths):
        j = np.arange(m // 2, dtype=np.float64)
        omega = 10000.0 ** (-2.0 * j / m)
        ang = coords[:, axis:axis + 1] * omega[None, :]
        blocks += [np.sin(ang), np.cos(ang)]
    return np.concatenate(blocks, axis=1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_inputs(cfg, device="cpu", heads=None):
    """Returns (q, k, v) as contiguous [B, heads, N, d] tensors of cfg.dtype on device.

    `heads` optionally restricts generation to a subset of head indices (the
    values of a head do not depend on which other heads are generated).
    """
    device = torch.device(device)
    N, d = cfg.N, cfg.head_dim
    heads = list(range(cfg.heads)) if heads is None else list(heads)
    P = torch.from_numpy(positional_features(cfg.T, cfg.H, cfg.W, d)).to(torch.float32).to(device)
    dt = _DT[cfg.dtype]
    B = cfg.batch
    q = torch.empty((B, len(heads), N, d), dtype=dt, device=device)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    lo, hi = math.log(cfg.s_lo), math.log(cfg.s_hi)
    for b in range(B):
        for slot, h in enumerate(heads):
            g = _gen(device, cfg.seed * 1_000_003 + b * 10_007 + h)
            u = torch.rand((N, 1), generator=g, device=device, dtype=torch.float32)
            s = torch.exp(lo + (hi - lo) * u)
            nq = torch.randn((N, d), generator=g, device=device, dtype=torch.float32)
            nk = torch.randn((N, d), generator=g, device=device, dtype=torch.float32)
            vv = torch.randn((N, d), generator=g, device=device, dtype=torch.float32)
            q[b, slot] = (s * (P + 0.3 * nq)).to(dt)
            k[b, slot] = (P + 0.3 * nk).to(dt)
            v[b, slot] = vv.to(dt)
    return q, k, v


def perturb(x: torch.Tensor, call: int, which: int, rel: float = 0.01) -> torch.Tensor:
    """x + rel * std(x) * n with fresh N(0,1) draws from seed 1000 + call.

    Used for the plan-reuse workload: calls after the first get slightly moved
    Q (which=0) and K (which=1) while the plan of the first call is reused.
    """
    g = _gen(x.device, 1000 + 17 * call + which)
    sigma = float(x.double().std())
    n = torch.randn(x.shape, generator=g, device=x.device, dtype=torch.float32)
    return (x.float() + (rel * sigma) * n).to(x.dtype)
