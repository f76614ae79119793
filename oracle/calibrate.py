"""Calibrate the budget scale c = ln(tau) of a workload to a target mean density.

TEST INFRASTRUCTURE ONLY.  Uses the oracle and the seeded CPU generator; the
chosen constants are then written by hand into workloads/configs.py.

The entropy-to-budget map is ln B = a*H + c with a = 1 (the analytic map
B ~ tau*exp(H) of the method's summary page, section 2, Intuition I).  With
c = 0 the pooled entropies of the synthetic inputs are close to ln N, so every
query would sit at any cap that gives the target density; the scale tau is the
free constant of that map, so it is what gets calibrated.  Candidates are
c = -j/16; the one whose exact mean retained density (oracle counts, every
query of the sampled heads) is closest to the target is reported.

usage: python -m oracle.calibrate <workload> <target_density> [n_heads]
"""
import sys
import time

import numpy as np

from workloads import get_config, make_inputs
from . import tra_oracle as O


def head_entropies(cfg, heads):
    q, k, _ = make_inputs(cfg, heads=heads)
    pools = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w)
    out = []
    for slot in range(len(heads)):
        kbar = O.pool_keys(k[0, slot].double().numpy(), pools, cfg.dtype)
        out.append(O.entropy(q[0, slot].double().numpy(), kbar, pools.block_sizes()))
    return np.stack(out)


def density_for(cfg, H, count_cache):
    p = cfg.params()
    lv = O.levels(H.reshape(-1), p).reshape(H.shape)
    R2 = O.radius_table(p, cfg.T)
    total = 0
    for level in np.unique(lv):
        key = (cfg.budget_min, cfg.budget_max, cfg.decay, int(level))
        if key not in count_cache:
            count_cache[key] = O.retained_counts(np.full(cfg.N, level), R2, cfg.T, cfg.H, cfg.W, p)
        tab = count_cache[key]
        for row in range(H.shape[0]):
            total += int(tab[lv[row] == level].sum())
    return total / (H.size * cfg.N), lv


def main(argv):
    name, target = argv[0], float(argv[1])
    cfg = get_config(name)
    n_heads = int(argv[2]) if len(argv) > 2 else cfg.heads
    t0 = time.time()
    H = head_entropies(cfg, list(range(n_heads)))
    print(f"{name}: entropies of {n_heads} heads in {time.time() - t0:.1f}s; "
          f"H percentiles 0/50/100 = {np.percentile(H, [0, 50, 100]).round(4).tolist()}")
    cache, best = {}, None
    for j in range(0, 97):
        c = -j / 16.0
        dens, lv = density_for(cfg.with_(c=c), H, cache)
        k_lo, k_hi = O.level_range(cfg.with_(c=c).params())
        print(f"  c={c:+.4f} density={dens:.5f} levels {lv.min()}..{lv.max()} "
              f"capped={np.mean(lv == k_hi):.3f}")
        if best is None or abs(dens - target) < abs(best[1] - target):
            best = (c, dens)
        if dens < target * 0.8:
            break
    print(f"chosen c={best[0]:+.4f} density={best[1]:.5f} (target {target})")


if __name__ == "__main__":
    main(sys.argv[1:])
