"""Benchmark of the Token Radius Attention hot path on one MI355X.

One step = one pass of the whole path over the Wan2.1-14B-shaped 720p layer
call (B=1, 40 heads, d=128, latent grid 21x45x80 = 75,600 tokens, bf16): the
plan (key pooling, entropy, levels, tile lists) is rebuilt from (Q, K) and then
reused by four attention calls whose Q and K are perturbed by 1% (the warm-up
reuse path).  All inputs are synthetic, generated on the GPU and resident in
HBM before the timed region.

Printed: one JSON line.  `value` is retained-FLOP throughput of the whole step,
4*d*(retained pairs) per attention call times 4 calls, divided by the step time.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

The CPU baseline runs the fp64 oracle, unchanged, on the host's cores (one
worker process per core, at most 16) and times the plan of every head and
exact attention of a random query sample separately.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sparse_self_attention_amd as tra  # noqa: E402
from workloads import get_config, make_inputs, perturb  # noqa: E402

WORKLOAD = "wan21_14b_720p"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0


def measured_traffic():
    """HBM-side bytes per attention launch from the committed rocprofv3 byte
    counters (calibrated against a plain copy), or None when the kernel source
    has changed since they were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "attention_traffic.json")))
        src = open(os.path.join(ROOT, "sparse_self_attention_amd", "csrc", "tra_kernels.hip"), "rb").read()
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("kernel_source_sha256"):
        return None
    return rec["bytes_read_per_launch"] + rec["bytes_written_per_launch"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, q, k, v, plan_export, pool, attn_budget_s=15.0):
    """The oracle, unchanged, on the host's cores (a pool of worker processes,
    one core each, over heads and blocks of queries):
      - plan: pooled keys, entropies and levels of every head (the whole
        planning work of one call, all heads), timed;
      - attention: exact masked attention of random queries spread over all
        heads, blocks handed out until about `attn_budget_s` seconds of wall
        time have passed, timed; 4*d per retained pair.
    Also returns the queries whose entropy lies within the excuse band of a
    level boundary and whether every other level equals the GPU plan's."""
    import oracle as O
    from oracle import runner
    p = cfg.params()
    t0 = time.perf_counter()
    plans = runner.head_plans(pool, cfg, q, k, range(cfg.heads))
    t_plan = time.perf_counter() - t0
    excused = sum(len(plans[h]["excused"]) for h in range(cfg.heads))
    mismatch = 0
    for h in range(cfg.heads):
        lv_g = plan_export["levels"][h].astype(np.int64)
        bad = np.nonzero(lv_g != plans[h]["levels"])[0]
        mismatch += len(set(bad.tolist()) - set(plans[h]["excused"].tolist()))
    R2 = O.radius_table(p, cfg.T)
    rng = np.random.default_rng(0)
    heads = rng.permutation(cfg.heads)
    per_head_s = attn_budget_s / len(heads)
    pairs, nq, wall, busy = 0, 0, 0.0, 0.0
    for h in heads:
        rows = rng.choice(cfg.N, size=min(cfg.N, 4096), replace=False)
        done, _, n_pairs, w, b_s = runner.attention_rows(pool, cfg, q[0, h], k[0, h], v[0, h], rows,
                                                         plan_export["levels"][h], R2, block=16,
                                                         stop_after=per_head_s)
        pairs += n_pairs
        nq += len(done)
        wall += w
        busy += b_s
    attn_rate = 4.0 * cfg.head_dim * pairs / wall
    return {"attn_rate": attn_rate, "t_plan": t_plan, "pairs": pairs, "queries": nq, "wall": wall,
            "busy": busy, "excused": excused, "mismatch": mismatch}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--vote-threshold", type=int, default=None,
                    help="plan variant: list a key tile only with at least this many retained pairs")
    ap.add_argument("--block-mask", action="store_true",
                    help="plan variant: block-only masks (every key of a listed tile)")
    ap.add_argument("--regroup", action="store_true",
                    help="plan variant: each query-tile group's queries dealt to the attention "
                         "kernel's waves in level order")
    ap.add_argument("--group-rows", type=int, choices=[2, 3], default=None,
                    help="query-tile rows per attention group (default: the plan's choice)")
    ap.add_argument("--generator", choices=["entropy_disk", "manhattan", "radial", "window_1d"],
                    default="entropy_disk")
    ap.add_argument("--radius", type=float, default=None, help="fixed radius (static generators)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-attention comparison")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a reference for "
                         "hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    # The CPU oracle's worker processes start before this process touches the GPU.
    pool = None
    if not args.no_cpu_baseline:
        from oracle import runner
        pool = runner.make_pool()
        list(pool.map(abs, range(pool._max_workers)))  # start every worker now
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    tra.load_library()  # fails loudly when libtra.so is missing

    cfg = get_config(args.workload)
    variant = {}
    if args.vote_threshold is not None:
        variant["vote_threshold"] = args.vote_threshold
    if args.block_mask:
        variant["block_mask"] = 1
    if args.regroup:
        variant["regroup"] = 1
    if args.group_rows is not None:
        variant["group_rows"] = args.group_rows
    if args.generator != "entropy_disk":
        variant["generator"] = tra.GENERATORS[args.generator]
        if args.radius is not None or args.generator != "window_1d":
            variant["radius_override"] = args.radius if args.radius is not None else 16.0
    if variant:
        from dataclasses import replace
        cfg = replace(cfg, **variant)
    dev = torch.device("cuda:0")
    if args.copy_probe_mb > 0:
        src = torch.ones(args.copy_probe_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    grid = (cfg.T, cfg.H, cfg.W)
    calls = max(1, cfg.reuse_calls)
    log(f"[bench] generating {cfg.name}: heads={cfg.heads} N={cfg.N} d={cfg.head_dim} {cfg.dtype}")
    q, k, v = make_inputs(cfg, device=dev)
    qs, ks = [q], [k]
    for c in range(2, calls + 1):
        qs.append(perturb(q, c, 0))
        ks.append(perturb(k, c, 1))
    outs = [torch.empty_like(q) for _ in range(calls)]
    torch.cuda.synchronize()

    plan = tra.plan(q, k, grid=grid, **cfg.params())
    retained, listed = plan.stats()
    info = plan.info()
    flops_call = 4.0 * cfg.head_dim * retained
    log(f"[bench] plan: nnz={info['nnz']} retained={retained} density={retained / (cfg.heads * cfg.N ** 2):.4f} "
        f"tile efficiency={retained / listed:.3f}")

    stream = torch.cuda.current_stream(dev)

    def step(rec=None):
        if rec is not None:
            rec["p0"].record(stream)
        plan.rebuild(qs[0], ks[0])
        if rec is not None:
            rec["p1"].record(stream)
        for c in range(calls):
            if rec is not None:
                rec["a0"][c].record(stream)
            tra.attention(qs[c], ks[c], v, plan, out=outs[c])
            if rec is not None:
                rec["a1"][c].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup}")

    recs = [{"p0": torch.cuda.Event(enable_timing=True), "p1": torch.cuda.Event(enable_timing=True),
             "a0": [torch.cuda.Event(enable_timing=True) for _ in range(calls)],
             "a1": [torch.cuda.Event(enable_timing=True) for _ in range(calls)]} for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(recs[i])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    plan_ms = float(np.mean([r["p0"].elapsed_time(r["p1"]) for r in recs]))
    attn_ms_all = [r["a0"][c].elapsed_time(r["a1"][c]) for r in recs for c in range(calls)]
    attn_ms = float(np.mean(attn_ms_all))
    log(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step, plan {plan_ms:.3f} ms, attention {attn_ms:.3f} ms/call")

    # Cold caches: before each of a few extra calls, 512 MiB are written so that
    # neither the L2s nor the 256 MB last-level cache hold Q, K, V or the plan.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold_plan, cold_attn = [], []
    for i in range(3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        flush.fill_(i + 1)
        ev[0].record(stream)
        plan.rebuild(qs[0], ks[0])
        ev[1].record(stream)
        flush.fill_(i + 7)
        ev[2].record(stream)
        tra.attention(qs[-1], ks[-1], v, plan, out=outs[-1])
        ev[3].record(stream)
        torch.cuda.synchronize()
        cold_plan.append(ev[0].elapsed_time(ev[1]))
        cold_attn.append(ev[2].elapsed_time(ev[3]))
    del flush
    # Drift of the reused plan: queries whose level a re-plan from the inputs of
    # the last call would change.
    drift = plan.drift(qs[-1], ks[-1])
    log(f"[bench] cold: plan {np.median(cold_plan):.3f} ms, attention {np.median(cold_attn):.3f} ms; "
        f"plan drift at call {calls}: {drift} queries")

    # Dense attention over all keys on the same inputs (the full attention the
    # sparse path replaces) and the dense warm-up pass that also yields each
    # query's exact entropy.
    def time_ms(fn, reps):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    H_warm = torch.empty((cfg.batch, cfg.heads, cfg.N), dtype=torch.float32, device=dev)

    def dense(with_entropy):
        tra.dense_attention(q, k, v, grid, out=outs[0], entropy=H_warm if with_entropy else False)

    if args.no_dense:
        dense_ms = dense_ent_ms = float("nan")
    else:
        dense(False)
        dense(True)
        torch.cuda.synchronize()
        dense_ms = time_ms(lambda: dense(False), 3)
        dense_ent_ms = time_ms(lambda: dense(True), 3)
    dense_flops = 4.0 * cfg.head_dim * cfg.batch * cfg.heads * float(cfg.N) ** 2
    log(f"[bench] dense attention {dense_ms:.2f} ms, dense warm-up pass with entropy {dense_ent_ms:.2f} ms")

    def pct(xs):
        return {"p10": float(np.percentile(xs, 10)), "p50": float(np.percentile(xs, 50)),
                "p90": float(np.percentile(xs, 90))}

    plan_ms_all = [r["p0"].elapsed_time(r["p1"]) for r in recs]
    value = calls * flops_call / (ms_step * 1e-3) / 1e12
    achieved = flops_call / (attn_ms * 1e-3) / 1e12
    elem = 2 if cfg.dtype == "bf16" else 4
    # Algorithmic bytes of the planning steps: read Q and K, write the levels
    # (2 B per query) and the tile lists the pass builds: for bf16 plans
    # without a vote threshold the group lists the attention kernel reads
    # (8 B per entry, 8 B per group: offset and length), otherwise the CSR
    # (4 B per entry and per row offset).  The fp32 entropy the plan also
    # keeps (for export) is not counted.
    if cfg.dtype == "bf16" and variant.get("vote_threshold", 1) <= 1:
        _, glen, _ = plan.export_groups()
        list_bytes = 8 * int(glen.sum()) + 8 * len(glen)
    else:
        list_bytes = 4 * (info["nnz"] + info["n_rows"] + 1)
    plan_bytes = (2 * cfg.heads * cfg.N * cfg.head_dim * elem
                  + cfg.heads * cfg.N * 2
                  + list_bytes)
    result = {
        "metric": "ms/call + retained-FLOP TFLOPS (% bf16 MFMA peak), Wan2.1-14B 720p, 1 GPU",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name + ("+" + "+".join(f"{k}={v}" for k, v in variant.items()) if variant else ""),
                   "B": cfg.batch, "heads": cfg.heads, "grid": list(grid),
                   "head_dim": cfg.head_dim, "attention_calls_per_plan": calls,
                   "group_rows": info["group_rows"],
                   "retained_density": retained / (cfg.heads * cfg.N ** 2),
                   "tile_efficiency": retained / listed},
        "ms_per_call": {"attention": attn_ms, "plan": plan_ms, "step_per_call": ms_step / calls},
        "timing_ms": {"attention": pct(attn_ms_all), "plan": pct(plan_ms_all),
                      "cold_attention_median": float(np.median(cold_attn)),
                      "cold_plan_median": float(np.median(cold_plan))},
        "plan_drift": {"call": calls, "changed_levels": drift,
                       "fraction": drift / (cfg.batch * cfg.heads * cfg.N)},
        "attention": {"retained_tflops": achieved, "frac_bf16_peak": achieved / PEAK_BF16_TFLOPS,
                      "listed_flops_per_call": 4.0 * cfg.head_dim * listed,
                      "listed_pair_tflops": 4.0 * cfg.head_dim * listed / (attn_ms * 1e-3) / 1e12,
                      "retained_flops_per_call": flops_call},
        "plan": {"ms": plan_ms, "algorithmic_bytes": plan_bytes,
                 "gbps": plan_bytes / (plan_ms * 1e-3) / 1e9,
                 "frac_hbm_peak": plan_bytes / (plan_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic() if cfg.name == WORKLOAD else None},
    }
    if not args.no_dense:
        result["dense"] = {"ms": dense_ms, "tflops": dense_flops / (dense_ms * 1e-3) / 1e12,
                           "frac_bf16_peak": dense_flops / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "warmup_with_entropy_ms": dense_ent_ms,
                           "sparse_attention_speedup": dense_ms / attn_ms,
                           "step_speedup": (calls * dense_ms) / ms_step}
    if pool is not None and not variant:
        log(f"[bench] timing the CPU oracle on {pool._max_workers} host cores")
        cb = cpu_baseline(cfg, q, k, v, plan.export(), pool)
        pool.shutdown()
        from oracle import runner
        attn_call_s = flops_call / cb["attn_rate"]
        step_s = cb["t_plan"] + calls * attn_call_s
        result["cpu_baseline"] = {
            "value": calls * flops_call / step_s / 1e12, "unit": "TFLOP/s", "cores": pool._max_workers,
            "kind": "oracle", "nproc": os.cpu_count(), "affinity_cores": runner.host_cores(),
            "cpu_model": runner.cpu_model(),
            "plan_s": cb["t_plan"], "attention_tflops": cb["attn_rate"] / 1e12,
            "attention_s_per_call_estimated": attn_call_s, "step_s_estimated": step_s,
            "sample": (f"plan: pooled keys, entropies and levels of all {cfg.heads} heads in {cb['t_plan']:.2f} s; "
                       f"attention: exact masked attention of {cb['queries']} random queries over all heads "
                       f"({cb['pairs']} retained pairs) in {cb['wall']:.2f} s wall; value = {calls} calls' "
                       f"retained FLOP / (plan time + {calls} x estimated attention time per call)")}
        result["excused"] = {"count": cb["excused"], "fraction": cb["excused"] / (cfg.batch * cfg.heads * cfg.N),
                             "levels_differing_outside_excused": cb["mismatch"]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
