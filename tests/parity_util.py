"""GPU-vs-oracle comparison used by the parity tests and the smoke check.

Procedure for one (batch, head) slice, following the parity bar of the path:
  1. pooled keys: bit-exact;
  2. entropy: reported (|H_gpu - H_oracle|, fp32 export of an fp64 epilogue);
  3. levels: equal to the oracle's everywhere except at queries whose oracle
     entropy lies within 1e-5 of a level boundary (the excused set E, which
     must hold <= 0.1% of the queries and is reported);
  4. tile lists: the oracle's CSR built from the GPU levels (identical to the
     oracle's own outside E) must equal the GPU's, bit for bit;
  5. output: the oracle's fp64 attention under the same levels, max-abs <= 2e-2
     and mean-abs <= 2e-3 of the GPU output.
"""
import numpy as np
import torch

import oracle as O
import sparse_self_attention_amd as tra
from oracle import runner

import ref_tiles
from workloads import make_inputs

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
EXCUSE_FRACTION = 1e-3


def bf16_bits_to_f64(u16):
    return (np.asarray(u16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_run(cfg, device, inputs=None):
    q, k, v = inputs if inputs is not None else make_inputs(cfg, device=device)
    plan = tra.plan(q, k, grid=(cfg.T, cfg.H, cfg.W), **cfg.params())
    o = tra.attention(q, k, v, plan)
    torch.cuda.synchronize()
    return {"q": q, "k": k, "v": v, "o": o, "plan": plan, "export": plan.export()}


def check_head(cfg, run, b, h, tile_sample=None, query_sample=None, rng=None, oracle_plan=None,
               tile_lists="oracle", pool=None):
    """Compares one head; returns a metrics dict (asserts on failure).

    tile_lists: "oracle" compares each query tile's list with the oracle's
    query-by-query definition (`tile_sample` rows, default all); "reference"
    compares every row of the head with the vectorised reference lists
    (tests/ref_tiles.py, pinned to the oracle's definition on the CPU).
    oracle_plan: the oracle's pooled keys, entropies, levels and excused set of
    this head when already computed (oracle.runner.head_plans).
    pool: an oracle.runner pool that computes the reference outputs."""
    p = cfg.params()
    bh = b * cfg.heads + h
    exp = run["export"]
    og = run["o"][b, h].double().cpu().numpy()
    lv_g = exp["levels"][bh].astype(np.int64)
    R2 = O.radius_table(p, cfg.T)
    assert np.array_equal(exp["r2"].astype(np.int64), R2)
    out = {"bh": bh}
    if p["radius_override"] < 0:
        if oracle_plan is None:
            qh = run["q"][b, h].double().cpu().numpy()
            kh = run["k"][b, h].double().cpu().numpy()
            pools = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w)
            kbar_o = O.pool_keys(kh, pools, cfg.dtype)
            H_o = O.entropy(qh, kbar_o, pools.block_sizes())
            oracle_plan = {"kbar": kbar_o, "H": H_o, "levels": O.levels(H_o, p),
                           "excused": O.excused_queries(H_o, p)}
        check_levels(cfg, exp, bh, oracle_plan, out)
    else:
        assert np.all(lv_g == -1)
    row_ptr = exp["row_ptr"].astype(np.int64)
    col_idx = exp["col_idx"].astype(np.int64)
    tiles = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.tile_h, cfg.tile_w)
    base = bh * tiles.count
    if tile_lists == "reference":
        rp_r, ci_r = ref_tiles.csr(lv_g, R2, cfg.T, cfg.H, cfg.W, p)
        rows_h = row_ptr[base:base + tiles.count + 1]
        assert np.array_equal(rows_h - rows_h[0], rp_r), "tile-list lengths differ"
        assert np.array_equal(col_idx[rows_h[0]:rows_h[-1]], ci_r), "tile-list columns differ"
        out["tile_rows_compared"] = tiles.count
    else:
        tile_ids = range(tiles.count) if tile_sample is None else tile_sample
        for a in tile_ids:
            got = col_idx[row_ptr[base + a]:row_ptr[base + a + 1]]
            ref = O.query_tile_row(a, lv_g, R2, tiles, p)
            assert np.array_equal(got, ref), f"tile list of query tile {a} differs"
        out["tile_rows_compared"] = len(tile_ids)
    queries = np.arange(cfg.N) if query_sample is None else np.asarray(query_sample)
    if pool is not None:
        done, o_ref, _, _, _ = runner.attention_rows(pool, cfg, run["q"][b, h], run["k"][b, h], run["v"][b, h],
                                                     queries, lv_g, R2)
        assert np.array_equal(done, queries)
    else:
        qh, kh, vh = (run[x][b, h].double().cpu().numpy() for x in "qkv")
        o_ref = O.attention_rows(qh, kh, vh, queries, lv_g, R2, cfg.T, cfg.H, cfg.W, p)
    err = np.abs(og[queries] - o_ref)
    out["queries_compared"] = len(queries)
    out["o_max_abs"] = float(err.max())
    out["o_mean_abs"] = float(err.mean())
    assert np.all(np.isfinite(og[queries]))
    assert out["o_max_abs"] <= MAX_ABS and out["o_mean_abs"] <= MEAN_ABS, out
    return out


def check_levels(cfg, exp, bh, oracle_plan, out=None):
    """Pooled keys bit-exact; levels equal to the oracle's outside the excused
    set (queries within 1e-5 nat of a level boundary, at most 0.1% of them)."""
    out = {} if out is None else out
    kbar_g = exp["kbar"][bh]
    kbar_g = bf16_bits_to_f64(kbar_g) if cfg.dtype == "bf16" else kbar_g.astype(np.float64)
    assert np.array_equal(kbar_g, oracle_plan["kbar"]), "pooled keys differ"
    E = np.asarray(oracle_plan["excused"])
    out["entropy_max_abs_err"] = float(np.max(np.abs(exp["entropy"][bh].astype(np.float64) - oracle_plan["H"])))
    out["excused"] = E.tolist()
    assert len(E) <= EXCUSE_FRACTION * cfg.N, f"{len(E)} queries near a boundary"
    lv_g = exp["levels"][bh].astype(np.int64)
    bad = np.nonzero(lv_g != oracle_plan["levels"])[0]
    out["level_mismatch"] = bad.tolist()
    assert set(bad.tolist()) <= set(E.tolist()), f"levels differ outside the excused set: {bad[:10]}"
    return out


def check_csr_properties(cfg, run):
    """Properties that hold at any size: monotone offsets, ascending in-range columns."""
    exp = run["export"]
    tiles = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.tile_h, cfg.tile_w)
    rp = exp["row_ptr"].astype(np.int64)
    ci = exp["col_idx"].astype(np.int64)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 1)  # every query tile lists at least its own tile
    assert rp[-1] == len(ci)
    assert ci.min() >= 0 and ci.max() < tiles.count
    starts = np.zeros(len(ci), dtype=bool)
    starts[rp[:-1][rp[:-1] < len(ci)]] = True
    d = np.diff(ci)
    assert np.all((d > 0) | starts[1:]), "columns not ascending within a row"
    # every query tile lists its own tile (the self key is always retained)
    rows = np.arange(len(rp) - 1) % tiles.count
    own = [rows[r] in ci[rp[r]:rp[r + 1]] for r in range(0, len(rp) - 1, max(1, (len(rp) - 1) // 500))]
    assert all(own)


def expected_group_lists(cfg, row_ptr, col_idx, bh, rows=2):
    """The bf16 kernel's group lists of head slice bh, derived from CSR rows:
    per group of rows x 2 query tiles, the ascending union of the members' key
    tiles with member bits and edge flags (as the C ABI exports them)."""
    tiles = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.tile_h, cfg.tile_w)
    nh, nw = tiles.nbh, tiles.nbw
    ngh, ngw = (nh + rows - 1) // rows, (nw + 1) // 2
    out = {}
    for t in range(cfg.T):
        for gr in range(ngh):
            for gc in range(ngw):
                members = {}
                for m in range(2 * rows):
                    tr, tc = rows * gr + (m >> 1), 2 * gc + (m & 1)
                    if tr < nh and tc < nw:
                        r = bh * tiles.count + (t * nh + tr) * nw + tc
                        for K in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                            members[int(K)] = members.get(int(K), 0) | (1 << m)
                ent = []
                for K in sorted(members):
                    tk, rem = divmod(K, tiles.per_frame)
                    ktr, kc = divmod(rem, nw)
                    kr0, kc0 = ktr * 8, kc * 8
                    edge = kr0 + 8 > cfg.H or kc0 + 8 > cfg.W
                    x = (tk | (members[K] << 16) | (1 << 31 if edge else 0)) - (1 << 32 if edge else 0)
                    ent.append((x, kr0 | (kc0 << 16)))
                gid = (bh * cfg.T + t) * ngh * ngw + gr * ngw + gc
                out[gid] = np.array(ent, dtype=np.int64).reshape(-1, 2)
    return out


def check_group_lists(cfg, run, bh):
    """Group lists of head slice bh equal those derived from the plan's CSR
    (which the other checks compare with the oracle), entry for entry."""
    gptr, glen, gl = run["plan"].export_groups()
    exp = run["export"]
    rows = run["plan"].info()["group_rows"]
    assert rows in (2, 3)
    want = expected_group_lists(cfg, exp["row_ptr"].astype(np.int64), exp["col_idx"].astype(np.int64), bh, rows)
    for gid, ent in want.items():
        got = gl[gptr[gid]:gptr[gid] + glen[gid]].astype(np.int64)
        assert np.array_equal(got, ent), f"group {gid}: {got[:6].tolist()} vs {ent[:6].tolist()}"
    return len(want)


def _onehot_values(N, perm, gpu):
    j = perm if perm is not None else np.arange(N)
    v = torch.zeros((N, 128), dtype=torch.float32)
    v[np.arange(N), torch.from_numpy(j % 64)] = 1.0
    v[np.arange(N), torch.from_numpy(64 + j // 64)] = 1.0
    return v.to(torch.bfloat16).reshape(1, 1, N, 128).to(gpu)


def check_key_sets(cfg, plan, lv, gpu, seed):
    """Every query's retained key set, recovered exactly from O (Q = 0, so each
    retained key weighs the same, and V one-hot encodes the key index; see the
    exact key-set tests in test_gpu_parity.py), against the oracle's
    brute-force mask for the levels lv.  Returns (largest set, worst distance
    of a scaled entry from its integer count)."""
    p = cfg.params()
    N = cfg.N
    assert N <= 64 * 64
    R2 = O.radius_table(p, cfg.T)
    mask = O.dense_mask(lv, R2, cfg.T, cfg.H, cfg.W, p)  # oracle's brute-force N x N mask
    size = mask.sum(axis=1).astype(np.float64)
    q = torch.zeros((1, 1, N, 128), dtype=torch.bfloat16, device=gpu)
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = torch.randn((1, 1, N, 128), generator=g).to(torch.bfloat16).to(gpu)
    perm = np.random.default_rng(seed).permutation(N)
    worst = 0.0
    for enc in (None, perm):
        v = _onehot_values(N, enc, gpu)
        o = tra.attention(q, k, v, plan)
        torch.cuda.synchronize()
        scaled = o[0, 0].double().cpu().numpy() * size[:, None]
        got = np.rint(scaled).astype(np.int64)
        want = np.rint(mask.astype(np.float64) @ v[0, 0].double().cpu().numpy()).astype(np.int64)
        bad = np.nonzero(np.any(got != want, axis=1))[0]
        assert len(bad) == 0, f"{len(bad)} queries with a different key set, first {bad[:8].tolist()}"
        worst = max(worst, float(np.abs(scaled - got).max()))
    return int(size.max()), worst


LISTED_MAX_ABS, LISTED_MEAN_ABS = 2e-2, 2e-3


def check_listed(cfg, run, h, block_only, tile_sample=None, query_sample=None):
    """Head h of a plan with a vote threshold and/or block-only masks: each
    query tile's filtered list against the oracle's token votes, and O against
    the oracle's attention over exactly the listed tiles (every key of a listed
    tile with block_only, else the exact mask inside them)."""
    p = cfg.params()
    exp = run["export"]
    lv = exp["levels"][h].astype(np.int64)
    R2 = O.radius_table(p, cfg.T)
    tiles = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.tile_h, cfg.tile_w)
    rp = exp["row_ptr"].astype(np.int64)
    base = h * tiles.count
    rows_h = rp[base:base + tiles.count + 1]
    ci_h = exp["col_idx"][rows_h[0]:rows_h[-1]].astype(np.int64)
    rp_h = rows_h - rows_h[0]
    theta = p["vote_threshold"]
    for a in (range(tiles.count) if tile_sample is None else tile_sample):
        votes = O.tile_votes(int(a), lv, R2, tiles, p)
        ref = np.array(sorted(b for b, n in votes.items() if n >= theta), dtype=np.int64)
        assert np.array_equal(ci_h[rp_h[a]:rp_h[a + 1]], ref), f"tile list of query tile {a} differs"
    qs = np.arange(cfg.N) if query_sample is None else np.asarray(query_sample)
    qh, kh, vh = (run[x][0, h].double().cpu().numpy() for x in ("q", "k", "v"))
    ref = O.attention_rows_listed(qh, kh, vh, qs, lv, R2, tiles, p, rp_h, ci_h, block_only)
    err = np.abs(run["o"][0, h].double().cpu().numpy()[qs] - ref)
    assert err.max() <= LISTED_MAX_ABS and err.mean() <= LISTED_MEAN_ABS, (err.max(), err.mean())
    return err
