"""Runs the unchanged oracle over independent pieces of a workload (heads,
blocks of queries) in a pool of worker processes.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): used by tests/ for
full-size parity and by the benchmark's CPU-baseline leg.  It adds no
arithmetic of its own: every worker calls the functions of tra_oracle as they
are, on exact copies of the inputs (bf16 values travel as their bit patterns
and are widened to float64 in the worker, which is exact).

Workers are started with the "spawn" method, so they hold no GPU state, and
each one is limited to one BLAS thread: `workers` processes use `workers`
cores.  Head tensors are handed over through memory-mapped .npy files in a
temporary directory instead of being pickled once per task.
"""
import multiprocessing
import os
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

# The box a GPU run lands on grants a 16-core share whatever os.cpu_count()
# reports there; the container the CPU tests run in has 8 cores.
MAX_WORKERS = 16


def host_cores():
    """Cores this process may run on (its affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_workers():
    return max(1, min(MAX_WORKERS, host_cores()))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _init_worker():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def make_pool(workers=None):
    """A process pool whose workers hold no GPU state and use one core each."""
    ctx = multiprocessing.get_context("spawn")
    return ProcessPoolExecutor(max_workers=workers or default_workers(), mp_context=ctx,
                               initializer=_init_worker)


def _to_bits(x):
    """A head's values as an exactly recoverable array: bf16 tensors as their
    uint16 bit patterns, everything else as float64."""
    import torch
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.bfloat16:
            return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return x.detach().double().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _from_bits(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


class HeadStore:
    """Head slices written once to memory-mapped files that workers read."""

    def __init__(self):
        self._dir = tempfile.TemporaryDirectory(prefix="tra_oracle_")
        self._n = 0

    def put(self, x):
        path = os.path.join(self._dir.name, f"a{self._n}.npy")
        self._n += 1
        np.save(path, _to_bits(x))
        return path

    def close(self):
        self._dir.cleanup()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _load(path):
    return _from_bits(np.load(path, mmap_mode="r"))


# ---------------------------------------------------------------------------
# Tasks (module-level so that spawned workers can import them)
# ---------------------------------------------------------------------------
def _plan_task(q_path, k_path, T, H, W, pool_h, pool_w, dtype, p):
    from . import tra_oracle as O
    t0 = time.perf_counter()
    q, k = _load(q_path), _load(k_path)
    pools = O.Geometry(T, H, W, pool_h, pool_w)
    kbar = O.pool_keys(k, pools, dtype)
    Hq = O.entropy(q, kbar, pools.block_sizes())
    lv = O.levels(Hq, p)
    exc = O.excused_queries(Hq, p)
    return {"kbar": kbar, "H": Hq, "levels": lv, "excused": exc, "seconds": time.perf_counter() - t0}


def _rows_task(q_path, k_path, v_path, rows, lv, R2, T, H, W, p):
    from . import tra_oracle as O
    t0 = time.perf_counter()
    q, k, v = _load(q_path), _load(k_path), _load(v_path)
    out = O.attention_rows(q, k, v, rows, lv, R2, T, H, W, p)
    pairs = int(sum(O.retained_count(int(i), int(lv[i]), R2, T, H, W, p) for i in rows))
    return out, pairs, time.perf_counter() - t0


# ---------------------------------------------------------------------------
# Drivers
# ---------------------------------------------------------------------------
def head_plans(pool, cfg, q, k, heads, batch=0):
    """Oracle pooled keys, entropies, levels and excused queries of the given
    heads of batch entry `batch` ([B, heads, N, d] tensors), one head per task.
    Returns {head: dict}."""
    p = cfg.params()
    with HeadStore() as st:
        futs = {}
        for h in heads:
            qp, kp = st.put(q[batch, h]), st.put(k[batch, h])
            futs[h] = pool.submit(_plan_task, qp, kp, cfg.T, cfg.H, cfg.W, cfg.pool_h, cfg.pool_w, cfg.dtype, p)
        return {h: f.result() for h, f in futs.items()}


def attention_rows(pool, cfg, q, k, v, rows, lv, R2, block=64, stop_after=None):
    """Oracle O_i (fp64) of the given query rows of one head ([N, d] tensors or
    arrays), in blocks of `block` queries spread over the pool.

    With `stop_after` (seconds), blocks are handed out in order and no new block
    is started once that much wall time has passed; the rows actually computed
    come back first.  Returns (rows_done, O [len(rows_done), d], retained
    pairs, wall seconds, summed worker seconds)."""
    p = cfg.params()
    rows = np.asarray(rows, dtype=np.int64)
    lv = np.asarray(lv, dtype=np.int64)
    blocks = [rows[i:i + block] for i in range(0, len(rows), block)]
    t0 = time.perf_counter()
    with HeadStore() as st:
        qp, kp, vp = st.put(q), st.put(k), st.put(v)
        args = (lv, R2, cfg.T, cfg.H, cfg.W, p)
        done, outs, pairs, busy = [], [], 0, 0.0
        inflight = []
        nxt = 0
        width = pool._max_workers
        while nxt < len(blocks) or inflight:
            while nxt < len(blocks) and len(inflight) < 2 * width and (
                    stop_after is None or time.perf_counter() - t0 < stop_after):
                inflight.append((blocks[nxt], pool.submit(_rows_task, qp, kp, vp, blocks[nxt], *args)))
                nxt += 1
            if not inflight:
                break
            blk, fut = inflight.pop(0)
            o, n, s = fut.result()
            done.append(blk)
            outs.append(o)
            pairs += n
            busy += s
            if stop_after is not None and time.perf_counter() - t0 >= stop_after:
                nxt = len(blocks)
    wall = time.perf_counter() - t0
    rows_done = np.concatenate(done) if done else np.zeros(0, dtype=np.int64)
    o = np.concatenate(outs) if outs else np.zeros((0, q.shape[-1]))
    return rows_done, o, pairs, wall, busy
