"""Token Radius Attention (TRA) on AMD Instinct MI355X.

Thin Python binding over the C ABI of libtra.so (include/tra.h).  It only
marshals arguments: every step of the hot path runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.

    plan = tra.plan(q, k, grid=(T, H, W), **params)   # entropy -> radius -> tile lists
    o    = tra.attention(q, k, v, plan)                 # block-sparse masked attention

Dense warm-up variant (the entropy taken on the full attention):

    o, H = tra.dense_attention(q, k, v, grid=(T, H, W), entropy=True)
    plan = tra.plan_from_entropy(H, grid=(T, H, W), head_dim=d, dtype=q.dtype, **params)

q, k, v: contiguous [B, heads, T*H*W, d] CUDA tensors (bfloat16 or float32).
"""
import ctypes
import os

import torch

__all__ = ["TraError", "Plan", "plan", "plan_from_entropy", "import_plan", "attention", "dense_attention", "Schedule",
           "STEP_MODES", "radius_table",
           "validate", "library_path", "drift_noalloc_max_bytes",
           "load_library", "DEFAULT_PARAMS", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.environ.get("TRA_LIBRARY", os.path.join(_HERE, "libtra.so"))


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("heads", ctypes.c_int32), ("T", ctypes.c_int32),
                ("H", ctypes.c_int32), ("W", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [("a", ctypes.c_double), ("c", ctypes.c_double), ("budget_min", ctypes.c_double),
                ("budget_max", ctypes.c_double), ("decay", ctypes.c_double),
                ("radius_override", ctypes.c_double), ("levels_per_nat", ctypes.c_int32),
                ("pool_h", ctypes.c_int32), ("pool_w", ctypes.c_int32), ("tile_h", ctypes.c_int32),
                ("tile_w", ctypes.c_int32), ("generator", ctypes.c_int32), ("vote_threshold", ctypes.c_int32),
                ("block_mask", ctypes.c_int32), ("regroup", ctypes.c_int32), ("group_rows", ctypes.c_int32)]


class _Info(ctypes.Structure):
    _fields_ = [("n_queries", ctypes.c_int64), ("n_rows", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("n_qtiles", ctypes.c_int32), ("n_pool", ctypes.c_int32),
                ("n_levels", ctypes.c_int32), ("k_lo", ctypes.c_int32), ("T", ctypes.c_int32),
                ("max_row_len", ctypes.c_int32), ("group_rows", ctypes.c_int32)]


class _SchedParams(ctypes.Structure):
    _fields_ = [("warmup_steps", ctypes.c_int32), ("refresh_every", ctypes.c_int32),
                ("drift_threshold", ctypes.c_double)]


class _StepInfo(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("mode", ctypes.c_int32), ("drift", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIGS = {
    "tra_params_validate": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Params)]),
    "tra_radius_table": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Params), _P, _P,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
    "tra_plan_create": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Params), _P, _P, _P,
                                       ctypes.POINTER(_P)]),
    "tra_attention": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "tra_plan_rebuild": (ctypes.c_int, [_P, _P, _P, _P]),
    "tra_plan_matches": (ctypes.c_int, [_P, ctypes.POINTER(_Shape)]),
    "tra_plan_get_info": (ctypes.c_int, [_P, ctypes.POINTER(_Info)]),
    "tra_plan_export": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "tra_plan_stats": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_int64), _P]),
    "tra_plan_drift": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(ctypes.c_int64), _P]),
    "tra_plan_drift_noalloc": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(ctypes.c_int64), _P]),
    "tra_drift_noalloc_max_bytes": (ctypes.c_size_t, []),
    "tra_plan_import": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Params), _P, _P, _P, _P,
                                       ctypes.POINTER(_P)]),
    "tra_plan_create_from_entropy": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Params), _P, _P,
                                                    ctypes.POINTER(_P)]),
    "tra_plan_rebuild_from_entropy": (ctypes.c_int, [_P, _P, _P]),
    "tra_dense_attention": (ctypes.c_int, [ctypes.POINTER(_Shape), _P, _P, _P, _P, _P, _P]),
    "tra_plan_export_groups": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                              _P, _P, _P, _P]),
    "tra_plan_export_regroup": (ctypes.c_int, [_P, _P, _P]),
    "tra_schedule_create": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.POINTER(_Params),
                                           ctypes.POINTER(_SchedParams), ctypes.POINTER(_P)]),
    "tra_schedule_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(_StepInfo)]),
    "tra_schedule_plan": (ctypes.c_int, [_P, ctypes.POINTER(_P)]),
    "tra_schedule_destroy": (None, [_P]),
    "tra_plan_destroy": (None, [_P]),
    "tra_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tra_last_error": (ctypes.c_char_p, []),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None


def load_library():
    """Loads libtra.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m sparse_self_attention_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class TraError(RuntimeError):
    def __init__(self, status, fn):
        lib = load_library()
        self.status = status
        self.name = lib.tra_status_string(status).decode()
        super().__init__(f"{fn}: {self.name}: {lib.tra_last_error().decode()}")


def _check(status, fn):
    if status != 0:
        raise TraError(status, fn)


DEFAULT_PARAMS = dict(a=1.0, c=0.0, budget_min=16.0, budget_max=2048.0, decay=0.5,
                      radius_override=-1.0, levels_per_nat=8, pool_h=16, pool_w=16,
                      tile_h=8, tile_w=8, generator=0, vote_threshold=1, block_mask=0, regroup=0,
                      group_rows=0)
GENERATORS = {"entropy_disk": 0, "manhattan": 1, "radial": 2, "window_1d": 3}
_DTYPES = {torch.bfloat16: 1, torch.float32: 0}


def _make_params(params):
    unknown = set(params) - set(DEFAULT_PARAMS)
    if unknown:
        raise TypeError(f"unknown TRA parameters: {sorted(unknown)}")
    p = dict(DEFAULT_PARAMS)
    p.update(params)
    return _Params(**{k: (float(v) if isinstance(DEFAULT_PARAMS[k], float) else int(v)) for k, v in p.items()})


def _make_shape(B, heads, grid, head_dim, dtype_code):
    T, H, W = grid
    return _Shape(B, heads, T, H, W, head_dim, dtype_code)


def _shape_of(x, grid):
    if x.dim() != 4:
        raise ValueError("expected a [B, heads, T*H*W, d] tensor")
    if x.dtype not in _DTYPES:
        raise TypeError("dtype must be torch.bfloat16 or torch.float32")
    T, H, W = grid
    if x.shape[2] != T * H * W:
        raise ValueError(f"token axis {x.shape[2]} != T*H*W = {T * H * W}")
    return _make_shape(x.shape[0], x.shape[1], grid, x.shape[3], _DTYPES[x.dtype])


def _dev_ptr(x, name):
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(x.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def validate(B, heads, grid, head_dim, dtype=torch.bfloat16, **params):
    """Host-only check of a shape and parameter set; raises TraError if invalid."""
    lib = load_library()
    shape = _make_shape(B, heads, grid, head_dim, _DTYPES[dtype])
    _check(lib.tra_params_validate(ctypes.byref(shape), ctypes.byref(_make_params(params))), "tra_params_validate")


def radius_table(grid, dtype=torch.bfloat16, head_dim=128, **params):
    """Host-only radius table: returns (R2 int32 [n_levels, T], r0^2 float64 [n_levels], k_lo)."""
    import numpy as np
    lib = load_library()
    shape = _make_shape(1, 1, grid, head_dim, _DTYPES[dtype])
    prm = _make_params(params)
    n_levels, k_lo = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.tra_radius_table(ctypes.byref(shape), ctypes.byref(prm), None, None,
                                ctypes.byref(n_levels), ctypes.byref(k_lo)), "tra_radius_table")
    r2 = np.zeros((n_levels.value, grid[0]), dtype=np.int32)
    r0sq = np.zeros(n_levels.value, dtype=np.float64)
    _check(lib.tra_radius_table(ctypes.byref(shape), ctypes.byref(prm), r2.ctypes.data_as(_P),
                                r0sq.ctypes.data_as(_P), ctypes.byref(n_levels), ctypes.byref(k_lo)),
           "tra_radius_table")
    return r2, r0sq, k_lo.value


class Plan:
    """Owns a tra_plan.  Built by `plan(...)`; reusable across attention calls."""

    def __init__(self, handle, shape, grid, params, device):
        self._h = handle
        self.shape = shape
        self.grid = grid
        self.params = params
        self.device = device

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("plan was destroyed")
        return self._h

    def info(self):
        inf = _Info()
        _check(load_library().tra_plan_get_info(self.handle, ctypes.byref(inf)), "tra_plan_get_info")
        return {f: getattr(inf, f) for f, _ in _Info._fields_}

    def rebuild(self, q, k):
        """Re-plan from new q and k into the same buffers (a warm-up refresh)."""
        for x, nm in ((q, "q"), (k, "k")):
            self._check_tensor(x, nm)
        _check(load_library().tra_plan_rebuild(self.handle, _dev_ptr(q, "q"), _dev_ptr(k, "k"),
                                               _stream(self.device)), "tra_plan_rebuild")

    def export(self):
        """Host copies of the plan (numpy): levels, entropy, r2, row_ptr, col_idx, kbar."""
        import numpy as np
        inf = self.info()
        levels = np.zeros(inf["n_queries"], dtype=np.int16)
        entropy = np.zeros(inf["n_queries"], dtype=np.float32)
        r2 = np.zeros((inf["n_levels"], inf["T"]), dtype=np.int32)
        row_ptr = np.zeros(inf["n_rows"] + 1, dtype=np.int32)
        col_idx = np.zeros(max(1, inf["nnz"]), dtype=np.int32)
        s = self.shape
        kb_dtype = np.uint16 if s.dtype == 1 else np.float32
        kbar = np.zeros(s.B * s.heads * inf["n_pool"] * s.head_dim, dtype=kb_dtype)
        _check(load_library().tra_plan_export(
            self.handle, levels.ctypes.data_as(_P), entropy.ctypes.data_as(_P), r2.ctypes.data_as(_P),
            row_ptr.ctypes.data_as(_P), col_idx.ctypes.data_as(_P), kbar.ctypes.data_as(_P),
            _stream(self.device)), "tra_plan_export")
        BH, N = s.B * s.heads, s.T * s.H * s.W
        return {"levels": levels.reshape(BH, N), "entropy": entropy.reshape(BH, N), "r2": r2,
                "row_ptr": row_ptr, "col_idx": col_idx[:inf["nnz"]],
                "kbar": kbar.reshape(BH, inf["n_pool"], s.head_dim), "k_lo": inf["k_lo"],
                "n_qtiles": inf["n_qtiles"]}

    def export_groups(self):
        """bf16 plans: host copies of the attention kernel's group lists as
        (gptr, glen, entries [n, 2]) numpy int32 arrays."""
        import numpy as np
        lib = load_library()
        ng, ne = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.tra_plan_export_groups(self.handle, ctypes.byref(ng), ctypes.byref(ne), None, None, None,
                                          _stream(self.device)), "tra_plan_export_groups")
        gptr = np.zeros(ng.value, dtype=np.int32)
        glen = np.zeros(ng.value, dtype=np.int32)
        gl = np.zeros((max(1, ne.value), 2), dtype=np.int32)
        _check(lib.tra_plan_export_groups(self.handle, ctypes.byref(ng), ctypes.byref(ne), gptr.ctypes.data_as(_P),
                                          glen.ctypes.data_as(_P), gl.ctypes.data_as(_P), _stream(self.device)),
               "tra_plan_export_groups")
        return gptr, glen, gl[:ne.value]

    def export_regroup(self):
        """Plans created with regroup=1: each group's query slots (row * 16 +
        column inside the group) in the order the attention kernel deals them
        to its waves, as a numpy uint8 array [n_groups, 256]."""
        import numpy as np
        lib = load_library()
        ng, ne = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.tra_plan_export_groups(self.handle, ctypes.byref(ng), ctypes.byref(ne), None, None, None,
                                          _stream(self.device)), "tra_plan_export_groups")
        perm = np.zeros((ng.value, 256), dtype=np.uint8)
        _check(lib.tra_plan_export_regroup(self.handle, perm.ctypes.data_as(_P), _stream(self.device)),
               "tra_plan_export_regroup")
        return perm

    def stats(self):
        """(retained pairs, listed pairs): exact counts over the whole plan."""
        ret, lst = ctypes.c_int64(), ctypes.c_int64()
        _check(load_library().tra_plan_stats(self.handle, ctypes.byref(ret), ctypes.byref(lst),
                                             _stream(self.device)), "tra_plan_stats")
        return ret.value, lst.value

    def drift(self, q, k):
        """Number of queries whose budget level would change if the plan were
        rebuilt from (q, k); the plan itself is not modified."""
        self._check_tensor(q, "q")
        self._check_tensor(k, "k")
        n = ctypes.c_int64()
        _check(load_library().tra_plan_drift(self.handle, _dev_ptr(q, "q"), _dev_ptr(k, "k"), ctypes.byref(n),
                                             _stream(self.device)), "tra_plan_drift")
        return n.value

    def drift_noalloc(self, q, k):
        """`drift` computed in the library's static scratch: allocates no device
        memory (for callers that cannot allocate).  Calls that overlap on one
        GPU share that scratch and must not run concurrently."""
        self._check_tensor(q, "q")
        self._check_tensor(k, "k")
        n = ctypes.c_int64()
        _check(load_library().tra_plan_drift_noalloc(self.handle, _dev_ptr(q, "q"), _dev_ptr(k, "k"),
                                                     ctypes.byref(n), _stream(self.device)),
               "tra_plan_drift_noalloc")
        return n.value

    def rebuild_from_entropy(self, entropy):
        """Re-plan from per-query entropies ([B, heads, N] float32 device tensor)."""
        _check_entropy(entropy, self.shape)
        _check(load_library().tra_plan_rebuild_from_entropy(self.handle, _dev_ptr(entropy, "entropy"),
                                                            _stream(self.device)), "tra_plan_rebuild_from_entropy")

    def _check_tensor(self, x, name):
        shape = _shape_of(x, self.grid)
        st = load_library().tra_plan_matches(self.handle, ctypes.byref(shape))
        if st != 0:
            raise TraError(st, f"{name} vs plan")

    def destroy(self):
        if self._h is not None:
            load_library().tra_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def drift_noalloc_max_bytes():
    """Size of the static scratch `Plan.drift_noalloc` works in (bytes per GPU)."""
    return int(load_library().tra_drift_noalloc_max_bytes())


def plan(q, k, grid, **params):
    """Builds a TRA plan from q and k ([B, heads, T*H*W, d] device tensors)."""
    lib = load_library()
    shape = _shape_of(q, grid)
    if tuple(k.shape) != tuple(q.shape) or k.dtype != q.dtype:
        raise ValueError("q and k must have the same shape and dtype")
    prm = _make_params(params)
    h = ctypes.c_void_p()
    _check(lib.tra_plan_create(ctypes.byref(shape), ctypes.byref(prm), _dev_ptr(q, "q"),
                               _dev_ptr(k, "k"), _stream(q.device), ctypes.byref(h)), "tra_plan_create")
    return Plan(h, shape, tuple(grid), prm, q.device)


def attention(q, k, v, plan, out=None):
    """O = block-sparse masked softmax attention of q, k, v under `plan`."""
    for x, nm in ((q, "q"), (k, "k"), (v, "v")):
        plan._check_tensor(x, nm)
    if out is None:
        out = torch.empty_like(q)
    else:
        plan._check_tensor(out, "out")
    _check(load_library().tra_attention(plan.handle, _dev_ptr(q, "q"), _dev_ptr(k, "k"),
                                        _dev_ptr(v, "v"), _dev_ptr(out, "out"), _stream(q.device)),
           "tra_attention")
    return out


def _check_entropy(entropy, shape):
    N = shape.T * shape.H * shape.W
    if entropy.dtype != torch.float32 or tuple(entropy.shape) != (shape.B, shape.heads, N):
        raise ValueError(f"entropy must be a float32 [{shape.B}, {shape.heads}, {N}] tensor")


def plan_from_entropy(entropy, grid, head_dim, dtype=torch.bfloat16, **params):
    """Plan whose budget levels come from given per-query entropies (for example
    the exact ones of `dense_attention(..., entropy=True)`) instead of pooled keys."""
    if entropy.dim() != 3:
        raise ValueError("entropy must be [B, heads, T*H*W]")
    shape = _make_shape(entropy.shape[0], entropy.shape[1], grid, head_dim, _DTYPES[dtype])
    _check_entropy(entropy, shape)
    prm = _make_params(params)
    h = _P()
    _check(load_library().tra_plan_create_from_entropy(ctypes.byref(shape), ctypes.byref(prm),
                                                       _dev_ptr(entropy, "entropy"), _stream(entropy.device),
                                                       ctypes.byref(h)), "tra_plan_create_from_entropy")
    return Plan(h, shape, tuple(grid), prm, entropy.device)


def import_plan(saved, B, heads, grid, head_dim, dtype=torch.bfloat16, device="cuda", **params):
    """Plan rebuilt from `Plan.export()` output (its levels, entropy and pooled
    keys; the tile lists are rebuilt from the levels)."""
    import numpy as np
    shape = _make_shape(B, heads, grid, head_dim, _DTYPES[dtype])
    prm = _make_params(params)
    N = shape.T * shape.H * shape.W
    lv = np.ascontiguousarray(saved["levels"], dtype=np.int16).reshape(-1)
    if lv.size != B * heads * N:
        raise ValueError(f"levels must hold {B * heads * N} entries")
    ent = saved.get("entropy")
    ent = None if ent is None else np.ascontiguousarray(ent, dtype=np.float32).reshape(-1)
    kb = saved.get("kbar")
    kb = None if kb is None else np.ascontiguousarray(kb, dtype=np.uint16 if shape.dtype == 1 else np.float32)
    if ent is not None and ent.size != lv.size:
        raise ValueError("entropy must match levels")
    dev = torch.device(device)
    h = _P()
    _check(load_library().tra_plan_import(
        ctypes.byref(shape), ctypes.byref(prm), lv.ctypes.data_as(_P),
        None if ent is None else ent.ctypes.data_as(_P), None if kb is None else kb.ctypes.data_as(_P),
        _stream(dev), ctypes.byref(h)), "tra_plan_import")
    return Plan(h, shape, tuple(grid), prm, dev)


def dense_attention(q, k, v, grid, out=None, entropy=False):
    """Dense softmax attention over all keys of each head (the warm-up pass).
    With entropy=True (or a float32 [B, heads, N] device tensor to fill) also
    returns each query's exact attention entropy: (out, H)."""
    shape = _shape_of(q, grid)
    for x, nm in ((k, "k"), (v, "v")):
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError(f"{nm} must match q in shape and dtype")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if isinstance(entropy, torch.Tensor):
        H = entropy
        _check_entropy(H, shape)
    elif entropy:
        H = torch.empty((q.shape[0], q.shape[1], q.shape[2]), dtype=torch.float32, device=q.device)
    else:
        H = None
    _check(load_library().tra_dense_attention(ctypes.byref(shape), _dev_ptr(q, "q"), _dev_ptr(k, "k"),
                                              _dev_ptr(v, "v"), _dev_ptr(out, "out"),
                                              _dev_ptr(H, "entropy") if H is not None else None,
                                              _stream(q.device)),
           "tra_dense_attention")
    return (out, H) if H is not None else out


STEP_MODES = ("dense", "dense_replan", "sparse")


class _BorrowedPlan(Plan):
    """A plan owned by a Schedule (never destroyed from Python)."""

    def destroy(self):
        self._h = None


class Schedule:
    """Reuse schedule across denoising steps: `warmup_steps` dense steps (the last
    one measures exact entropies and builds the plan), then sparse steps under
    that plan; the plan is rebuilt by a dense step every `refresh_every` sparse
    steps (0 = never) and after a sparse step whose pooled-level drift exceeds
    `drift_threshold` of the queries (< 0: not tracked)."""

    def __init__(self, q, grid, warmup_steps=1, refresh_every=0, drift_threshold=-1.0, **params):
        self.shape = _shape_of(q, grid)
        self.grid = tuple(grid)
        self.device = q.device
        self.params = _make_params(params)
        sp = _SchedParams(int(warmup_steps), int(refresh_every), float(drift_threshold))
        h = _P()
        _check(load_library().tra_schedule_create(ctypes.byref(self.shape), ctypes.byref(self.params),
                                                  ctypes.byref(sp), ctypes.byref(h)), "tra_schedule_create")
        self._h = h

    def step(self, q, k, v, out=None):
        """Attention output of the next step and {"step", "mode", "drift"}."""
        fields = lambda sh: tuple(getattr(sh, f) for f, _ in _Shape._fields_)
        for x, nm in ((q, "q"), (k, "k"), (v, "v")):
            if fields(_shape_of(x, self.grid)) != fields(self.shape):
                raise ValueError(f"{nm} does not match the schedule's shape")
        if out is None:
            out = torch.empty_like(q)
        info = _StepInfo()
        _check(load_library().tra_schedule_step(self._h, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                                _dev_ptr(out, "out"), _stream(q.device), ctypes.byref(info)),
               "tra_schedule_step")
        return out, {"step": info.step, "mode": STEP_MODES[info.mode], "drift": info.drift}

    def plan(self):
        """The schedule's current plan (a borrowed view), or None before the first re-plan."""
        h = _P()
        _check(load_library().tra_schedule_plan(self._h, ctypes.byref(h)), "tra_schedule_plan")
        return None if not h.value else _BorrowedPlan(h, self.shape, self.grid, self.params, self.device)

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            load_library().tra_schedule_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
