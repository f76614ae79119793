"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function include/tra.h declares, reject bad
shapes and parameters with the documented status codes, and compute the same
radius table as the oracle, bit for bit.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest
import torch

import oracle as O
import sparse_self_attention_amd as tra
from workloads import CONFIGS, small_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "tra.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(tra_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = tra.load_library()
    declared = _declared_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(tra.EXPORTED_SYMBOLS)


def test_status_strings():
    lib = tra.load_library()
    assert lib.tra_status_string(0) == b"TRA_OK"
    assert lib.tra_status_string(4) == b"TRA_ERR_PLAN_MISMATCH"


def _validate(**kw):
    shape = dict(B=1, heads=2, grid=(4, 9, 10), head_dim=128, dtype=torch.bfloat16)
    params = {}
    for k, v in kw.items():
        if k in shape:
            shape[k] = v
        else:
            params[k] = v
    return tra.validate(shape["B"], shape["heads"], shape["grid"], shape["head_dim"], shape["dtype"], **params)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), "TRA_ERR_DTYPE"),
    (dict(grid=(0, 4, 4)), "TRA_ERR_SHAPE"),
    (dict(B=0), "TRA_ERR_SHAPE"),
    (dict(decay=0.0), "TRA_ERR_INVALID_ARG"),
    (dict(decay=1.5), "TRA_ERR_INVALID_ARG"),
    (dict(budget_min=0.0), "TRA_ERR_INVALID_ARG"),
    (dict(budget_min=100.0, budget_max=50.0), "TRA_ERR_INVALID_ARG"),
    (dict(budget_min=17.0, budget_max=17.5), "TRA_ERR_INVALID_ARG"),  # no level inside
    (dict(levels_per_nat=0), "TRA_ERR_INVALID_ARG"),
    (dict(pool_h=0), "TRA_ERR_INVALID_ARG"),
    (dict(tile_h=4, tile_w=16), "TRA_ERR_INVALID_ARG"),
    (dict(a=math.inf), "TRA_ERR_INVALID_ARG"),
    (dict(radius_override=1e9), "TRA_ERR_INVALID_ARG"),
    (dict(budget_max=1e12), "TRA_ERR_INVALID_ARG"),
    # one bf16 head of K would span 2^31 bytes or more (32-bit buffer offsets)
    (dict(grid=(2, 32767, 256), heads=1), "TRA_ERR_SHAPE"),
    (dict(generator=4), "TRA_ERR_INVALID_ARG"),
    (dict(generator=3, grid=(2, 8, 520)), "TRA_ERR_SHAPE"),  # the 1-D window: at most 64 tile columns
    (dict(generator=3, vote_threshold=2), "TRA_ERR_INVALID_ARG"),
    (dict(generator=1), "TRA_ERR_INVALID_ARG"),  # the static generators need radius_override >= 0
    (dict(generator=2, radius_override=-1.0), "TRA_ERR_INVALID_ARG"),
    (dict(regroup=2), "TRA_ERR_INVALID_ARG"),
    (dict(regroup=1, dtype=torch.float32), "TRA_ERR_INVALID_ARG"),  # a layout of the bf16 kernel
    (dict(regroup=1, block_mask=1), "TRA_ERR_INVALID_ARG"),  # block masks are per query tile
    (dict(regroup=1, vote_threshold=4), "TRA_ERR_INVALID_ARG"),  # so are vote-filtered lists
    (dict(group_rows=1), "TRA_ERR_INVALID_ARG"),  # attention groups have 2 or 3 query-tile rows
    (dict(group_rows=4), "TRA_ERR_INVALID_ARG"),
    (dict(group_rows=3, regroup=1), "TRA_ERR_INVALID_ARG"),  # regrouping orders 2 x 2 groups
    # every frame active (decay 1) over 2,000 frames at 88 levels: the radius
    # table's active entries (88 x 2,000) exceed what the tile-list kernel stages
    (dict(grid=(2000, 4, 4), heads=1, dtype=torch.float32, decay=1.0, budget_max=float(2 ** 20)),
     "TRA_ERR_INVALID_ARG"),
])
def test_validation_rejects(kw, code):
    with pytest.raises(tra.TraError) as ei:
        _validate(**kw)
    assert ei.value.name == code


def test_validation_accepts_regroup():
    _validate(regroup=1)
    _validate(regroup=1, generator=3)
    _validate(regroup=1, group_rows=2)


def test_validation_accepts_group_rows():
    for r in (0, 2, 3):
        _validate(group_rows=r)
        _validate(group_rows=r, dtype=torch.float32)


def test_validation_accepts_large_fp32_head():
    # the per-head byte limit applies to the bf16 path only
    _validate(grid=(2, 32767, 256), heads=1, dtype=torch.float32)


def test_validation_accepts_every_workload():
    for cfg in CONFIGS.values():
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        tra.validate(cfg.batch, cfg.heads, (cfg.T, cfg.H, cfg.W), cfg.head_dim, dt, **cfg.params())


@pytest.mark.parametrize("name", list(CONFIGS))
def test_radius_table_matches_oracle(name):
    cfg = CONFIGS[name]
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    r2, r0sq, k_lo = tra.radius_table((cfg.T, cfg.H, cfg.W), dt, cfg.head_dim, **cfg.params())
    ref = O.radius_table(cfg.params(), cfg.T)
    assert k_lo == O.level_range(cfg.params())[0]
    assert np.array_equal(r2.astype(np.int64), ref)


@pytest.mark.parametrize("r", [0.0, 1.0, 2.5, 7.0, 40.0])
@pytest.mark.parametrize("decay", [1.0, 0.5, 0.35])
def test_radius_table_override_matches_oracle(r, decay):
    cfg = small_workload(T=9, radius_override=r, decay=decay)
    r2, _, k_lo = tra.radius_table((cfg.T, cfg.H, cfg.W), torch.bfloat16, 128, **cfg.params())
    assert k_lo == -1
    assert np.array_equal(r2.astype(np.int64), O.radius_table(cfg.params(), cfg.T))


@pytest.mark.parametrize("gen,r,T", [(1, 0.0, 5), (1, 7.9, 12), (1, 40.0, 66), (2, 0.0, 4), (2, 5.5, 21),
                                     (2, 60.0, 66)])
def test_radius_table_generators_match_oracle(gen, r, T):
    cfg = small_workload(T=T, radius_override=r, generator=gen)
    r2, _, k_lo = tra.radius_table((cfg.T, cfg.H, cfg.W), torch.bfloat16, 128, **cfg.params())
    assert k_lo == -1
    assert np.array_equal(r2.astype(np.int64), O.radius_table(cfg.params(), cfg.T))


@pytest.mark.parametrize("r,bmax,T", [(-1.0, 2048.0, 4), (-1.0, 9000.0, 21), (0.0, 2048.0, 3), (33.7, 2048.0, 5)])
def test_radius_table_window_matches_oracle(r, bmax, T):
    cfg = small_workload(T=T, radius_override=r, generator=3, budget_max=bmax)
    r2, _, k_lo = tra.radius_table((cfg.T, cfg.H, cfg.W), torch.bfloat16, 128, **cfg.params())
    assert np.array_equal(r2.astype(np.int64), O.radius_table(cfg.params(), cfg.T))


def test_binding_rejects_host_tensors():
    q = torch.zeros((1, 1, 8 * 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tra.plan(q, q, grid=(1, 8, 8))


def _shape(dtype=1, head_dim=128, grid=(2, 8, 8)):
    T, H, W = grid
    return tra._Shape(1, 2, T, H, W, head_dim, dtype)


def test_dense_attention_rejects_bad_arguments_before_any_device_call():
    """Argument checks of the dense warm-up entry point run on the host."""
    lib = tra.load_library()
    P = ctypes.c_void_p
    ok = P(4096)  # never dereferenced: every call below fails validation first
    name = lambda st: lib.tra_status_string(st).decode()
    assert name(lib.tra_dense_attention(None, ok, ok, ok, P(8192), None, None)) == "TRA_ERR_INVALID_ARG"
    assert name(lib.tra_dense_attention(ctypes.byref(_shape(head_dim=96)), ok, ok, ok, P(8192), None, None)) \
        == "TRA_ERR_DTYPE"
    assert name(lib.tra_dense_attention(ctypes.byref(_shape()), None, ok, ok, P(8192), None, None)) \
        == "TRA_ERR_INVALID_ARG"
    assert name(lib.tra_dense_attention(ctypes.byref(_shape()), P(4100), ok, ok, P(8192), None, None)) \
        == "TRA_ERR_INVALID_ARG"  # misaligned
    assert name(lib.tra_dense_attention(ctypes.byref(_shape()), ok, ok, ok, ok, None, None)) \
        == "TRA_ERR_INVALID_ARG"  # o aliases q
    assert name(lib.tra_dense_attention(ctypes.byref(_shape()), ok, ok, ok, P(8192), P(8194), None)) \
        == "TRA_ERR_INVALID_ARG"  # misaligned entropy


def test_plan_from_entropy_rejects_bad_arguments_before_any_device_call():
    lib = tra.load_library()
    out = ctypes.c_void_p()
    prm = tra._make_params({})
    name = lambda st: lib.tra_status_string(st).decode()
    assert name(lib.tra_plan_create_from_entropy(ctypes.byref(_shape()), ctypes.byref(prm), None, None,
                                                 ctypes.byref(out))) == "TRA_ERR_INVALID_ARG"
    assert out.value is None
    bad = tra._make_params({"decay": 0.0})
    assert name(lib.tra_plan_create_from_entropy(ctypes.byref(_shape()), ctypes.byref(bad),
                                                 ctypes.c_void_p(4096), None, ctypes.byref(out))) \
        == "TRA_ERR_INVALID_ARG"
    assert name(lib.tra_plan_rebuild_from_entropy(None, ctypes.c_void_p(4096), None)) == "TRA_ERR_INVALID_ARG"


def test_plan_import_rejects_bad_levels_before_any_device_call():
    """tra_plan_import checks every level against the radius table on the host
    and allocates nothing when one is outside it."""
    import numpy as np
    lib = tra.load_library()
    out = ctypes.c_void_p()
    name = lambda st: lib.tra_status_string(st).decode()
    sh = _shape(grid=(2, 8, 8))
    n = sh.B * sh.heads * sh.T * sh.H * sh.W
    prm = tra._make_params({})
    r2, _, k_lo = tra.radius_table((2, 8, 8))
    k_hi = k_lo + r2.shape[0] - 1
    P = ctypes.c_void_p
    assert name(lib.tra_plan_import(ctypes.byref(sh), ctypes.byref(prm), None, None, None, None,
                                    ctypes.byref(out))) == "TRA_ERR_INVALID_ARG"
    assert name(lib.tra_plan_import(ctypes.byref(sh), ctypes.byref(prm), P(4096), None, None, None,
                                    None)) == "TRA_ERR_INVALID_ARG"
    for bad in (k_lo - 1, k_hi + 1, -1):
        lv = np.full(n, k_lo, dtype=np.int16)
        lv[n - 1] = bad
        assert name(lib.tra_plan_import(ctypes.byref(sh), ctypes.byref(prm), lv.ctypes.data_as(P), None, None,
                                        None, ctypes.byref(out))) == "TRA_ERR_INVALID_ARG"
        assert out.value is None
    # under radius_override every level must be -1
    fixed = tra._make_params({"radius_override": 3.0})
    lv = np.zeros(n, dtype=np.int16)
    assert name(lib.tra_plan_import(ctypes.byref(sh), ctypes.byref(fixed), lv.ctypes.data_as(P), None, None,
                                    None, ctypes.byref(out))) == "TRA_ERR_INVALID_ARG"
    bad_prm = tra._make_params({"decay": 0.0})
    lv = np.full(n, k_lo, dtype=np.int16)
    assert name(lib.tra_plan_import(ctypes.byref(sh), ctypes.byref(bad_prm), lv.ctypes.data_as(P), None, None,
                                    None, ctypes.byref(out))) == "TRA_ERR_INVALID_ARG"


def test_binding_dense_checks_shapes_on_host():
    q = torch.zeros((1, 1, 2 * 8 * 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tra.dense_attention(q, q, q, grid=(2, 8, 8))  # host tensors
    with pytest.raises(ValueError):
        tra.dense_attention(q, q[..., :32].contiguous(), q, grid=(2, 8, 8))
    with pytest.raises(ValueError):
        tra.plan_from_entropy(torch.zeros((1, 1, 5)), grid=(2, 8, 8), head_dim=64)


def test_schedule_rejects_bad_arguments_before_any_device_call():
    lib = tra.load_library()
    out = ctypes.c_void_p()
    prm = tra._make_params({})
    name = lambda st: lib.tra_status_string(st).decode()
    for sp, code in [(tra._SchedParams(0, 0, -1.0), "TRA_ERR_INVALID_ARG"),
                     (tra._SchedParams(1, -1, -1.0), "TRA_ERR_INVALID_ARG"),
                     (tra._SchedParams(1, 0, float("nan")), "TRA_ERR_INVALID_ARG")]:
        assert name(lib.tra_schedule_create(ctypes.byref(_shape()), ctypes.byref(prm), ctypes.byref(sp),
                                            ctypes.byref(out))) == code
        assert out.value is None
    assert name(lib.tra_schedule_create(ctypes.byref(_shape(head_dim=80)), ctypes.byref(prm),
                                        ctypes.byref(tra._SchedParams(1, 0, -1.0)), ctypes.byref(out))) \
        == "TRA_ERR_DTYPE"
    assert name(lib.tra_schedule_step(None, None, None, None, None, None, None)) == "TRA_ERR_INVALID_ARG"


# ---------------------------------------------------------------------------
# Failure handling forced from the host (TRA_FAULT), with no device work: the
# injected failure comes before any runtime call that would need a GPU.
# ---------------------------------------------------------------------------
@pytest.fixture
def fault(monkeypatch):
    def arm(value):
        monkeypatch.setenv("TRA_FAULT", value)
    yield arm


def _name(st):
    return tra.load_library().tra_status_string(st).decode()


def test_injected_allocation_failure_in_plan_create(fault):
    lib = tra.load_library()
    fault("alloc")
    out = ctypes.c_void_p(1234)
    prm = tra._make_params({})
    q = ctypes.c_void_p(4096)
    st = lib.tra_plan_create(ctypes.byref(_shape()), ctypes.byref(prm), q, q, None, ctypes.byref(out))
    assert _name(st) == "TRA_ERR_OOM"
    assert out.value is None
    assert b"out of memory" in lib.tra_last_error().lower() or b"alloc" in lib.tra_last_error()
    fault("alloc:1")
    st = lib.tra_plan_create_from_entropy(ctypes.byref(_shape()), ctypes.byref(prm), q, None, ctypes.byref(out))
    assert _name(st) == "TRA_ERR_OOM" and out.value is None


def test_injected_allocation_failure_in_schedule_create(fault):
    lib = tra.load_library()
    fault("alloc")
    out = ctypes.c_void_p(1234)
    st = lib.tra_schedule_create(ctypes.byref(_shape()), ctypes.byref(tra._make_params({})),
                                 ctypes.byref(tra._SchedParams(2, 0, 0.1)), ctypes.byref(out))
    assert _name(st) == "TRA_ERR_OOM" and out.value is None


def test_injected_launch_failure_is_distinct(fault):
    lib = tra.load_library()
    fault("launch")
    P = ctypes.c_void_p
    st = lib.tra_dense_attention(ctypes.byref(_shape()), P(4096), P(8192), P(12288), P(16384), None, None)
    assert _name(st) == "TRA_ERR_HIP"
    assert b"injected launch failure" in lib.tra_last_error()


@pytest.mark.parametrize("value", ["", "none", "alloc:0", "launch:x", "allocate"])
def test_unrecognised_fault_settings_inject_nothing(fault, value):
    """A malformed TRA_FAULT arms nothing: the call then fails for its real
    reason on this machine (no GPU), not with an injected status."""
    lib = tra.load_library()
    fault(value)
    P = ctypes.c_void_p
    lib.tra_dense_attention(ctypes.byref(_shape()), P(4096), P(8192), P(12288), P(16384), None, None)
    assert b"injected" not in lib.tra_last_error()


def test_plan_invalid_status_string():
    assert _name(8) == "TRA_ERR_PLAN_INVALID"


def test_null_plan_is_rejected_by_every_plan_call():
    lib = tra.load_library()
    P = ctypes.c_void_p
    n, m = ctypes.c_int64(), ctypes.c_int64()
    assert _name(lib.tra_attention(None, P(4096), P(4096), P(4096), P(8192), None)) == "TRA_ERR_INVALID_ARG"
    assert _name(lib.tra_plan_stats(None, ctypes.byref(n), ctypes.byref(m), None)) == "TRA_ERR_INVALID_ARG"
    assert _name(lib.tra_plan_drift(None, P(4096), P(4096), ctypes.byref(n), None)) == "TRA_ERR_INVALID_ARG"
    assert _name(lib.tra_plan_export(None, None, None, None, None, None, None, None)) == "TRA_ERR_INVALID_ARG"
    assert _name(lib.tra_plan_rebuild(None, P(4096), P(4096), None)) == "TRA_ERR_INVALID_ARG"
    lib.tra_plan_destroy(None)  # a no-op
