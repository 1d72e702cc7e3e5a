"""Python binding of ``libstepq.so`` — argument marshalling only.

Every function keeps the name of the C entry point it wraps (see
``include/stepq.h``); device arguments are torch tensors (their data pointers
are passed through) or raw integer addresses.  All computation runs in the
library's HIP kernels; if the library is not built this module raises instead
of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SQ_LIBRARY names another build of the library to load instead (the tests'
# checked host build); by default the in-tree libstepq.so
LIB_PATH = os.environ.get("SQ_LIBRARY") or os.path.join(_HERE, "libstepq.so")

SQ_OK, SQ_EINVAL, SQ_EUNSUPPORTED, SQ_ESLOT_RANGE, SQ_EDUP_SLOT = 0, 1, 2, 3, 4
SQ_EPLAN_MISMATCH, SQ_EBUDGET, SQ_EHIP, SQ_ENOMEM, SQ_ENONFINITE = 5, 6, 7, 8, 9
SQ_MODE_UNIFORM, SQ_MODE_STEP, SQ_MODE_WINDOW = 0, 1, 2
SQ_KIND_GDN, SQ_KIND_KDA = 0, 1
SQ_PIVOT_BITS = 16

EXPORTED = (
    "sq_calibrate_bits", "sq_plan_create_step", "sq_plan_create_uniform",
    "sq_plan_create_window", "sq_plan_create_window_lowrank", "sq_plan_query", "sq_plan_destroy", "sq_plan_device_bytes",
    "sq_plan_upload", "sq_pool_bytes", "sq_pool_init", "sq_pool_pack", "sq_pool_unpack",
    "sq_decode_step", "sq_window_flush", "sq_quantize_tiles", "sq_max_head_bytes",
    "sq_dense_step", "sq_prefill_chunk", "sq_prefill_chunkwise", "sq_calib_gate_stats", "sq_impact_factors", "sq_calib_distortion",
    "sq_calib_distortion_noalloc", "sq_last_error",
)


class StepqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"stepq status {status}: {message}")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("kind", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("uniform_bits", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_units", ctypes.c_int32), ("slot_bytes", ctypes.c_int64),
                ("payload_bytes", ctypes.c_int64), ("analytic_bytes", ctypes.c_int64),
                ("head_off", ctypes.POINTER(ctypes.c_int64)),
                ("unit_bits", ctypes.POINTER(ctypes.c_int32)),
                ("w", ctypes.POINTER(ctypes.c_float)), ("window_c_floor", ctypes.c_float),
                ("window_rank", ctypes.c_int32), ("window_iters", ctypes.c_int32)]


class _Stats(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("n_cand", ctypes.c_int32),
                ("cand_bits", ctypes.POINTER(ctypes.c_int32)),
                ("ell", ctypes.POINTER(ctypes.c_double)),
                ("dist", ctypes.POINTER(ctypes.c_double)),
                ("omega", ctypes.POINTER(ctypes.c_double))]


class _Opts(ctypes.Structure):
    _fields_ = [("nominal_bits", ctypes.c_double), ("pivot_frac", ctypes.c_double),
                ("gamma", ctypes.c_double), ("horizon", ctypes.c_int32),
                ("omega_floor_rel", ctypes.c_double)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SZ = ctypes.POINTER(ctypes.c_size_t)
_PP = ctypes.POINTER(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "quantized_recurrent_state_decode_amd._build.build()")
        # One HIP runtime per process: torch's bundled runtime carries the same
        # soname as the one the library links, so loading torch first makes the
        # library bind to it and share its device memory and streams.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "sq_calibrate_bits": [ctypes.POINTER(_Stats), ctypes.POINTER(_Opts), _PP],
            "sq_plan_create_step": [_I32, _I32, _I32, _I32, _P, _P, _PP],
            "sq_plan_create_uniform": [_I32, _I32, _I32, _I32, _PP],
            "sq_plan_create_window": [_I32, _I32, _I32, _I32, _F32, _PP],
            "sq_plan_create_window_lowrank": [_I32, _I32, _I32, _I32, _F32, _I32, _I32, _PP],
            "sq_plan_query": [_P, ctypes.POINTER(_Desc)],
            "sq_plan_destroy": [_P],
            "sq_plan_device_bytes": [_P, _SZ],
            "sq_plan_upload": [_P, _P, _P],
            "sq_pool_bytes": [_P, _I64, _SZ],
            "sq_pool_init": [_P, _P, _P, _I64, _P],
            "sq_pool_pack": [_P, _P, _P, _I64, _P, _I32, _P, _P],
            "sq_pool_unpack": [_P, _P, _P, _I64, _P, _I32, _P, _P],
            "sq_decode_step": [_P, _P, _P, _I64, _P, _I32, _P, _P, _P, _P, _P, _P, _P],
            "sq_window_flush": [_P, _P, _P, _I64, _P, _I32, _P],
            "sq_quantize_tiles": [_P, _P, _P, _I32, _P, _P, _P],
            "sq_max_head_bytes": [_P, _SZ],
            "sq_dense_step": [_I32, _I32, _I32, _I32, _P, _I64, _P, _I32, _P, _P, _P, _P,
                              _P, _P, _P],
            "sq_prefill_chunk": [_I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                 _P],
            "sq_prefill_chunkwise": [_I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                     _P, _P],
            "sq_calib_gate_stats": [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P],
            "sq_impact_factors": [_I32, _I32, _P, ctypes.c_double, ctypes.c_double, _P],
            "sq_calib_distortion": [_P, _P, _I32, _P, _P, _I32, _P, _P],
            "sq_calib_distortion_noalloc": [_P, _P, _I32, _P, _I32, _P, _P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _I32
        L.sq_last_error.argtypes = []
        L.sq_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def sq_last_error() -> str:
    return lib().sq_last_error().decode()


def _check(status: int) -> None:
    if status != SQ_OK:
        raise StepqError(status, sq_last_error())


def _ptr(x, dtype=None):
    """Device/host address of a torch tensor (contiguous, dtype-checked) or int."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if isinstance(x, torch.Tensor):
        if not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        if dtype is not None and x.dtype != dtype:
            raise TypeError(f"expected {dtype}, got {x.dtype}")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owner of an ``sq_plan*`` handle (destroyed with the object)."""

    def __init__(self, handle: int):
        self.handle = handle

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.sq_plan_destroy(self.handle)
            self.handle = None

    @property
    def _as_parameter_(self):
        return ctypes.c_void_p(self.handle)


def _new_plan(fn, *args) -> Plan:
    out = ctypes.c_void_p()
    _check(fn(*args, ctypes.byref(out)))
    return Plan(out.value)


def sq_plan_create_uniform(heads: int, d_k: int, d_v: int, bits: int) -> Plan:
    return _new_plan(lib().sq_plan_create_uniform, heads, d_k, d_v, bits)


def sq_plan_create_window(heads: int, d_k: int, d_v: int, p: int, c_floor: float = 1e-6) -> Plan:
    return _new_plan(lib().sq_plan_create_window, heads, d_k, d_v, p, c_floor)


def sq_plan_create_window_lowrank(heads: int, d_k: int, d_v: int, p: int, rank: int,
                                  power_iters: int = 4, c_floor: float = 1e-6) -> Plan:
    return _new_plan(lib().sq_plan_create_window_lowrank, heads, d_k, d_v, p, c_floor, rank,
                     power_iters)


def sq_plan_create_step(kind: int, heads: int, d_k: int, d_v: int, unit_bits, w) -> Plan:
    ub = np.ascontiguousarray(unit_bits, dtype=np.int32)
    ww = np.ascontiguousarray(w, dtype=np.float32)
    return _new_plan(lib().sq_plan_create_step, kind, heads, d_k, d_v,
                     ub.ctypes.data, ww.ctypes.data)


def sq_calibrate_bits(stats: dict, opts: dict) -> Plan:
    """stats: kind, heads, d_k, d_v, cand_bits, ell [U], dist [U, n_cand],
    omega [heads, d_k]; opts: nominal_bits, pivot_frac, gamma, horizon,
    omega_floor_rel."""
    cand = np.ascontiguousarray(stats["cand_bits"], dtype=np.int32)
    ell = np.ascontiguousarray(stats["ell"], dtype=np.float64)
    dist = np.ascontiguousarray(stats["dist"], dtype=np.float64)
    omega = np.ascontiguousarray(stats["omega"], dtype=np.float64)
    st = _Stats(stats["kind"], stats["heads"], stats["d_k"], stats["d_v"], len(cand),
                cand.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                ell.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                dist.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                omega.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    op = _Opts(opts.get("nominal_bits", 6.0), opts.get("pivot_frac", 0.0),
               opts.get("gamma", 0.25), opts.get("horizon", 2048),
               opts.get("omega_floor_rel", 1e-12))
    return _new_plan(lib().sq_calibrate_bits, ctypes.byref(st), ctypes.byref(op))


def sq_plan_query(plan: Plan) -> dict:
    d = _Desc()
    _check(lib().sq_plan_query(plan, ctypes.byref(d)))
    out = {k: getattr(d, k) for k in ("mode", "kind", "heads", "d_k", "d_v", "uniform_bits",
                                      "window", "n_units", "slot_bytes", "payload_bytes",
                                      "analytic_bytes", "window_c_floor", "window_rank",
                                      "window_iters")}
    out["head_off"] = np.ctypeslib.as_array(d.head_off, (d.heads,)).copy()
    out["unit_bits"] = (np.ctypeslib.as_array(d.unit_bits, (d.n_units,)).copy()
                        if d.n_units else None)
    out["w"] = (np.ctypeslib.as_array(d.w, (d.heads * d.d_k,)).copy().reshape(d.heads, d.d_k)
                if bool(d.w) else None)
    return out


def _size(fn, *args) -> int:
    n = ctypes.c_size_t()
    _check(fn(*args, ctypes.byref(n)))
    return n.value


def sq_plan_device_bytes(plan: Plan) -> int:
    return _size(lib().sq_plan_device_bytes, plan)


def sq_max_head_bytes(plan: Plan) -> int:
    return _size(lib().sq_max_head_bytes, plan)


def sq_pool_bytes(plan: Plan, n_slots: int) -> int:
    return _size(lib().sq_pool_bytes, plan, n_slots)


def sq_plan_upload(plan: Plan, dev_plan, stream=None) -> None:
    _check(lib().sq_plan_upload(plan, _ptr(dev_plan), _stream(stream)))


def sq_pool_init(plan, dev_plan, pool, n_slots, stream=None) -> None:
    _check(lib().sq_pool_init(plan, _ptr(dev_plan), _ptr(pool), n_slots, _stream(stream)))


def _f32():
    import torch
    return torch.float32


def _i32():
    import torch
    return torch.int32


def sq_pool_pack(plan, dev_plan, pool, n_slots, slots, batch, S, stream=None) -> None:
    _check(lib().sq_pool_pack(plan, _ptr(dev_plan), _ptr(pool), n_slots, _ptr(slots, _i32()),
                              batch, _ptr(S, _f32()), _stream(stream)))


def sq_pool_unpack(plan, dev_plan, pool, n_slots, slots, batch, S_out, stream=None) -> None:
    _check(lib().sq_pool_unpack(plan, _ptr(dev_plan), _ptr(pool), n_slots, _ptr(slots, _i32()),
                                batch, _ptr(S_out, _f32()), _stream(stream)))


def sq_decode_step(plan, dev_plan, pool, n_slots, slots, batch, q, k, v, beta, gate, y,
                   stream=None) -> None:
    f = _f32()
    _check(lib().sq_decode_step(plan, _ptr(dev_plan), _ptr(pool), n_slots, _ptr(slots, _i32()),
                                batch, _ptr(q, f), _ptr(k, f), _ptr(v, f), _ptr(beta, f),
                                _ptr(gate, f), _ptr(y, f), _stream(stream)))


def sq_window_flush(plan, dev_plan, pool, n_slots, slots, batch, stream=None) -> None:
    _check(lib().sq_window_flush(plan, _ptr(dev_plan), _ptr(pool), n_slots, _ptr(slots, _i32()),
                                 batch, _stream(stream)))


def sq_quantize_tiles(plan, dev_plan, X, n_tiles, head_ids, packed_out, stream=None) -> None:
    _check(lib().sq_quantize_tiles(plan, _ptr(dev_plan), _ptr(X, _f32()), n_tiles,
                                   _ptr(head_ids, _i32()), _ptr(packed_out), _stream(stream)))


def sq_dense_step(kind, heads, d_k, d_v, S, n_slots, slots, batch, q, k, v, beta, gate, y,
                  stream=None) -> None:
    f = _f32()
    _check(lib().sq_dense_step(kind, heads, d_k, d_v, _ptr(S, f), n_slots, _ptr(slots, _i32()),
                               batch, _ptr(q, f), _ptr(k, f), _ptr(v, f), _ptr(beta, f),
                               _ptr(gate, f), _ptr(y, f), _stream(stream)))


def sq_prefill_chunk(kind, heads, d_k, d_v, batch, T, S, q, k, v, beta, gate, y,
                     stream=None) -> None:
    f = _f32()
    _check(lib().sq_prefill_chunk(kind, heads, d_k, d_v, batch, T, _ptr(S, f), _ptr(q, f),
                                  _ptr(k, f), _ptr(v, f), _ptr(beta, f), _ptr(gate, f),
                                  _ptr(y, f), _stream(stream)))


def sq_prefill_chunkwise(kind, heads, d_k, d_v, batch, T, S, q, k, v, beta, gate, y,
                         stream=None) -> None:
    f = _f32()
    _check(lib().sq_prefill_chunkwise(kind, heads, d_k, d_v, batch, T, _ptr(S, f), _ptr(q, f),
                                      _ptr(k, f), _ptr(v, f), _ptr(beta, f), _ptr(gate, f),
                                      _ptr(y, f), _stream(stream)))


def sq_calib_gate_stats(kind, heads, d_k, n, q, k, beta, gate, log_sum, omega_sum,
                        stream=None) -> None:
    import torch
    f, d = _f32(), torch.float64
    _check(lib().sq_calib_gate_stats(kind, heads, d_k, n, _ptr(q, f), _ptr(k, f), _ptr(beta, f),
                                     _ptr(gate, f), _ptr(log_sum, d), _ptr(omega_sum, d),
                                     _stream(stream)))


def sq_impact_factors(omega, gamma: float = 0.25, floor_rel: float = 1e-12) -> np.ndarray:
    """omega: host float64 [heads, d_k] -> w float32 [heads, d_k]."""
    om = np.ascontiguousarray(omega, dtype=np.float64)
    heads, d_k = om.shape
    w = np.zeros((heads, d_k), dtype=np.float32)
    _check(lib().sq_impact_factors(heads, d_k, om.ctypes.data, gamma, floor_rel, w.ctypes.data))
    return w


def sq_calib_distortion(plan, dev_plan, n, S, packed, per_row, dist_sum, stream=None) -> None:
    import torch
    _check(lib().sq_calib_distortion(plan, _ptr(dev_plan), n, _ptr(S, _f32()), _ptr(packed),
                                     1 if per_row else 0, _ptr(dist_sum, torch.float64),
                                     _stream(stream)))


def sq_calib_distortion_noalloc(plan, dev_plan, n, S, per_row, dist_sum, stream=None) -> None:
    import torch
    _check(lib().sq_calib_distortion_noalloc(plan, _ptr(dev_plan), n, _ptr(S, _f32()),
                                             1 if per_row else 0, _ptr(dist_sum, torch.float64),
                                             _stream(stream)))


def device_plan(plan: Plan, device="cuda", stream=None):
    """Allocate (torch) and fill the device copy of a plan's tables."""
    import torch
    buf = torch.zeros(sq_plan_device_bytes(plan), dtype=torch.uint8, device=device)
    sq_plan_upload(plan, buf, stream)
    return buf
