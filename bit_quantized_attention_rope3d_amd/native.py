"""ctypes declarations of libra_attn.so (the C ABI in include/ra_attn.h).

Argument marshalling only.  The library is loaded from this package's
directory; if it is missing the import of this module fails with an error that
says how to build it -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra_attn.so")

c_i32, c_i64, c_f64, c_size, c_void = (ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                       ctypes.c_size_t, ctypes.c_void_p)

RA_OK = 0
STATUS = ["RA_OK", "RA_ERR_INVALID_ARG", "RA_ERR_SHAPE", "RA_ERR_SEGMENTS", "RA_ERR_DTYPE",
          "RA_ERR_ALIGNMENT", "RA_ERR_WORKSPACE", "RA_ERR_UNSUPPORTED", "RA_ERR_OOM", "RA_ERR_HIP"]
ROT = {"none": 0, "interleaved": 1, "half": 2, "full": 3}
PREC = {"int4": 0, "bf16": 1}
DT = {"f32": 0, "bf16": 1}


class RaShape(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("heads", c_i32), ("head_dim", c_i32),
                ("grid_f", c_i32), ("grid_h", c_i32), ("grid_w", c_i32),
                ("seg", c_i32 * 3)]


class RaOpts(ctypes.Structure):
    _fields_ = [("rot", c_i32), ("prec", c_i32), ("in_dtype", c_i32), ("out_dtype", c_i32),
                ("rope_theta", c_f64), ("softmax_scale", c_f64), ("p_mode", c_i32),
                ("v_hadamard", c_i32)]


class RaSchedule(ctypes.Structure):
    _fields_ = [("steps_head", c_i32), ("steps_tail", c_i32),
                ("blocks_head", c_i32), ("blocks_tail", c_i32)]


class RaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__("%s: %s (%s)" % (where, name, message))
        self.status = status
        self.name = name


_SIGS = {
    "ra_opts_default": (c_i32, [ctypes.POINTER(RaOpts)]),
    "ra_plan_create": (c_i32, [ctypes.POINTER(RaShape), ctypes.POINTER(RaOpts), ctypes.POINTER(c_void)]),
    "ra_plan_destroy": (c_i32, [c_void]),
    "ra_plan_workspace_size": (c_i32, [c_void, ctypes.POINTER(c_size)]),
    "ra_workspace_size": (c_i32, [ctypes.POINTER(RaShape), ctypes.POINTER(RaOpts), ctypes.POINTER(c_size)]),
    "ra_attn_fwd": (c_i32, [c_void, c_void, c_void, c_void, c_void, c_void, c_size, c_void]),
    "ra_attn_prologue": (c_i32, [c_void, c_void, c_void, c_void, c_void, c_size, c_void]),
    "ra_attn_main": (c_i32, [c_void, c_void, c_void, c_size, c_void]),
    "ra_attn_fwd_noalloc": (c_i32, [c_void, c_void, c_void, c_void, c_void, c_void]),
    "ra_attn_fwd_simple": (c_i32, [c_void, c_void, c_void, c_void] + [c_i32] * 13 + [c_void, c_size, c_void]),
    "ra_schedule_pick": (c_i32, [ctypes.POINTER(RaSchedule), c_i32, c_i32, c_i32, c_i32]),
    "ra_status_str": (ctypes.c_char_p, [c_i32]),
    "ra_last_error_message": (ctypes.c_char_p, []),
    "ra_plan_upload": (c_i32, [c_void]),
    "ra_pmap_thresholds": (c_i32, [c_i32, c_void]),
    "ra_pmap_table": (c_i32, [c_i32, c_void, c_size, ctypes.POINTER(c_i32)]),
    "ra_debug_row_digests": (c_i32, [c_void, c_void, c_void, c_size, c_void, c_void]),
    "ra_debug_prologue": (c_i32, [c_void, c_void, c_void, c_void, c_void, c_size,
                                  c_void, c_void, c_void, c_void, c_void, c_void, c_void]),
    "ra_debug_tile": (c_i32, [c_void, c_void, c_size, c_i32, c_i32, c_i32, c_i32,
                              c_void, c_void, c_void, c_void, c_void]),
    "ra_debug_pmap": (c_i32, [c_void, c_void, c_i64, c_i32, c_void]),
    "ra_debug_tables": (c_i32, [c_void, c_i32, c_void, c_void]),
    "ra_copy": (c_i32, [c_void, c_void, c_size, c_void]),
    "ra_bench_mfma_peak": (c_i32, [c_i32, c_i32, c_i32, c_void, c_void, ctypes.POINTER(ctypes.c_double), c_void]),
}

_lib = None
_lock = threading.Lock()


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    "libra_attn.so is not built (%s); run "
                    "`python -m bit_quantized_attention_rope3d_amd.build`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def last_error() -> str:
    return lib().ra_last_error_message().decode()


def check(rc: int, where: str) -> None:
    if rc != RA_OK:
        raise RaError(rc, where, last_error())


def status_str(code: int) -> str:
    return lib().ra_status_str(code).decode()


def make_shape(batch, heads, head_dim, grid, seg) -> RaShape:
    s = RaShape()
    s.batch, s.heads, s.head_dim = batch, heads, head_dim
    s.grid_f, s.grid_h, s.grid_w = grid
    s.seg[0], s.seg[1], s.seg[2] = seg
    return s


def make_opts(rot="half", prec="int4", in_dtype="bf16", out_dtype="f32", rope_theta=10000.0,
              softmax_scale=0.0, p_mode=0, v_hadamard=0) -> RaOpts:
    o = RaOpts()
    check(lib().ra_opts_default(ctypes.byref(o)), "ra_opts_default")
    o.rot = ROT[rot] if isinstance(rot, str) else int(rot)
    o.prec = PREC[prec] if isinstance(prec, str) else int(prec)
    o.in_dtype = DT[in_dtype] if isinstance(in_dtype, str) else int(in_dtype)
    o.out_dtype = DT[out_dtype] if isinstance(out_dtype, str) else int(out_dtype)
    o.rope_theta = float(rope_theta)
    o.softmax_scale = float(softmax_scale)
    o.p_mode = int(p_mode)
    o.v_hadamard = int(v_hadamard)
    return o
