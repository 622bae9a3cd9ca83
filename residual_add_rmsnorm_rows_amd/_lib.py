"""ctypes view of the C ABI declared in include/rmsnorm_rows.h.

Loads the in-tree ``librmsnorm_rows.so``; there is no fallback of any kind:
if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "librmsnorm_rows.so")

# rn_status codes
RN_OK = 0
RN_ERR_INVALID_ARG = 1
RN_ERR_UNSUPPORTED = 2
RN_ERR_MISALIGNED = 3
RN_ERR_HIP = 4

# dtype codes and flag layout
RN_DTYPE_BF16 = 0
RN_DTYPE_F32 = 1
RN_DTYPE_FP8_E4M3FN = 2
RN_DTYPE_FP4_E2M1 = 3  # outputs only
RN_FLAGS_X_SHIFT = 0
RN_FLAGS_RES_SHIFT = 2
RN_FLAGS_W_SHIFT = 4
RN_FLAGS_OUT_SHIFT = 6
RN_FLAG_WEIGHT_PLUS_ONE = 1 << 8
RN_FLAGS_SCALE_SHIFT = 9
SCALE_SCHEMES = {"row": 0, "group128": 1, "mx32": 2, "nv16": 3}

RN_KERNEL_ROWS = 0
RN_KERNEL_HEADS = 1

DTYPE_CODES = {"bf16": RN_DTYPE_BF16, "f32": RN_DTYPE_F32, "fp8_e4m3fn": RN_DTYPE_FP8_E4M3FN,
               "fp4_e2m1": RN_DTYPE_FP4_E2M1}

# Every symbol include/rmsnorm_rows.h declares.
EXPORTED_SYMBOLS = (
    "rmsnorm_fwd", "rmsnorm_fwd_ex", "rmsnorm_fwd_config", "qknorm_fwd", "qknorm_fwd_config",
    "rmsnorm_query_config", "qknorm_query_config", "silu_mul_fwd", "silu_mul_fwd_config",
    "silu_mul_query_config", "rn_launch_empty", "rn_launch_copy", "rn_status_string", "rn_last_error",
    "rn_abi_version", "rmsnorm_fwd_partials", "rmsnorm_fwd_partials_config", "rmsnorm_partials_query_config",
    "rmsnorm_fwd_call",
)
ABI_VERSION = 4
MAX_PARTIALS = 8


def make_flags(x: str, res: str | None, w: str, out: str, weight_plus_one: bool,
               scale_scheme: str = "row") -> int:
    f = DTYPE_CODES[x] << RN_FLAGS_X_SHIFT
    f |= SCALE_SCHEMES[scale_scheme] << RN_FLAGS_SCALE_SHIFT
    f |= DTYPE_CODES[res or "bf16"] << RN_FLAGS_RES_SHIFT
    f |= DTYPE_CODES[w] << RN_FLAGS_W_SHIFT
    f |= DTYPE_CODES[out] << RN_FLAGS_OUT_SHIFT
    if weight_plus_one:
        f |= RN_FLAG_WEIGHT_PLUS_ONE
    return f


class LaunchConfig(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("vec", ctypes.c_int32),
        ("waves_per_row", ctypes.c_int32),
        ("vecs_per_lane", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
        ("rows_per_lane", ctypes.c_int32),
        ("block_threads", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("grid", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}


class RmsnormCall(ctypes.Structure):
    """rn_rmsnorm_call: the arguments of one rmsnorm_fwd_ex call."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("residual", ctypes.c_void_p),
        ("weight", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("residual_out", ctypes.c_void_p),
        ("out_scale", ctypes.c_void_p),
        ("out_amax", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("eps", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("stream", ctypes.c_void_p),
    ]


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_fp = ctypes.POINTER(ctypes.c_float)

_SIGNATURES = {
    "rmsnorm_fwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _u32, _vp], ctypes.c_int),
    "rmsnorm_fwd_ex": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _u32, _vp], ctypes.c_int),
    "rmsnorm_fwd_call": ([ctypes.POINTER(RmsnormCall)], ctypes.c_int),
    "rmsnorm_fwd_config": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _u32,
                            ctypes.POINTER(LaunchConfig), _vp], ctypes.c_int),
    "qknorm_fwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i64, _f32, _u32, _vp],
                   ctypes.c_int),
    "qknorm_fwd_config": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i64, _f32, _u32,
                           ctypes.POINTER(LaunchConfig), _vp], ctypes.c_int),
    "rmsnorm_fwd_partials": ([ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _u32,
                              _vp], ctypes.c_int),
    "rmsnorm_fwd_partials_config": ([ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32,
                                     _u32, ctypes.POINTER(LaunchConfig), _vp], ctypes.c_int),
    "rmsnorm_query_config": ([_i64, _i64, _u32, _i32, _i32, ctypes.POINTER(LaunchConfig)], ctypes.c_int),
    "rmsnorm_partials_query_config": ([_i64, _i64, _i32, _u32, _i32, _i32, ctypes.POINTER(LaunchConfig)],
                                      ctypes.c_int),
    "qknorm_query_config": ([_i64, _i32, _i32, _i32, _u32, _i32, ctypes.POINTER(LaunchConfig)], ctypes.c_int),
    "silu_mul_fwd": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _u32, _vp], ctypes.c_int),
    "silu_mul_fwd_config": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _u32, ctypes.POINTER(LaunchConfig), _vp],
                            ctypes.c_int),
    "silu_mul_query_config": ([_i64, _i64, _u32, _i32, ctypes.POINTER(LaunchConfig)], ctypes.c_int),
    "rn_launch_empty": ([_vp], ctypes.c_int),
    "rn_launch_copy": ([_vp, _vp, _i64, _vp], ctypes.c_int),
    "rn_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "rn_last_error": ([], ctypes.c_char_p),
    "rn_abi_version": ([], ctypes.c_int32),
}

_lock = threading.Lock()
_lib = None


class RNError(RuntimeError):
    """A non-OK rn_status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library {LIB_PATH} is not built; run "
                    "`python -c 'import __graft_entry__ as g; g.build()'` or "
                    "`python -m residual_add_rmsnorm_rows_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGNATURES.items():
                fn = getattr(handle, name)
                fn.argtypes = args
                fn.restype = res
            if handle.rn_abi_version() != ABI_VERSION:
                raise RuntimeError(f"{LIB_PATH}: ABI version {handle.rn_abi_version()} != {ABI_VERSION}")
            _lib = handle
    return _lib


def check(status: int) -> None:
    """Raise RNError for a non-OK status, with the library's message."""
    if status != RN_OK:
        L = lib()
        detail = L.rn_last_error().decode()
        raise RNError(status, f"{L.rn_status_string(status).decode()}: {detail}")
