"""ctypes view of ``libw4a16.so`` (the C ABI in ``include/w4a16.h``).

Loads the in-tree library only.  There is no fallback: if the library is missing
or fails to load, :func:`lib` raises.
"""

from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a16.so")

ABI_VERSION = 7
WORKSPACE_HEAD_BYTES = 147456   # W4A16_WORKSPACE_HEAD_BYTES
WORKSPACE_ERROR_OFFSET = 12928  # W4A16_WORKSPACE_ERROR_OFFSET
NOALLOC_SCRATCH_BYTES = 64 << 20  # W4A16_NOALLOC_SCRATCH_BYTES

W4A16_OK = 0
W4A16_ERR_INVALID_ARG = 1
W4A16_ERR_UNSUPPORTED = 2
W4A16_ERR_WORKSPACE = 3
W4A16_ERR_HIP = 4
W4A16_ERR_TIMEOUT = 5

W4A16_F32 = 0
W4A16_BF16 = 1

FORMATS = {"int": 0, "fp8": 1, "mxfp4": 2}   # w4a16_format
W4A16_FLAG_NO_COOPERATIVE = 1                  # w4a16_flags
MXFP4_METHODS = {"rtn": 0, "mse": 1}         # w4a16_mxfp4_method

EXPORTED = (
    "w4a16_abi_version",
    "w4a16_status_string",
    "w4a16_last_error",
    "rtn_quantize_pack",
    "fp8_quantize_pack",
    "mxfp4_quantize_pack",
    "moe_w4a16_workspace_size",
    "moe_w4a16_workspace_init",
    "moe_w4a16_workspace_check",
    "moe_w4a16_forward",
    "moe_w4a16_forward_timed",
    "moe_w4a16_forward_noalloc",
    "w4a16_linear_workspace_size",
    "w4a16_linear",
    "w4a16_stream_read",
)


class MoeArgs(C.Structure):
    """Mirror of ``moe_w4a16_args`` (field order and types must match the header)."""
    _fields_ = [
        ("T", C.c_int64), ("H", C.c_int64), ("I", C.c_int64), ("E", C.c_int64), ("top_k", C.c_int64),
        ("bits", C.c_int32), ("group", C.c_int32),
        ("x", C.c_void_p),
        ("router_logits", C.c_void_p),
        ("w13", C.c_void_p), ("s13", C.c_void_p), ("w2", C.c_void_p), ("s2", C.c_void_p),
        ("shared_bits", C.c_int32),
        ("shared_I", C.c_int64),
        ("shared_w13", C.c_void_p), ("shared_s13", C.c_void_p),
        ("shared_w2", C.c_void_p), ("shared_s2", C.c_void_p),
        ("residual", C.c_void_p),
        ("y", C.c_void_p),
        ("topk_ids", C.c_void_p), ("topk_w", C.c_void_p),
        ("expert_counts", C.c_void_p), ("expert_offsets", C.c_void_p), ("sorted_pairs", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
        ("router_w", C.c_void_p), ("shared_gate_w", C.c_void_p),
        ("logits_out", C.c_void_p), ("shared_gate_out", C.c_void_p),
        ("weight_format", C.c_int32),
        ("flags", C.c_int32),
    ]


class LinearArgs(C.Structure):
    """Mirror of ``w4a16_linear_args``."""
    _fields_ = [
        ("T", C.c_int64), ("K", C.c_int64), ("N", C.c_int64),
        ("bits", C.c_int32), ("group", C.c_int32), ("weight_format", C.c_int32),
        ("x", C.c_void_p), ("w", C.c_void_p), ("s", C.c_void_p), ("residual", C.c_void_p), ("y", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
    ]


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {message}")


_lib = None


def lib():
    """The loaded library (raises when it is missing or has the wrong ABI version)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m weight_only_int4_rtn_amd.build`")
    # torch first: its HIP runtime is then the one the library's libamdhip64 dependency
    # binds to.  Loaded the other way round, the process maps two HIP runtimes, and the
    # library's own one need not see the GPU that torch uses.
    import torch  # noqa: F401
    L = C.CDLL(LIB_PATH)
    L.w4a16_abi_version.restype = C.c_int
    L.w4a16_abi_version.argtypes = []
    L.w4a16_status_string.restype = C.c_char_p
    L.w4a16_status_string.argtypes = [C.c_int]
    L.w4a16_last_error.restype = C.c_char_p
    L.w4a16_last_error.argtypes = []
    L.rtn_quantize_pack.restype = C.c_int
    L.rtn_quantize_pack.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int,
                                    C.c_void_p, C.c_void_p, C.c_void_p]
    L.fp8_quantize_pack.restype = C.c_int
    L.fp8_quantize_pack.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                    C.c_void_p]
    L.mxfp4_quantize_pack.restype = C.c_int
    L.mxfp4_quantize_pack.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_void_p,
                                      C.c_void_p, C.c_void_p]
    L.moe_w4a16_workspace_size.restype = C.c_size_t
    L.moe_w4a16_workspace_size.argtypes = [C.c_int64] * 6
    L.moe_w4a16_workspace_init.restype = C.c_int
    L.moe_w4a16_workspace_init.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p]
    L.moe_w4a16_workspace_check.restype = C.c_int
    L.moe_w4a16_workspace_check.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p]
    L.moe_w4a16_forward.restype = C.c_int
    L.moe_w4a16_forward.argtypes = [C.POINTER(MoeArgs), C.c_void_p]
    L.w4a16_linear_workspace_size.restype = C.c_size_t
    L.w4a16_linear_workspace_size.argtypes = [C.c_int64] * 3
    L.w4a16_linear.restype = C.c_int
    L.w4a16_linear.argtypes = [C.POINTER(LinearArgs), C.c_void_p]
    L.moe_w4a16_forward_noalloc.restype = C.c_int
    L.moe_w4a16_forward_noalloc.argtypes = [C.POINTER(MoeArgs), C.c_void_p]
    L.moe_w4a16_forward_timed.restype = C.c_int
    L.moe_w4a16_forward_timed.argtypes = [C.POINTER(MoeArgs), C.c_void_p, C.c_int, C.POINTER(C.c_float),
                                          C.POINTER(C.c_char_p), C.POINTER(C.c_int)]
    L.w4a16_stream_read.restype = C.c_int
    L.w4a16_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
    if L.w4a16_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH}: ABI version {L.w4a16_abi_version()}, expected {ABI_VERSION}")
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().w4a16_status_string(status).decode()


def last_error() -> str:
    return lib().w4a16_last_error().decode()


def check(status: int, where: str) -> None:
    if status != W4A16_OK:
        raise W4A16Error(status, where, last_error())
