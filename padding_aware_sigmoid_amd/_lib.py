"""ctypes binding to libsigattn.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
declared in include/sigattn.h. This module loads the library and converts
tensors into pointers and sizes. It has no fallback: if the library is missing
or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import pathlib

_LIB_PATH = pathlib.Path(__file__).resolve().parent / "libsigattn.so"
_lib = None

BF16, FP32 = 0, 1
KERNEL_FWD, KERNEL_DQ, KERNEL_DKDV = 0, 1, 2
LAYOUT_PADDED, LAYOUT_PACKED = 0, 1
BIAS_CONSTANT, BIAS_NEG_LOG_NK = 0, 1
NOALLOC_ROWS = 1 << 21  # SIGATTN_NOALLOC_ROWS

EXPORTED_SYMBOLS = (
    "sigattn_fwd",
    "sigattn_bwd",
    "sigattn_bwd_dkdv",
    "sigattn_bwd_dq",
    "sigattn_bwd_dk",
    "sigattn_bwd_dv",
    "sigattn_fwd_ex",
    "sigattn_bwd_ex",
    "sigattn_softmax_fwd",
    "sigattn_softmax_bwd",
    "sigattn_softmax_bwd_workspace_size",
    "sigattn_softmax_bwd_noalloc",
    "sigattn_quantize_fp8",
    "sigattn_fwd_fp8",
    "sigattn_tile_config",
    "sigattn_strerror",
    "sigattn_last_error",
    "sigattn_version",
)


class SigattnError(RuntimeError):
    pass


def lib_path() -> pathlib.Path:
    return _LIB_PATH


def load():
    """Load libsigattn.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise SigattnError(f"{_LIB_PATH} is missing: build it first (python -m padding_aware_sigmoid_amd.build)")
    lib = ctypes.CDLL(str(_LIB_PATH))
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.sigattn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp]
    lib.sigattn_fwd.restype = i32
    lib.sigattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp, vp]
    lib.sigattn_bwd.restype = i32
    lib.sigattn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp]
    lib.sigattn_bwd_dkdv.restype = i32
    lib.sigattn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp]
    lib.sigattn_bwd_dq.restype = i32
    lib.sigattn_bwd_dk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp]
    lib.sigattn_bwd_dk.restype = i32
    lib.sigattn_bwd_dv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp]
    lib.sigattn_bwd_dv.restype = i32
    lib.sigattn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, i32, vp, vp]
    lib.sigattn_fwd_ex.restype = i32
    lib.sigattn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, i32, vp,
                                   vp, vp]
    lib.sigattn_bwd_ex.restype = i32
    lib.sigattn_softmax_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.sigattn_softmax_fwd.restype = i32
    lib.sigattn_softmax_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                        i32, vp, sz, vp]
    lib.sigattn_softmax_bwd.restype = i32
    lib.sigattn_softmax_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                f32, i32, vp]
    lib.sigattn_softmax_bwd_noalloc.restype = i32
    lib.sigattn_softmax_bwd_workspace_size.argtypes = [ctypes.c_longlong, i32]
    lib.sigattn_softmax_bwd_workspace_size.restype = sz
    lib.sigattn_quantize_fp8.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.sigattn_quantize_fp8.restype = i32
    lib.sigattn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    lib.sigattn_fwd_fp8.restype = i32
    lib.sigattn_tile_config.argtypes = [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.sigattn_tile_config.restype = i32
    lib.sigattn_strerror.argtypes = [i32]
    lib.sigattn_strerror.restype = ctypes.c_char_p
    lib.sigattn_last_error.argtypes = []
    lib.sigattn_last_error.restype = ctypes.c_char_p
    lib.sigattn_version.argtypes = []
    lib.sigattn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        lib = load()
        raise SigattnError(
            f"sigattn status {status} ({lib.sigattn_strerror(status).decode()}): {lib.sigattn_last_error().decode()}")


def tile_config(kernel: int, D: int, dtype: int):
    lib = load()
    bq, bk = ctypes.c_int(), ctypes.c_int()
    check(lib.sigattn_tile_config(kernel, D, dtype, ctypes.byref(bq), ctypes.byref(bk)))
    return bq.value, bk.value


def version() -> str:
    return load().sigattn_version().decode()
