"""ctypes loader for libsherry.so (the C ABI declared in include/sherry.h).

There is no fallback: if the library is missing this raises, so nothing can
silently run a different implementation.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsherry.so")

# status codes (sherry_status)
OK = 0
ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_GRANULARITY, ERR_DTYPE, ERR_UNSUPPORTED = 1, 2, 3, 4, 5, 6
ERR_ALIGN, ERR_WORKSPACE, ERR_BATCH, ERR_HIP = 7, 8, 9, 10

# enums
PER_TENSOR, PER_CHANNEL, PER_GROUP = 0, 1, 2
GRANULARITY = {"per_tensor": PER_TENSOR, "per_channel": PER_CHANNEL, "per_group": PER_GROUP}
CMP_2BIT, CMP_TL2 = 0, 1
F32, BF16, I8 = 0, 1, 2
OP_QUANTIZE_PACK, OP_UNPACK, OP_GEMV, OP_GEMM, OP_FAKE_QUANT, OP_ARENAS_GEMM = 0, 1, 2, 3, 4, 5
QUANTIZE_SCRATCH_BYTES = 8 << 20   # SHERRY_QUANTIZE_SCRATCH_BYTES

# every symbol include/sherry.h declares
SYMBOLS = (
    "sherry_abi_version", "sherry_status_string", "sherry_packed_bytes", "sherry_num_scales",
    "sherry_workspace_bytes", "sherry_quantize_pack", "sherry_unpack", "sherry_gemv", "sherry_gemm",
    "sherry_fake_quant", "sherry_arenas_gemm", "sherry_compare_bytes", "sherry_compare_repack",
    "sherry_compare_gemv", "sherry_arenas_lambda", "sherry_quantize_pack_noalloc",
)

_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "sherry_abi_version": ([], _i32),
    "sherry_status_string": ([_i32], ctypes.c_char_p),
    "sherry_packed_bytes": ([_i64, _i64], _sz),
    "sherry_num_scales": ([_i64, _i64, _i32, _i32], _i64),
    "sherry_workspace_bytes": ([_i32, _i64, _i64, _i32, _i32, _i64, _i32], _sz),
    "sherry_quantize_pack": ([_i64, _i64, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "sherry_quantize_pack_noalloc": ([_i64, _i64, _i32, _i32, _vp, _i32, _vp, _vp, _vp], _i32),
    "sherry_unpack": ([_i64, _i64, _i32, _i32, _vp, _vp, _vp, _i32, _vp], _i32),
    "sherry_gemv": ([_i64, _i64, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i64, _i64, _i64,
                     _vp, _sz, _vp], _i32),
    "sherry_gemm": ([_i64, _i64, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp], _i32),
    "sherry_fake_quant": ([_i64, _i64, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _sz, _vp], _i32),
    "sherry_arenas_gemm": ([_i64, _i64, _i32, _i32, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _vp, _vp, _sz, _vp],
                           _i32),
    "sherry_arenas_lambda": ([_i64, _i64, ctypes.c_double], ctypes.c_double),
    "sherry_compare_bytes": ([_i32, _i64, _i64], _sz),
    "sherry_compare_repack": ([_i32, _i64, _i64, _vp, _vp, _vp], _i32),
    "sherry_compare_gemv": ([_i32, _i64, _i64, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp], _i32),
}

_lib = None


class SherryError(RuntimeError):
    """A non-argument failure reported by libsherry (the HIP runtime)."""


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m ternary_weight_quantization_sparse_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().sherry_status_string(int(code)).decode()


def check(code: int) -> None:
    """Raise for a non-zero status: ValueError for argument errors (the
    conditions the pages' quantizer rejects and this build's limits),
    SherryError for runtime failures."""
    if code == OK:
        return
    msg = status_string(code)
    if code == ERR_HIP:
        raise SherryError(msg)
    if code == ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise ValueError(msg)
