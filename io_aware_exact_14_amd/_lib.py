"""ctypes view of libfa.so (declarations mirror include/fa.h)."""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
ABI_VERSION = 2

STATUS_NAMES = {
    0: "FA_OK",
    1: "FA_ERR_NULL",
    2: "FA_ERR_SHAPE",
    3: "FA_ERR_DTYPE",
    4: "FA_ERR_HEADDIM",
    5: "FA_ERR_DROPOUT",
    6: "FA_ERR_MASK",
    7: "FA_ERR_ALIGN",
    8: "FA_ERR_WORKSPACE",
    9: "FA_ERR_HIP",
    10: "FA_ERR_SCALE",
    11: "FA_ERR_RANGE",
    12: "FA_ERR_SCRATCH",
}
BWD_NOALLOC_MAX_ROWS = 1 << 22
STATUS = {v: k for k, v in STATUS_NAMES.items()}

# Every symbol the header declares.
EXPORTS = (
    "fa_abi_version",
    "fa_status_string",
    "fa_check_params",
    "fa_fwd",
    "fa_bwd_workspace_bytes",
    "fa_bwd",
    "fa_bwd_noalloc",
    "fa_bwd_dq",
    "fa_bwd_dkdv",
    "fa_dropout_mask",
)


class FaParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("dropout_p", ctypes.c_double),
        ("seed", ctypes.c_uint64),
        ("block_mask", ctypes.c_void_p),
        ("mask_block", ctypes.c_int32),
    ]


def _declare(lib):
    P = ctypes.POINTER(FaParams)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fa_abi_version.restype = i32
    lib.fa_abi_version.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i32]
    lib.fa_check_params.restype = i32
    lib.fa_check_params.argtypes = [P]
    lib.fa_fwd.restype = i32
    lib.fa_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_bytes.argtypes = [P]
    lib.fa_bwd.restype = i32
    lib.fa_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fa_bwd_dq.restype = i32
    lib.fa_bwd_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_dkdv.restype = i32
    lib.fa_bwd_dkdv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fa_dropout_mask.restype = i32
    lib.fa_dropout_mask.argtypes = [P, i64, i64, i64, i64, i64, i64, vp, vp]
    return lib


_LIB = None


def load():
    """Load libfa.so once. Raises OSError when the library has not been built:
    there is no fallback implementation."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it with `python io_aware_exact_14_amd/build.py`")
        lib = _declare(ctypes.CDLL(LIB_PATH))
        if lib.fa_abi_version() != ABI_VERSION:
            raise OSError(f"libfa ABI version {lib.fa_abi_version()} != {ABI_VERSION}")
        _LIB = lib
    return _LIB
