"""ctypes view of libattn.so: the C ABI declared in include/attn.h, one Python callable
per exported symbol, with the same names and argument order.  Loading fails loudly
when the library has not been built."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3 = 0, 1, 2
STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_ALIGN",
    4: "ATTN_ERR_UNSUPPORTED", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP", 7: "ATTN_ERR_ARG",
}
ATTN_MAX_SPLITS = 4096
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/attn.h
SIGNATURES = {
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "attn_fwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp]),
    "attn_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                             _i, _i, _vp]),
    "attn_splitkv_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "attn_splitkv_num_splits": (_i, [_i, _i, _i, _i, _i, _i]),
    "attn_fwd_splitkv": (_i, [_vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                              _f, _f, _f, _vp]),
    "attn_merge": (_i, [_vp, _sz, _i, _vp, _vp, _i, _i, _i, _i, _vp]),
    "attn_fwd_splitkv_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                                      _f, _f, _f, _vp]),
    "attn_block_m": (_i, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "attn_block_n": (_i, [_i, _i]),
    "attn_num_workgroups": (ctypes.c_int64, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "attn_kernel_name": (ctypes.c_char_p, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "attn_tune": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i,
                       ctypes.POINTER(_i), _vp]),
    "attn_tune_splitkv": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _f, _f,
                               _f, _i, ctypes.POINTER(_i), _vp]),
    "attn_plan_get": (_i, [_i, _i, _i, _i, _i, _i, _i]),
    "attn_plan_set": (_i, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "attn_plan_clear": (None, []),
    "attn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _i, _i,
                      _f, _i, _i, _vp]),
    "attn_bwd_kernel_name": (ctypes.c_char_p, [_i, _i, _i]),
    "attn_status_string": (ctypes.c_char_p, [_i]),
    "attn_last_hip_error": (_i, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libattn.so once; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m exact_attention_82_amd.build` "
                "(the HIP library is the only implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class AttnError(RuntimeError):
    """A library call returned a status other than ATTN_OK."""

    def __init__(self, fn: str, status: int):
        lib = load()
        text = lib.attn_status_string(status).decode()
        extra = ""
        if status == 6:
            extra = f" (hipError {lib.attn_last_hip_error()})"
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {text}{extra}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise AttnError(fn, status)
