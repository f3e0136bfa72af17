"""ctypes loader for libbsattn.so (the C-ABI in include/bsattn.h).

There is no fallback: if the library is missing the import of the compute
entry points fails loudly with instructions to build it.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsattn.so")

BS_OK = 0
BS_ERR_INVALID_ARG = -1
BS_ERR_UNSUPPORTED = -2
BS_ERR_LAYOUT = -3
BS_ERR_SHAPE = -4
BS_ERR_HIP = -5
BS_ERR_OOM = -6
BS_ERR_NO_DEVICE = -7
BS_F32 = 0
BS_BF16 = 1
BS_F16 = 2
BS_F8E4M3 = 3
BS_CAUSAL = 1
BS_TRANS_A = 1
BS_TRANS_B = 2

# every symbol the header declares, with (restype, argtypes)
_vp, _i, _f, _i64p = C.c_void_p, C.c_int, C.c_float, C.POINTER(C.c_int64)
_i32p = C.POINTER(C.c_int32)
_ip = C.POINTER(C.c_int)


class AcsrTerm(C.Structure):
    _fields_ = [("row_begin", C.c_int32), ("row_end", C.c_int32), ("slope", C.c_int32),
                ("offset", C.c_int32), ("stride", C.c_int32), ("count", C.c_int32)]


SIGNATURES = {
    "bs_layout_build": (_i, [_vp, _i, _i, _i, _i, _vp, C.POINTER(_vp)]),
    "bs_layout_build_acsr": (_i, [C.POINTER(AcsrTerm), _i, _i, _i, _i, _i, _vp, C.POINTER(_vp)]),
    "bs_layout_nnz": (_i, [_vp, _i64p]),
    "bs_layout_kv_share": (_i, [_vp, _ip, _ip]),
    "bs_layout_set_kv_share": (_i, [_vp, _i]),
    "bs_layout_info": (_i, [_vp, _ip, _ip, _ip, _ip, _i64p]),
    "bs_layout_export": (_i, [_vp, _i32p, _i32p, _i32p, _i32p, _i32p]),
    "bs_layout_free": (None, [_vp]),
    "bs_sdd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "bs_softmax": (_i, [_vp, _vp, _vp, _i, _f, _i, _vp]),
    "bs_dsd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "bs_dds": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "bs_attention": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _i, _vp]),
    "bs_softmax_backward": (_i, [_vp, _vp, _vp, _vp, _i, _f, _vp]),
    "bs_dsd_t": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "bs_attention_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _i, _vp]),
    "bs_softmax_masked": (_i, [_vp, _vp, _vp, _i, _f, _i, _vp, _vp, _vp]),
    "bs_attention_masked": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _vp, _vp, _i, _vp]),
    "bs_attention_backward_masked": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _vp,
                                          _vp, _i, _vp]),
    "bs_attention_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _vp, _vp, _i, _vp]),
    "bs_attention_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _vp, _vp, _i,
                              _vp]),
    "bs_attention_bwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _vp, _vp,
                                      _i, _vp]),
    "bs_sdd_ex": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "bs_dsd_ex": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "bs_dds_ex": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "bs_last_error": (C.c_char_p, []),
    "bs_version": (_i, []),
}

_lib = None


class BsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"bsattn error {code}: {msg}")
        self.code = code


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_sparse_matmul_amd.build` "
                "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(rc: int) -> None:
    if rc != BS_OK:
        raise BsError(rc, lib().bs_last_error().decode(errors="replace"))
