"""ctypes declarations of libattn_jvp.so (the C ABI in include/attn_jvp.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_jvp.so")

ATTN_JVP_OK = 0
ATTN_JVP_ERR_NULL = -1
ATTN_JVP_ERR_SHAPE = -2
ATTN_JVP_ERR_DTYPE = -3
ATTN_JVP_ERR_ALIGN = -4
ATTN_JVP_ERR_MASK = -5
ATTN_JVP_ERR_UNSUPPORTED = -6
ATTN_JVP_ERR_HIP = -7
ATTN_JVP_ERR_OOM = -8
ATTN_JVP_ERR_NOT_READY = -9
ATTN_JVP_ERR_SCRATCH = -10
NOALLOC_SCRATCH_BYTES = 64 << 20

ATTN_JVP_BF16 = 0
ATTN_JVP_F32 = 1

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)
_pu32 = ctypes.POINTER(ctypes.c_uint32)


class AttnJvpArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", _i32), ("B", _i32), ("H", _i32), ("n_q", _i32), ("n_k", _i32), ("D", _i32),
        ("q", _p), ("k", _p), ("v", _p), ("dq", _p), ("dk", _p), ("dv", _p),
        ("o", _p), ("d_o", _p), ("lse", _p),
        ("q_stride_b", _i64), ("q_stride_n", _i64), ("q_stride_h", _i64),
        ("k_stride_b", _i64), ("k_stride_n", _i64), ("k_stride_h", _i64),
        ("scale", ctypes.c_float),
        ("d_lse", _p),
    ]


class AttnJvpBwdArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", _i32), ("B", _i32), ("H", _i32), ("n_q", _i32), ("n_k", _i32), ("D", _i32),
        ("q", _p), ("k", _p), ("v", _p), ("o", _p), ("g_o", _p), ("lse", _p),
        ("g_q", _p), ("g_k", _p), ("g_v", _p), ("delta", _p),
        ("q_stride_b", _i64), ("q_stride_n", _i64), ("q_stride_h", _i64),
        ("k_stride_b", _i64), ("k_stride_n", _i64), ("k_stride_h", _i64),
        ("scale", ctypes.c_float),
    ]


_PPMASK = ctypes.POINTER(ctypes.c_void_p)

SIGNATURES = {
    "attn_jvp_mask_tf": (_i32, [_i32, _i32, _i32, _PPMASK]),
    "attn_jvp_mask_rects": (_i32, [_i32, _i32, _i32, _pi32, _pi32, _pi32, _pi32, _PPMASK]),
    "attn_jvp_mask_dense": (_i32, [_i32, _i32, _PPMASK]),
    "attn_jvp_mask_block_causal": (_i32, [_i32, _i32, _PPMASK]),
    "attn_jvp_mask_info": (_i32, [_p, _pi32, _pi32, _pi32, _pi32, _pi64]),
    "attn_jvp_mask_export": (_i32, [_p, _pi32, _pi32, _pi32, _pi32]),
    "attn_jvp_mask_schedule": (_i32, [_p, _i32, _i32, _pi32, _pi64, _pi64, _pi32, _pi32,
                                      _pi32, _pi32, _pu32]),
    "attn_jvp_mask_split_schedule": (_i32, [_p, _i32, _i32, _i32, _pi32, _pi32, _pi32, _pi32,
                                            _pi32, _pi32]),
    "attn_jvp_mask_transpose": (_i32, [_p, _PPMASK]),
    "attn_jvp_mask_free": (None, [_p]),
    "attn_jvp_fwd": (_i32, [ctypes.POINTER(AttnJvpArgs), _p, _p]),
    "attn_jvp_fwd_split_workspace": (_i32, [ctypes.POINTER(AttnJvpArgs), _p, _i32,
                                            ctypes.POINTER(ctypes.c_uint64)]),
    "attn_jvp_fwd_split": (_i32, [ctypes.POINTER(AttnJvpArgs), _p, _i32, _p, ctypes.c_uint64, _p]),
    "attn_jvp_fwd_split_noalloc": (_i32, [ctypes.POINTER(AttnJvpArgs), _p, _i32, _p]),
    "attn_jvp_split_choose": (_i32, [ctypes.POINTER(AttnJvpArgs), _p, _i32, _pi32]),
    "attn_jvp_bwd": (_i32, [ctypes.POINTER(AttnJvpBwdArgs), _p, _p]),
    "attn_jvp_tile_shape": (_i32, [_i32, _i32, _i32, _pi32, _pi32]),
    "attn_jvp_status_str": (ctypes.c_char_p, [_i32]),
    "attn_jvp_version": (_i32, []),
}

_LIB = None


def lib():
    """The loaded library (raises ImportError when it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python attention_jvp_causal_attn_amd/csrc/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB
