"""ctypes declarations of the C ABI in include/nsn.h (libnsn.so, built in-tree).

The library is required: there is no fallback implementation.  A missing or
stale build raises at load time with the command that fixes it.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnsn.so")

NSN_OK = 0
NSN_ERR_INVALID_ARG = 1
NSN_ERR_UNSUPPORTED = 2
NSN_ERR_WORKSPACE = 3
NSN_ERR_HIP = 4
NSN_ERR_INTERNAL = 5
NSN_F16 = 0
NSN_F32 = 1
NSN_SCALE_ADJUST = 1
NSN_DQ = 2
NSN_RHT = 4


class nsn_params(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("sub_dim", ctypes.c_int32),
        ("n_codes", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("rht_signs", ctypes.c_uint32 * 4),
    ]


class nsn_attn_shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("n_quant_tok", ctypes.c_int32),
        ("n_resid_tok", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int64),
        ("resid_capacity", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
    ]


class nsn_rope(ctypes.Structure):
    _fields_ = [
        ("q_pos", ctypes.c_int64),
        ("base", ctypes.c_float),
    ]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_ST = ctypes.c_int

# name -> (restype, argtypes)
SIGNATURES = {
    "nsn_table_size": (_SZ, [ctypes.POINTER(nsn_params)]),
    "nsn_build_codebook_workspace_size": (_SZ, [_I32, _I32, _I64]),
    "nsn_build_codebook": (_ST, [_I32, _I32, _I64, _I32, _P, _P, _P, _SZ, _P]),
    "nsn_tune_codebook_workspace_size": (_SZ, [_I32, _I32, _I64]),
    "nsn_tune_codebook": (_ST, [_I32, _I32, _I64, _I32, ctypes.c_double, _P, _P, _P, _SZ, _P]),
    "nsn_prepare_codebook": (_ST, [ctypes.POINTER(nsn_params), _P, _P, _SZ, _P]),
    "nsn_nearest_codeword": (_ST, [ctypes.POINTER(nsn_params), _P, _P, _I64, _P, _P]),
    "nsn_quantize": (_ST, [ctypes.POINTER(nsn_params), _ST, _P, _I64, _I64, _I64, _P,
                           _P, _I64, _P, _I64, _P, _I64, _P]),
    "nsn_dequantize": (_ST, [ctypes.POINTER(nsn_params), _P, _I64, _P, _I64, _P, _I64, _P,
                             _I64, _I64, _ST, _P, _I64, _P]),
    "nsn_residual_append": (_ST, [_P, _I64, _P, _I64, _I64, _I64, _P]),
    "nsn_decode_attention_workspace_size": (_SZ, [ctypes.POINTER(nsn_params),
                                                  ctypes.POINTER(nsn_attn_shape)]),
    "nsn_decode_attention": (_ST, [ctypes.POINTER(nsn_params), ctypes.POINTER(nsn_attn_shape),
                                   _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "nsn_decode_attention_noalloc": (_ST, [ctypes.POINTER(nsn_params), ctypes.POINTER(nsn_attn_shape),
                                           _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "nsn_decode_attention_rope": (_ST, [ctypes.POINTER(nsn_params), ctypes.POINTER(nsn_attn_shape),
                                        ctypes.POINTER(nsn_rope), _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _SZ, _P, _P]),
    "nsn_status_string": (ctypes.c_char_p, [_ST]),
    "nsn_last_error": (ctypes.c_char_p, []),
    "nsn_version": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libnsn.so (once) and declare every exported function."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m kv_cache_calibration_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class NsnError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{detail} [status {status}]")


def check(status):
    if status != NSN_OK:
        lib = load()
        detail = lib.nsn_last_error().decode() or lib.nsn_status_string(status).decode()
        raise NsnError(status, detail)
