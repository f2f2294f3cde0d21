"""ctypes loader and prototypes for libflux.so (declared in include/flux.h and
include/flux_probe.h).

Loading fails loudly: there is no fallback implementation of any entry point.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libflux.so")

FLUX_OK = 0
FLUX_ERR_INVALID_ARG = -1
FLUX_ERR_UNSUPPORTED = -2
FLUX_ERR_WORKSPACE = -3
FLUX_ERR_HIP = -4
FLUX_F32 = 0
FLUX_BF16 = 1
FLUX_DECODE_SCRATCH_BYTES = 9 << 20
FLUX_PREFILL_WORKSPACE_BYTES = 1024


class SAParamsC(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("sink_blocks", ctypes.c_int32),
                ("local_blocks", ctypes.c_int32)]


class DynParamsC(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("sink_blocks", ctypes.c_int32),
                ("tau", ctypes.c_float), ("max_blocks", ctypes.c_int32)]


# (name, restype, argtypes) for every symbol of include/flux.h
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t
SIGNATURES = [
    ("flux_status_str", ctypes.c_char_p, [_I]),
    ("flux_route_workspace_size", _S, [_I, _I, _I]),
    ("flux_route", _I, [_P, _I, _P, _I, _I, _P, _P, _I, _P, _P, _I, _P, _P, _P, _S, _P]),
    ("flux_mask_blocks", ctypes.c_int64, [_I, SAParamsC]),
    ("flux_mask_nnz", ctypes.c_int64, [_I, SAParamsC]),
    ("flux_build_block_mask", _I, [_I, SAParamsC, _P, _P, _P, _P]),
    ("flux_dynamic_mask_workspace_size", _S, [_I, _I, _I, _I, _I]),
    ("flux_build_block_mask_dynamic", _I, [_P, _P, _I, _I, _I, _I, _F, DynParamsC, _P, _P,
                                           ctypes.c_int64, _P, _S, _P]),
    ("flux_attn_prefill_workspace_size", _S, []),
    ("flux_attn_prefill", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I, _P, _P,
                               _I, SAParamsC, _P, _S, _P]),
    ("flux_attn_decode_workspace_size", _S, [_I, _I, _I, _I, _I]),
    ("flux_attn_decode", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I, _P, _P, _I,
                              SAParamsC, _P, _S, _P]),
    ("flux_attn_prefill_heads", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I, _P,
                                     _P, _I, SAParamsC, _P]),
    ("flux_attn_prefill_soft", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I, _P,
                                    _P, _I, SAParamsC, _P, _S, _P]),
    ("flux_attn_decode_append", _I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I,
                                     _P, _P, _I, SAParamsC, _P, _S, _P]),
    ("flux_attn_decode_noalloc", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I, _P, _P,
                                      _I, SAParamsC, _P]),
    ("flux_attn_decode_heads", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I, _P, _P,
                                    _I, SAParamsC, _P, _S, _P]),
    ("flux_kv_rows", ctypes.c_int64, [_I, SAParamsC, _I]),
    ("flux_kv_store_prefill", _I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _I, SAParamsC, _P]),
    ("flux_kv_append", _I, [_P, _P, _P, _I, _I, _I, _P, _P, _I, _I, SAParamsC, _P]),
    ("flux_attn_decode_sa_compact", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _I,
                                         SAParamsC, _P, _S, _P]),
]
# measurement probes (include/flux_probe.h)
PROBE_SIGNATURES = [
    ("flux_probe_mfma", _I, [_P, _I, _I, _P]),
    ("flux_probe_mfma_flops", ctypes.c_double, [_I, _I]),
    ("flux_probe_read", _I, [_P, _S, _P, _I, _P]),
]

_lib = None


def load(path=LIB_PATH):
    """Load libflux.so and attach prototypes.  Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libflux.so not found at {path}; build it first with "
            "`python block_sparse_attention_flux_amd/build.py` (needs hipcc)")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES + PROBE_SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib
