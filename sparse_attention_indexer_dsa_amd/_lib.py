"""ctypes view of libdsaidx.so (the C ABI of include/dsa_indexer.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsaidx.so")

DSAIDX_OK = 0
DSAIDX_ERR_INVALID_ARG = -1
DSAIDX_ERR_UNSUPPORTED = -2
DSAIDX_ERR_WORKSPACE = -3
DSAIDX_ERR_HIP = -4
DSAIDX_BF16 = 1
DSAIDX_FP8_E4M3 = 2
DSAIDX_FORCE_BANK = 1
DSAIDX_POOL_MEAN = 2
DSAIDX_NO_BANK = 8

# exported symbol -> (restype, argtypes)
_P, _I, _I64, _U, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint, ctypes.c_size_t
_D = ctypes.c_double


class Layer(ctypes.Structure):
    """dsaidx_layer: one layer of indexer_layers (field order of the C struct)."""
    _fields_ = [("q", _P), ("q_scale", _P), ("k", _P), ("k_scale", _P), ("w", _P), ("qbar", _P),
                ("qbar_scale", _P), ("wbar", _P), ("Hs", _I), ("G", _I), ("P", _I), ("flags", _U),
                ("out_idx", _P), ("out_score", _P), ("out_bank", _P)]


SIGNATURES = {
    "indexer_prefill": (_I, [_P, _P, _P, _P, _P, _I, _I64, _I64, _I, _I, _I64, _I, _P, _P, _P, _SZ, _P]),
    "indexer_prefill_workspace_size": (_SZ, [_I64, _I64, _I, _I, _I, _I]),
    "indexer_decode": (_I, [_P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "indexer_decode_workspace_size": (_SZ, [_I, _I64, _I, _I, _I]),
    "indexer_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _P, _P, _P]),
    "indexer_decode_noalloc_max_bytes": (_SZ, []),
    "indexer_group_bank": (_I, [_P, _P, _P, _P, _P, _I, _I64, _I64, _I, _I, _I64, _P, _P, _P, _I, _I, _I,
                                _I, _U, _P, _P, _P, _P, _SZ, _P]),
    "indexer_group_bank_workspace_size": (_SZ, [_I64, _I64, _I, _I, _I, _I, _I, _I, _I, _U]),
    "indexer_group_bank_pairs": (_I64, [_I64, _I64, _I, _I, _U]),
    "indexer_layers": (_I, [_P, _I, _I, _I64, _I64, _I, _I, _I64, _I, _P, _SZ, _P]),
    "indexer_layers_workspace_size": (_SZ, [_P, _I, _I64, _I64, _I, _I, _I, _I]),
    "indexer_mtp": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _I, _I, _I, _I, _U, _P, _P, _P, _P,
                         _SZ, _P]),
    "indexer_mtp_workspace_size": (_SZ, [_I, _I64, _I, _I, _I, _I, _I, _I, _I, _U]),
    "indexer_mtp_pairs": (_I64, [_P, _I, _I64, _I, _I, _I, _U]),
    "indexer_group_query": (_I, [_P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I64, _I, ctypes.c_float, _P, _P,
                                 _P, _SZ, _P]),
    "indexer_group_query_workspace_size": (_SZ, [_I64, _I, _I, _I, _I, _I]),
    "indexer_union_sizes": (_I, [_P, _I64, _I, _I, _P, _P]),
    "indexer_topk_overlap": (_I, [_P, _P, _I64, _I, _P, _P]),
    "indexer_union_stat": (_D, [_P, _I64, _I]),
    "indexer_speedup_joint": (_D, [_D, _I, _I, _I, _I, _D]),
    "indexer_select_setting": (_I, [_P, _D, _I, _I, _D, _P, _P]),
    "indexer_layerwise_speedup": (_D, [_P, _P, _I, _D, _I, _I, _D]),
    "indexer_read_probe": (_I, [_P, _I64, _P, _I, _P]),
    "indexer_mfma_probe": (_I, [_I, _I, _I, _I, ctypes.c_uint32, _P, _P, _P]),
    "indexer_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first (python -m sparse_attention_indexer_dsa_amd.build "
                "or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().indexer_last_error().decode()
