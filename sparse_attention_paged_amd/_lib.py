"""ctypes loader for libsap.so, the gfx950 library behind include/sap.h.

There is no fallback: if the library is missing every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsap.so")

SAP_BF16, SAP_F32, SAP_FP8_E4M3 = 0, 1, 2

# every entry point declared in include/sap.h: (restype, argtypes)
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "sap_version": (_I, []),
    "sap_status_string": (ctypes.c_char_p, [_I]),
    "sap_build_sparse_idx": (_I, [_P, _P, _I, _I, _P, _I64, _I, _P, _I64, _I, _P, _I64, _P, _I64, _P]),
    "sap_sparse_attn_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "sap_sparse_attn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "sap_sparse_attn_paged": (_I, [_P, _I, _I64, _I64, _P, _I64, _P, _I64, _I, _P, _I64, _I, _I,
                                   _P, _P, _P, _I, _I64, _I64, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "sap_sparse_attn_noalloc_max_bytes": (_SZ, []),
    "sap_sparse_attn_paged_noalloc": (_I, [_P, _I, _I64, _I64, _P, _I64, _P, _I64, _I, _P, _I64, _I, _I,
                                           _P, _P, _P, _I, _I64, _I64, _I, _I, _I, _F, _I, _P]),
    "sap_indexer_logits_packed": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I, _P, _P, _I64,
                                       _I, _I, _I, _I, _P]),
    "sap_indexer_logits_candidates": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I, _P, _I64, _P,
                                           _P, _I64, _I, _I, _I, _I, _P]),
    "sap_indexer_logits_prefill": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I, _P, _I, _I, _P,
                                        _P, _I64, _I, _I, _I, _P]),
    "sap_gated_pool": (_I, [_P, _I, _I64, _I64, _P, _I, _I64, _I64, _P, _I, _I64, _I, _I, _I, _P]),
    "sap_topk_workspace_bytes": (_SZ, [_I, _I, _I]),
    "sap_topk_select": (_I, [_P, _I64, _P, _I, _I, _I, _P, _I64, _P, _SZ, _P]),
    "sap_topk_sparse_idx": (_I, [_P, _I64, _P, _I, _I, _I, _P, _P, _I, _P, _I64, _P, _I64, _I, _P, _I64, _P,
                                 _SZ, _P]),
    "sap_debug_e4m3_table": (_I, [_P, _P, _P]),
    "sap_debug_e4m3_f16_table": (_I, [_P, _P]),
    "sap_debug_fp4_table": (_I, [_P, _P]),
}

_lib = None


class SapError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SapError(f"{LIB_PATH} is not built (python -m sparse_attention_paged_amd.build); "
                           "this package has no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return lib().sap_status_string(int(rc)).decode()


def check(rc: int, what: str) -> None:
    if rc != 0:
        raise SapError(f"{what}: {status_string(rc)} (status {rc})")
