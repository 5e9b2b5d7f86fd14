"""ctypes loader for libsals.so and the C prototypes of include/sals.h.

The library is loaded from this package's directory. There is no fallback: if it is missing or
fails to load, ``lib()`` raises, so nothing in the product path can silently run elsewhere.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsals.so")


class SalsShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("r", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class SalsSelect(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("w", ctypes.c_int32), ("G", ctypes.c_int32)]


class KvcShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


STATUS = {
    0: "SALS_OK", 1: "SALS_ERR_NULL", 2: "SALS_ERR_SHAPE", 3: "SALS_ERR_DTYPE",
    4: "SALS_ERR_RANGE", 5: "SALS_ERR_WORKSPACE", 6: "SALS_ERR_ALIGN", 7: "SALS_ERR_HIP",
}

_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_SP = ctypes.POINTER(_S)

PROTOTYPES = {
    "sals_abi_version": (_I, []),
    "sals_status_string": (ctypes.c_char_p, [_I]),
    "sals_last_hip_error": (_I, []),
    "sals_project_kv": (_I, [ctypes.POINTER(SalsShape), _P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "sals_decode_workspace_bytes": (_I, [ctypes.POINTER(SalsShape), ctypes.POINTER(SalsSelect), _I, _SP]),
    "sals_decode_step": (_I, [ctypes.POINTER(SalsShape), ctypes.POINTER(SalsSelect), ctypes.c_float,
                              _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _S, _P]),
    "sals_decode_step_threshold": (_I, [ctypes.POINTER(SalsShape), ctypes.POINTER(SalsSelect), ctypes.c_float,
                                        ctypes.c_float, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _S, _P]),
    "sals_decode_step_noalloc": (_I, [ctypes.POINTER(SalsShape), ctypes.POINTER(SalsSelect), ctypes.c_float,
                                      _P, _P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "sals_decode_step_traced": (_I, [ctypes.POINTER(SalsShape), ctypes.POINTER(SalsSelect), ctypes.c_float,
                                     _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _S, _P,
                                     ctypes.POINTER(ctypes.c_void_p), _I]),
    "kv_compact_workspace_bytes": (_I, [ctypes.POINTER(KvcShape), _I, _I, _I, _SP]),
    "kv_compact": (_I, [ctypes.POINTER(KvcShape), _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _S, _P]),
    "sals_dense_decode_workspace_bytes": (_I, [ctypes.POINTER(KvcShape), _I, _SP]),
    "sals_dense_decode": (_I, [ctypes.POINTER(KvcShape), _P, _P, _P, _I, _I, _P, _P, _S, _P]),
    "kv_importance_sparsity_workspace_bytes": (_I, [ctypes.POINTER(KvcShape), _I, _I, _SP]),
    "kv_importance_sparsity": (_I, [ctypes.POINTER(KvcShape), _P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P, _S,
                                    _P]),
    "kv_outlier_importance_workspace_bytes": (_I, [ctypes.POINTER(KvcShape), _I, _I, _SP]),
    "kv_outlier_importance": (_I, [ctypes.POINTER(KvcShape), _P, _P, _I, _I, _I, _P, _P, _S, _P]),
    "kv_quantize_mixed": (_I, [ctypes.POINTER(KvcShape), _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "sals_dense_decode_mixed_workspace_bytes": (_I, [ctypes.POINTER(KvcShape), _I, _I, _SP]),
    "sals_dense_decode_mixed": (_I, [ctypes.POINTER(KvcShape), _P, _P, _P, _I, _P, _P, _I, _P, _P, _S, _P]),
    "kv_importance_budget": (_I, [ctypes.POINTER(KvcShape), _P, _I, ctypes.c_float, _P, _P, _P, _P, _P]),
    "kv_compact_traced": (_I, [ctypes.POINTER(KvcShape), _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _S, _P,
                               ctypes.POINTER(ctypes.c_void_p), _I]),
    "sals_hbm_read": (_I, [_P, _S, _P, _I, _P]),
    "sals_mfma_peak": (_I, [_I, _I, _P, _P]),
    "kv_layer_budgets": (_I, [_P, _I, ctypes.c_int64, _I, _P]),
    "kv_compact_from_importance": (_I, [ctypes.POINTER(KvcShape), _P, _P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "sals_reconstruct_kv": (_I, [ctypes.POINTER(SalsShape), ctypes.c_float, _P, _P, _P, _P, _I, _I, _I,
                                 _P, _P, _I, _P, _P, _I, _P]),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if libsals.so is absent or does not load."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m kv_cache_compression_sals_amd.build` "
                    "(or __graft_entry__.build()); there is no fallback implementation")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in PROTOTYPES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib
