"""ctypes loader for libswiglu.so (the C ABI declared in include/swiglu.h).

The library is loaded from this package directory only; there is no fallback
of any kind: if it is missing, fails to load, or was built from sources other
than the ones in the tree (its embedded source hash differs), every call
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswiglu.so")

SWIGLU_F32 = 0
SWIGLU_BF16 = 1
SWIGLU_ACT_SILU = 0
SWIGLU_ACT_GELU_TANH = 1
SWIGLU_ERR_SCRATCH = 9
NOALLOC_SCRATCH_BYTES = 128 << 20    # SWIGLU_NOALLOC_SCRATCH_BYTES

_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p

# name -> (restype, argtypes), in the order of include/swiglu.h
SIGNATURES = {
    "swiglu_fwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_fwd_act": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr,
                                      _c_ptr, _c_ptr]),
    "swiglu_fwd_fp8": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                      _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_fwd_mult": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr,
                                       ctypes.c_float, ctypes.c_float, _c_ptr, _c_ptr]),
    "swiglu_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, _c_i64, _c_i64, _c_i64]),
    "swiglu_bwd": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                  _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr]),
    "swiglu_bwd_mult": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                       ctypes.c_float, ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_size_t,
                                       _c_ptr]),
    "swiglu_bwd_act_mult": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr,
                                           _c_ptr, _c_ptr, ctypes.c_float, ctypes.c_float, _c_ptr, _c_ptr, _c_ptr,
                                           _c_ptr, ctypes.c_size_t, _c_ptr]),
    "swiglu_bwd_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr,
                                          _c_ptr, _c_ptr, ctypes.c_float, ctypes.c_float, _c_ptr, _c_ptr, _c_ptr,
                                          _c_ptr]),
    "swiglu_gemv_fwd": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_gemv_fwd_act": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                           _c_ptr]),
    "swiglu_gemv_fwd_mult": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr,
                                            ctypes.c_float, ctypes.c_float, _c_ptr, _c_ptr]),
    "swiglu_act_fwd": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_ptr, ctypes.c_float,
                                      _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_act_quant": (ctypes.c_int, [_c_i64, _c_i64, _c_ptr, _c_ptr, ctypes.c_float, _c_ptr, _c_ptr,
                                        _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_act_quant_act": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_ptr, ctypes.c_float, _c_ptr,
                                            _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_act_bwd": (ctypes.c_int, [_c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_float,
                                      _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_act_bwd_dt": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                         ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_act_bwd_fp8": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                          ctypes.c_float, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_probe_mfma": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_ptr, _c_ptr]),
    "swiglu_probe_gemv_read": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_probe_act_quant_stream": (ctypes.c_int, [_c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "swiglu_probe_fp8_transitions": (ctypes.c_int, [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, _c_ptr,
                                                    ctypes.c_uint32, _c_ptr, _c_ptr]),
    "swiglu_probe_read2": (ctypes.c_int, [_c_ptr, _c_ptr, ctypes.c_size_t, _c_ptr, _c_ptr]),
    "swiglu_probe_read2_cfg": (ctypes.c_int, [_c_ptr, _c_ptr, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _c_ptr, _c_ptr]),
    "swiglu_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "swiglu_last_hip_error": (ctypes.c_int, []),
    "swiglu_version": (ctypes.c_int, []),
    "swiglu_source_hash": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


class SwigluError(RuntimeError):
    """A libswiglu call returned a non-zero status."""

    def __init__(self, fn: str, status: int, text: str, hip_error: int = 0):
        msg = f"{fn}: {text} (status {status})"
        if hip_error:
            msg += f", hipError {hip_error}"
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built; run `python -m swiglu_mlp_fwd_amd.build` "
                    "(there is no non-HIP fallback)")
            L = ctypes.CDLL(LIB_PATH)
            from .build import source_hash
            current = source_hash()
            if not hasattr(L, "swiglu_source_hash"):
                raise RuntimeError(f"{LIB_PATH} is stale (it has no source hash); rebuild with "
                                   "`python -m swiglu_mlp_fwd_amd.build`")
            for name, (res, args) in SIGNATURES.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            built = L.swiglu_source_hash().decode()
            if built != current:
                raise RuntimeError(
                    f"{LIB_PATH} is stale: built from sources with hash {built}, the tree's sources hash to "
                    f"{current}; rebuild with `python -m swiglu_mlp_fwd_amd.build`")
            _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != 0:
        L = lib()
        raise SwigluError(fn, status, L.swiglu_status_str(status).decode(),
                          L.swiglu_last_hip_error() if status == 8 else 0)
