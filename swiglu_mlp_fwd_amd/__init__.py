"""libswiglu: the fused SwiGLU gate/up stage on AMD Instinct MI355X (gfx950).

    h = SiLU(x Wg^T) * (x Wu^T)

Python surface (thin marshalling over the C ABI in include/swiglu.h):
    fwd, fwd_fp8, bwd, bwd_noalloc, gemv_fwd, act_fwd, act_quant, act_bwd, swiglu (autograd), probe_read2,
    probe_mfma
"""
from ._lib import LIB_PATH, SwigluError, lib  # noqa: F401
from .ops import (  # noqa: F401
    SwiGLUFunction, act_bwd, act_bwd_fp8, act_fwd, act_quant, probe_act_quant_stream, bwd, bwd_noalloc, bwd_workspace_bytes, fwd, fwd_fp8, gemv_fwd, probe_gemv_read,
    probe_mfma, probe_read2, swiglu,
)

__all__ = ["fwd", "fwd_fp8", "bwd", "bwd_noalloc", "gemv_fwd", "act_fwd", "act_quant", "act_bwd", "act_bwd_fp8", "swiglu", "SwiGLUFunction", "probe_read2", "probe_gemv_read", "probe_act_quant_stream", "probe_mfma",
           "bwd_workspace_bytes", "SwigluError", "lib", "LIB_PATH"]
