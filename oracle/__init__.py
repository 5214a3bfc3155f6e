"""fp64 CPU oracle (test infrastructure; see swiglu_oracle's header)."""
from .swiglu_oracle import *  # noqa: F401,F403
from .swiglu_oracle import (  # noqa: F401
    sigmoid, silu, silu_grad, gelu_tanh, gelu_tanh_grad, ACTIVATIONS, ACTIVATION_GRADS, gate_up, glu_fwd,
    swiglu_fwd, swiglu_fwd_rows, dswiglu, dglu, dswiglu_mult,
    swiglu_bwd, swiglu_bwd_dx_rows, swiglu_bwd_dw_rows, e4m3_decode, e4m3_encode,
    ue8m0_exponent, ue8m0_byte, clamp_nan_preserving, act_fwd, act_quant, quantize_1x32, act_bwd, act_bwd_fp8, normwise_rel_err,
    cosine, e4m3_ordinal, E4M3_MAX,
)
