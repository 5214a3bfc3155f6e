"""fp64 CPU oracle for the fused SwiGLU gate/up stage.

TEST INFRASTRUCTURE.  This module is the independent checker of the HIP path.
Only the tests, the smoke check in __graft_entry__ and the cpu_baseline leg of
bench.py may import or call it; the product package (swiglu_mlp_fwd_amd) never
does, and this module imports nothing from it.

It is written to be read against the pages, not to be fast.  Every function is
the plain definition of what the method computes, in float64, with numpy's
matmul as the only library primitive.  Inputs are float64 arrays holding the
exact values the device sees (bf16 or fp32 widened without rounding).

Sources (page title, then section):
  [Liger-1383]  "[RFC] Testing Methodology for FP32 Convergence Tests on Fused
                SwiGLU/dSwiGLU Kernels" (Liger-Kernel issue 1383): Background
                (the fused gate/up GEMM + SwiGLU, forward and backward), Root
                Cause (true IEEE fp32 is the reference, not TF32).
  [Liger-937]   "Another MLP implementation along with multiplier support"
                (Liger-Kernel issue 937): TL;DR (gate_proj, up_proj, SiLU-mul;
                approach 3, the dual GEMM with activation).
  [TRT-17693]   "VisualGen MLP: cublasLt GELU-tanh epilogue for the unquantized
                bf16 path" (TensorRT-LLM PR 17693): Change (nn.Linear layout,
                x @ weight.t(), rank>=3 flattened to [M, in]); the follow-up
                commit on numerics (activation applied to the fp32 accumulator).
  [PTO-20]      "quant: add SwiGLU forward/backward VMI kernels" (TileKernels-PTO
                PR 20): implementation notes (1x32 scale blocks, packed UE8M0
                scales, clamp with clamp counting, NOSAT FP8 cast keeping NaN),
                validation (amax=inf packed UE8M0, subnormals, non-finite inputs).

Readings taken where the pages are silent:
  * weights are [N, K] row-major and g = x @ Wg^T (nn.Linear layout);
  * silu(z) = z * sigmoid(z) evaluated by IEEE rules: silu(+inf)=+inf,
    silu(-inf)=NaN (-inf * 0), silu(NaN)=NaN;
  * the derivative of silu is the closed form s * (1 + z * (1 - s)), s = sigmoid(z);
  * the GeGLU variant replaces SiLU by the tanh GELU,
    z / 2 * (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)));
  * the clamp is symmetric [-L, L] on both gate and up, applied before the
    activation, NaN passing through; the clamp count is the number of gate and
    up values with |v| > L (NaN not counted);
  * the scale of a 1x32 block is the smallest power of two 2^E with
    amax <= 448 * 2^E (amax ignoring NaN; all-NaN or all-zero blocks have
    amax 0), E clamped to [-127, 127], stored as the byte E + 127; a block
    whose amax is +inf gets the byte 0xFF and E = 128;
  * codes are OCP E4M3FN (bias 7, max 448, no infinities), nearest value with
    ties to even, no saturation: NaN and +-inf become NaN, and a value that
    rounds past 448 becomes NaN.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# Activation.  [Liger-937] TL;DR: intermediate = SiLU(gate_proj(x)) * up_proj(x).
# ---------------------------------------------------------------------------

def sigmoid(z):
    """sigma(z) = 1 / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """SiLU(z) = z * sigma(z), float64 (IEEE: silu(-inf) = -inf * 0 = NaN)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return z * sigmoid(z)


def silu_grad(z):
    """d/dz SiLU(z) = s * (1 + z * (1 - s)) with s = sigma(z)  (closed form)."""
    z = np.asarray(z, dtype=np.float64)
    s = sigmoid(z)
    with np.errstate(over="ignore", invalid="ignore"):
        return s * (1.0 + z * (1.0 - s))


# GELU with the tanh approximation, the activation of the GeGLU variant:
# [Liger-937] feature pitch (the Liger MLP modules fuse swiglu and geglu) and
# [TRT-17693] (the cublasLt epilogue implements tanh-approximated GELU,
# gelu_tanh).  Reading: the standard tanh form
#   gelu_tanh(z) = z / 2 * (1 + tanh(sqrt(2 / pi) * (z + 0.044715 z^3))),
# and the gated form h = gelu_tanh(g) * u, in place of SiLU.
GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


def gelu_tanh(z):
    """z / 2 * (1 + tanh(y)), y = sqrt(2/pi) (z + 0.044715 z^3), evaluated as
    z * sigma(2 y): the identity (1 + tanh y) / 2 = 1 / (1 + e^-2y) is exact,
    and this form keeps full relative precision in the negative tail, where
    1 + tanh(y) cancels."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return z * sigmoid(2.0 * GELU_C * (z + GELU_A * z * z * z))


def gelu_tanh_grad(z):
    """d/dz gelu_tanh(z) = s + z s (1 - s) t'(z), with t = 2 y the argument of
    sigma above, s = sigma(t) and t'(z) = 2 sqrt(2/pi) (1 + 3 * 0.044715 z^2)
    (product and chain rule on z * sigma(t(z)), sigma' = sigma (1 - sigma))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        t = 2.0 * GELU_C * (z + GELU_A * z * z * z)
        s = sigmoid(t)
        dt = 2.0 * GELU_C * (1.0 + 3.0 * GELU_A * z * z)
        return s + z * s * (1.0 - s) * dt


ACTIVATIONS = {"silu": silu, "gelu_tanh": gelu_tanh}
ACTIVATION_GRADS = {"silu": silu_grad, "gelu_tanh": gelu_tanh_grad}


# ---------------------------------------------------------------------------
# Forward.  [Liger-1383] Background and [Liger-937] TL;DR approach 3:
# h = SiLU(x Wg^T) * (x Wu^T), weights in nn.Linear [N, K] layout
# ([TRT-17693] Change: x2d @ weight.t()).
# ---------------------------------------------------------------------------

def gate_up(x, wg, wu):
    """g = x @ Wg^T and u = x @ Wu^T in float64.  x [M,K], Wg/Wu [N,K]."""
    x = np.asarray(x, np.float64)
    wg = np.asarray(wg, np.float64)
    wu = np.asarray(wu, np.float64)
    return x @ wg.T, x @ wu.T


def glu_fwd(x, wg, wu, act="silu", gate_mult=1.0, up_mult=1.0):
    """h = act(gate_mult * x Wg^T) * (up_mult * x Wu^T) with act in ACTIVATIONS.

    The multipliers ([Liger-937] TL;DR: a gate multiplier passed to the dual
    GEMM with activation; the Falcon-H1 MLP's gate and up multipliers) scale
    each projection's output before the activation and the product.  Reading:
    the pages do not place them; this is the same as scaling Wg and Wu.
    """
    g, u = gate_up(x, wg, wu)
    return ACTIVATIONS[act](gate_mult * g) * (up_mult * u)


def swiglu_fwd(x, wg, wu):
    """h[M,N] = SiLU(x Wg^T) * (x Wu^T), float64.

    The fused epilogue applies the activation to the unrounded accumulators
    ([TRT-17693] follow-up commit on numerics); in the oracle every
    intermediate is exact float64, so only the device output is rounded.
    """
    g, u = gate_up(x, wg, wu)
    return silu(g) * u


def swiglu_fwd_rows(x, wg, wu, rows):
    """Selected rows of h (the forward is row-independent in M)."""
    x = np.asarray(x)[np.asarray(rows)]
    return swiglu_fwd(x, wg, wu)


# ---------------------------------------------------------------------------
# Backward.  [Liger-1383] Background ("full forward and backward dataflow",
# fused SwiGLU/dSwiGLU).  With L = sum(dh * h):
#   du = dh * SiLU(g)
#   dg = dh * u * SiLU'(g)
#   dX = dg Wg + du Wu,  dWg = dg^T x,  dWu = du^T x
# ---------------------------------------------------------------------------

def dswiglu(g, u, dh):
    """(dg, du) from the pre-activation g, the up value u and the upstream dh."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    dh = np.asarray(dh, np.float64)
    du = dh * silu(g)
    dg = dh * u * silu_grad(g)
    return dg, du


def dglu(g, u, dh, act="silu"):
    """(dg, du) of h = act(g) u: dg = dh u act'(g), du = dh act(g)."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    dh = np.asarray(dh, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return dh * u * ACTIVATION_GRADS[act](g), dh * ACTIVATIONS[act](g)


def dswiglu_mult(g, u, dh, gate_mult=1.0, up_mult=1.0, act="silu"):
    """(dg, du) of h = act(gate_mult g) (up_mult u): the chain rule through
    the scaled projections G = gate_mult g, U = up_mult u."""
    G, U = gate_mult * np.asarray(g, np.float64), up_mult * np.asarray(u, np.float64)
    dG, dU = dswiglu(G, U, dh) if act == "silu" else dglu(G, U, dh, act)
    return gate_mult * dG, up_mult * dU


def swiglu_bwd(x, wg, wu, dh, gate_mult=1.0, up_mult=1.0, act="silu"):
    """(dx [M,K], dwg [N,K], dwu [N,K]) in float64, for the forward
    glu_fwd(x, wg, wu, act, gate_mult, up_mult)."""
    x = np.asarray(x, np.float64)
    wg = np.asarray(wg, np.float64)
    wu = np.asarray(wu, np.float64)
    g, u = gate_up(x, wg, wu)
    dg, du = dswiglu_mult(g, u, dh, gate_mult, up_mult, act)
    dx = dg @ wg + du @ wu
    dwg = dg.T @ x
    dwu = du.T @ x
    return dx, dwg, dwu


def swiglu_bwd_dx_rows(x, wg, wu, dh, rows, gate_mult=1.0, up_mult=1.0, act="silu"):
    """Selected rows of dX (row m of dX needs only row m of x and dh)."""
    rows = np.asarray(rows)
    x = np.asarray(x, np.float64)[rows]
    wg = np.asarray(wg, np.float64)
    wu = np.asarray(wu, np.float64)
    g, u = gate_up(x, wg, wu)
    dg, du = dswiglu_mult(g, u, np.asarray(dh)[rows], gate_mult, up_mult, act)
    return dg @ wg + du @ wu


def swiglu_bwd_dw_rows(x, wg, wu, dh, cols, gate_mult=1.0, up_mult=1.0, act="silu"):
    """Selected rows n of dWg and dWu (they need column n of g, u and dh)."""
    cols = np.asarray(cols)
    x = np.asarray(x, np.float64)
    g, u = gate_up(x, np.asarray(wg)[cols], np.asarray(wu)[cols])
    dg, du = dswiglu_mult(g, u, np.asarray(dh, np.float64)[:, cols], gate_mult, up_mult, act)
    return dg.T @ x, du.T @ x


# ---------------------------------------------------------------------------
# FP8 E4M3FN codes.  [PTO-20] implementation notes: the FP8 cast is NOSAT and
# keeps NaN.  The format is OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7),
# 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; the code
# S.1111.111 is NaN; there is no infinity; the largest finite value is 448.
# ---------------------------------------------------------------------------

def e4m3_decode(codes):
    """Value of each E4M3FN code (uint8 array) as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# The non-negative finite lattice in code order (codes 0x00..0x7E, increasing
# values), followed by the first value past it, 480, which sits at code 0x7F:
# rounding there means overflow, which without saturation is NaN.
_POS_LATTICE = np.concatenate([e4m3_decode(np.arange(0x7F, dtype=np.uint8)), [480.0]])


def e4m3_encode(v):
    """Round float64 values to E4M3FN codes: nearest lattice value, ties to the
    even code, NaN/+-inf -> NaN, overflow (rounding past 448) -> NaN.

    Returns uint8 codes; NaN is written as S.1111.111 with the input's sign.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    neg = np.signbit(v)
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    hi = np.searchsorted(_POS_LATTICE, af, side="left")      # first lattice value >= a
    hi = np.minimum(hi, len(_POS_LATTICE) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = af - _POS_LATTICE[lo]
    d_hi = _POS_LATTICE[hi] - af
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(af > _POS_LATTICE[-1], 0x7F, idx)         # beyond 480: overflow
    idx = np.where(finite, idx, 0x7F)                        # NaN / inf -> NaN
    return (idx.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


# ---------------------------------------------------------------------------
# UE8M0 block scale.  [PTO-20] implementation notes: one scale per 1x32 block
# along the hidden dimension, packed as one byte per block; validation covers
# a block whose amax is inf.  Reading: the smallest power of two that brings
# amax into the E4M3 range, so that NOSAT never turns an in-range value into
# NaN.
# ---------------------------------------------------------------------------

def ue8m0_exponent(amax):
    """Smallest integer E with amax <= 448 * 2^E, clamped to [-127, 127];
    E = 128 where amax is +inf.  amax: non-negative float64 array (no NaN)."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = np.isfinite(amax) & (amax > 0)
    _, ex = np.frexp(np.where(pos, amax, 1.0))               # amax in [2^(ex-1), 2^ex)
    E = ex.astype(np.int64) - 10                              # 448 * 2^E < amax here
    for _ in range(4):                                        # linear search upwards
        E = np.where(pos & (amax > np.ldexp(E4M3_MAX, E)), E + 1, E)
    E = np.where(pos, E, -127)
    E = np.clip(E, -127, 127)
    E = np.where(np.isposinf(amax), 128, E)
    return E


def ue8m0_byte(E):
    """Stored scale byte: E + 127 (0xFF for E = 128)."""
    return (np.asarray(E, np.int64) + 127).astype(np.uint8)


# ---------------------------------------------------------------------------
# Elementwise SwiGLU + FP8 block quantisation.  [PTO-20] overview and
# implementation notes: optional clamp with clamp counting, SiLU(g) * u,
# per-row 1x32 block amax, packed UE8M0 scale, E4M3 cast without saturation.
# ---------------------------------------------------------------------------

def clamp_nan_preserving(v, limit):
    """v > L -> L, v < -L -> -L, otherwise v (NaN stays NaN, +-inf -> +-L)."""
    v = np.asarray(v, np.float64)
    return np.where(v > limit, limit, np.where(v < -limit, -limit, v))


def act_fwd(gate, up, clamp_limit=np.inf, act="silu"):
    """The elementwise gated activation without quantisation ([PTO-20]
    forward table: the same kernel with fp32 or bf16 output).  Returns
    (h float64 [rows, cols], clamp_count int): h = act(clamp(gate)) * clamp(up)
    in exact arithmetic, the clamp and its count as in act_quant."""
    gate = np.asarray(gate, np.float64)
    up = np.asarray(up, np.float64)
    assert up.shape == gate.shape
    L = float(clamp_limit)
    count = int(np.count_nonzero(gate > L) + np.count_nonzero(gate < -L)
                + np.count_nonzero(up > L) + np.count_nonzero(up < -L))
    with np.errstate(over="ignore", invalid="ignore"):
        h = ACTIVATIONS[act](clamp_nan_preserving(gate, L)) * clamp_nan_preserving(up, L)
    return h, count


def act_quant(gate, up, clamp_limit=np.inf, act="silu"):
    """Returns (q [rows, cols] uint8 E4M3 codes, scale [rows, cols/32] uint8,
    clamp_count int, h32 [rows, cols] float32).

    h32 is the activation rounded to fp32, the precision in which both sides
    take the scale and code decisions.  act selects the gate activation
    (ACTIVATIONS: "silu", or "gelu_tanh" for the GeGLU variant).
    """
    gate = np.asarray(gate, np.float64)
    up = np.asarray(up, np.float64)
    rows, cols = gate.shape
    assert up.shape == gate.shape and cols % 32 == 0
    L = float(clamp_limit)
    count = int(np.count_nonzero(gate > L) + np.count_nonzero(gate < -L)
                + np.count_nonzero(up > L) + np.count_nonzero(up < -L))
    g = clamp_nan_preserving(gate, L)
    u = clamp_nan_preserving(up, L)
    with np.errstate(over="ignore", invalid="ignore"):
        h64 = ACTIVATIONS[act](g) * u
        h32 = h64.astype(np.float32)
    q, scale = quantize_1x32(h32)
    return q, scale, count, h32


def quantize_1x32(h32):
    """1x32 block quantisation of fp32 activations h32 [rows, cols]:
    amax per block (NaN ignored, all-NaN -> 0), UE8M0 byte, E4M3FN codes of
    h * 2^-E.  Returns (q uint8 [rows, cols], scale uint8 [rows, cols/32])."""
    h32 = np.asarray(h32, dtype=np.float32)
    rows, cols = h32.shape
    blocks = h32.astype(np.float64).reshape(rows, cols // 32, 32)
    mag = np.abs(blocks)
    amax = np.where(np.isnan(mag), -np.inf, mag).max(axis=2)   # NaN ignored
    amax = np.where(amax == -np.inf, 0.0, amax)                 # all-NaN block
    E = ue8m0_exponent(amax)
    scaled = np.ldexp(blocks, -E[:, :, None])                   # exact in float64
    q = e4m3_encode(scaled).reshape(rows, cols)
    return q, ue8m0_byte(E)


# ---------------------------------------------------------------------------
# Elementwise SwiGLU backward on materialised gate/up.  [PTO-20] performance
# section (the backward table: gate/up given, optional clamp, optional
# routing weights with recompute) and implementation notes (weight_grad is a
# reassociated reduction, accepted at 1e-4).  Reading: the forward is
#   y[r, c] = w[r] * SiLU(clamp(g[r, c])) * clamp(u[r, c])
# (w = 1 without weights); the backward takes dy and returns dg, du and
# weight_grad[r] = dL/dw[r] = sum_c dy[r, c] * SiLU(clamp(g)) * clamp(u).
# The clamp passes the gradient where |v| <= L (or v is NaN) and stops it
# where it clamped (|v| > L), the same test as the clamp count.
# ---------------------------------------------------------------------------

def act_bwd(gate, up, dy, clamp_limit=np.inf, weights=None):
    """Returns (dgate, dup, weight_grad) in float64; weight_grad[r] is
    sum_c dy * h with h the (unweighted) activation, also without weights."""
    gate = np.asarray(gate, np.float64)
    up = np.asarray(up, np.float64)
    dy = np.asarray(dy, np.float64)
    assert up.shape == gate.shape == dy.shape
    L = float(clamp_limit)
    g = clamp_nan_preserving(gate, L)
    u = clamp_nan_preserving(up, L)
    pass_g = ~(np.abs(gate) > L)          # NaN compares false: passes
    pass_u = ~(np.abs(up) > L)
    w = np.ones(gate.shape[0]) if weights is None else np.asarray(weights, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        dh = w[:, None] * dy
        dgate = np.where(pass_g, dh * u * silu_grad(g), 0.0)
        dup = np.where(pass_u, dh * silu(g), 0.0)
        weight_grad = np.sum(dy * (silu(g) * u), axis=1)
    return dgate, dup, weight_grad


def act_bwd_fp8(gate, up, dy, clamp_limit=np.inf, weights=None):
    """The backward with E4M3 outputs ([PTO-20] backward table, fmt e4m3; the
    implementation notes' NOSAT FP8 output cast).  Reading: fmt is the format
    of dgate and dup, as it is of h in the forward table, so each leaves in the
    forward's 1x32 format; gate, up and dy keep their own type (bf16 or fp32).
    dgate and dup are act_bwd's exact values rounded once to fp32, the
    precision in which both sides take the scale and code decisions, then
    quantised by quantize_1x32.  weight_grad is act_bwd's.
    Returns (q_dgate, scale_dgate, q_dup, scale_dup, weight_grad)."""
    dgate, dup, weight_grad = act_bwd(gate, up, dy, clamp_limit, weights)
    with np.errstate(over="ignore", invalid="ignore"):
        qg, sg = quantize_1x32(dgate.astype(np.float32))
        qu, su = quantize_1x32(dup.astype(np.float32))
    return qg, sg, qu, su, weight_grad


# ---------------------------------------------------------------------------
# Comparison metrics (test infrastructure, float64).
# ---------------------------------------------------------------------------

def normwise_rel_err(y, r):
    """max|y - r| / max|r| over the whole tensor."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(y - r)) / den) if den > 0 else float(np.max(np.abs(y - r)))


def cosine(y, r):
    y = np.asarray(y, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    ny, nr = np.linalg.norm(y), np.linalg.norm(r)
    if ny == 0 and nr == 0:
        return 1.0
    return float(np.dot(y, r) / (ny * nr))


def e4m3_ordinal(codes):
    """Signed position on the E4M3 line (+0 and -0 are the same point)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)
