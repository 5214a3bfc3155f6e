"""Seeded synthetic inputs for the fused SwiGLU gate/up stage.

This module serves both sides of every comparison: the HIP path and the fp64
oracle receive the very same arrays from it.  It holds none of the method's
arithmetic: only random draws, the rounding of draws to the storage format
(bf16 round-to-nearest-even), and the injection of special values.

Every draw is a function of (seed, stream id), using numpy's PCG64 generator,
so any tensor can be regenerated on its own.

Stream ids: x=1, Wg=2, Wu=3, dh=4, gate=5, up=6, specials=7, dy=8, row
weights=9 (+100 per extra stream when a recipe needs more than one draw for a
tensor).
"""
from __future__ import annotations

import numpy as np

STREAM_X, STREAM_WG, STREAM_WU, STREAM_DH = 1, 2, 3, 4
STREAM_GATE, STREAM_UP, STREAM_SPECIALS = 5, 6, 7
STREAM_DY, STREAM_ROWW = 8, 9


def rng(seed: int, stream: int) -> np.random.Generator:
    """Independent PCG64 generator for one (seed, stream) pair."""
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def normal_f32(shape, std: float, seed: int, stream: int) -> np.ndarray:
    """N(0, std^2) draws, float32.  `std` is the standard deviation."""
    g = rng(seed, stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    NaN stays NaN (quiet), infinities stay infinite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16_bits(shape, std: float, seed: int, stream: int) -> np.ndarray:
    """N(0, std^2) draws rounded to bfloat16; uint16 bit patterns."""
    return f32_to_bf16_bits(normal_f32(shape, std, seed, stream))


def inject_specials(a: np.ndarray, seed: int, stream: int,
                    p_nonfinite: float = 1e-3, p_subnormal: float = 1e-2) -> np.ndarray:
    """Overwrite a float32 array in place with special values and return it.

    Each element independently: with probability p_nonfinite it becomes one
    of {+inf, -inf, NaN} (uniformly); otherwise, with probability p_subnormal,
    a float32 subnormal of random sign with mantissa uniform in [1, 2^23 - 1].
    """
    assert a.dtype == np.float32 and a.flags.c_contiguous
    g = rng(seed, stream)
    n = a.size
    u = g.random(n)
    flat = a.reshape(-1)
    nf = np.nonzero(u < p_nonfinite)[0]
    kinds = g.integers(0, 3, size=nf.size)
    vals = np.array([np.inf, -np.inf, np.nan], dtype=np.float32)
    flat[nf] = vals[kinds]
    sub = np.nonzero((u >= p_nonfinite) & (u < p_nonfinite + (1 - p_nonfinite) * p_subnormal))[0]
    mant = g.integers(1, 1 << 23, size=sub.size, dtype=np.uint32)
    sign = g.integers(0, 2, size=sub.size, dtype=np.uint32) << 31
    flat[sub] = (mant | sign).view(np.float32)
    return a


# --------------------------------------------------------------------------
# The workloads, one function per configuration.  Each returns a dict of
# numpy arrays: bf16 tensors as uint16 bit patterns, fp32 tensors as float32.
# --------------------------------------------------------------------------

def tiny_fp32(seed: int = 0, M: int = 4, N: int = 128, K: int = 64) -> dict:
    """fp32 forward+backward case: x~N(0,1), Wg,Wu~N(0,1)/sqrt(K), dh~N(0,1)."""
    s = 1.0 / np.sqrt(K)
    return dict(
        x=normal_f32((M, K), 1.0, seed, STREAM_X),
        wg=normal_f32((N, K), s, seed, STREAM_WG),
        wu=normal_f32((N, K), s, seed, STREAM_WU),
        dh=normal_f32((M, N), 1.0, seed, STREAM_DH),
    )


def decode_bf16(M: int, N: int, K: int, seed: int = 0) -> dict:
    """bf16 decode case: x~N(0,1) [M,K], Wg,Wu~N(0,0.02) [N,K]."""
    return dict(
        x=normal_bf16_bits((M, K), 1.0, seed, STREAM_X),
        wg=normal_bf16_bits((N, K), 0.02, seed, STREAM_WG),
        wu=normal_bf16_bits((N, K), 0.02, seed, STREAM_WU),
    )


def train_bf16(M: int, N: int, K: int, seed: int = 0, with_dh: bool = True) -> dict:
    """bf16 training case: x~N(0,1), Wg,Wu~N(0,0.02), dh~N(0,0.01)."""
    d = dict(
        x=normal_bf16_bits((M, K), 1.0, seed, STREAM_X),
        wg=normal_bf16_bits((N, K), 0.02, seed, STREAM_WG),
        wu=normal_bf16_bits((N, K), 0.02, seed, STREAM_WU),
    )
    if with_dh:
        d["dh"] = normal_bf16_bits((M, N), 0.01, seed, STREAM_DH)
    return d


def gemm_fp32(M: int, N: int, K: int, seed: int = 0) -> dict:
    """fp32 dual-GEMM case: x~N(0,1), Wg,Wu~N(0,1)/sqrt(K)."""
    s = 1.0 / np.sqrt(K)
    return dict(
        x=normal_f32((M, K), 1.0, seed, STREAM_X),
        wg=normal_f32((N, K), s, seed, STREAM_WG),
        wu=normal_f32((N, K), s, seed, STREAM_WU),
    )


def small_int_bf16(M: int, N: int, K: int, seed: int = 0) -> dict:
    """x, Wg, Wu with integer entries uniform in {-3, ..., 3} as bf16 bits:
    every product and every partial sum over K < 2^20 is an integer below
    2^24, so fp32 accumulation in any order is exact."""
    out = {}
    for name, shape, stream in (("x", (M, K), STREAM_X), ("wg", (N, K), STREAM_WG), ("wu", (N, K), STREAM_WU)):
        a = rng(seed, stream).integers(-3, 4, size=shape).astype(np.float32)
        out[name] = f32_to_bf16_bits(a)
    return out


def small_int_i8(M: int, N: int, K: int, seed: int = 0, amp: int = 1) -> dict:
    """x, Wg, Wu with integer entries uniform in {-amp, ..., amp}, as int8
    (amp <= 127).  Every such integer is exact in bf16 and fp32, so the
    arrays convert exactly to either storage format.  With amp = 1 every
    partial sum over K < 2^24 is an integer of magnitude at most K, so fp32
    accumulation in any order is exact, also at the longest reductions the
    library accepts; int8 keeps the host footprint of those shapes small."""
    out = {}
    for name, shape, stream in (("x", (M, K), STREAM_X), ("wg", (N, K), STREAM_WG), ("wu", (N, K), STREAM_WU)):
        out[name] = rng(seed, stream).integers(-amp, amp + 1, size=shape, dtype=np.int8)
    return out


def act_quant_f32(rows: int, cols: int, seed: int = 0, specials: bool = True) -> dict:
    """Elementwise case: gate,up~N(0,2) fp32 (std 2) with 0.1% +-inf/NaN and 1% subnormals."""
    gate = normal_f32((rows, cols), 2.0, seed, STREAM_GATE)
    up = normal_f32((rows, cols), 2.0, seed, STREAM_UP)
    if specials:
        inject_specials(gate, seed, STREAM_SPECIALS)
        inject_specials(up, seed, STREAM_SPECIALS + 100)
    return dict(gate=gate, up=up)


def act_bwd_f32(rows: int, cols: int, seed: int = 0, specials: bool = False) -> dict:
    """Elementwise backward case: gate, up ~ N(0, 2) and dy ~ N(0, 1) fp32,
    per-row weights ~ U(0, 1); optional specials in gate and up as in
    act_quant_f32."""
    d = act_quant_f32(rows, cols, seed, specials)
    d["dy"] = normal_f32((rows, cols), 1.0, seed, STREAM_DY)
    d["weights"] = rng(seed, STREAM_ROWW).uniform(0.0, 1.0, rows).astype(np.float32)
    return d


def act_bwd_bf16(rows: int, cols: int, seed: int = 0, specials: bool = False) -> dict:
    """act_bwd_f32's values with gate, up and dy rounded (RNE) to bf16 bits;
    weights stay fp32."""
    d = act_bwd_f32(rows, cols, seed, specials)
    for k in ("gate", "up", "dy"):
        d[k] = f32_to_bf16_bits(d[k])
    return d
