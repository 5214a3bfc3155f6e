"""Helpers shared by the GPU parity tests: host<->device transfer of the
synthetic inputs, and the tolerance checks.

Tolerances, with their derivation:
  * the gates stated for the path: normwise relative error max|y-r|/max|r|
    <= 1e-5 for fp32 and <= 2e-2 for bf16, cosine >= 0.9999 for bf16;
  * an elementwise bound per output built from |A||B| products: with
    u = 2^-24, fp32 accumulation of n exact products errs by at most
    gamma_n * sum|a||b| (gamma_n = n u / (1 - n u)); a bf16 operand rounding
    adds 2^-8 * sum|a||b|; the final rounding adds half an ulp of the output
    type (2^-8 relative for bf16, which keeps 8 significant bits; 2^-24 for
    fp32).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synth

U32 = 2.0 ** -24
BF16_HALF_ULP = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits)


GUARD_BYTES = 4096   # a multiple of 256: the view keeps the buffer's alignment


def _guard_pattern(device) -> torch.Tensor:
    return ((torch.arange(2 * GUARD_BYTES, dtype=torch.int64) * 37 + 11) % 251).to(torch.uint8).to(device)


class Guarded:
    """A device output that sits inside a larger buffer.

    GUARD_BYTES on each side hold a fixed byte pattern, and the output itself
    is filled with 0xFF bytes (NaN for bf16 and fp32, the NaN code for E4M3):
    an element the kernel leaves unwritten then fails the comparison, and a
    byte written before or after the output fails check().
    """

    def __init__(self, shape, dtype, device="cuda"):
        self.shape = tuple(int(v) for v in shape)
        self.n = math.prod(self.shape) * torch.empty((), dtype=dtype).element_size()
        self.pattern = _guard_pattern(device)
        self.buf = torch.empty(self.n + 2 * GUARD_BYTES, dtype=torch.uint8, device=device)
        self.buf[:GUARD_BYTES].copy_(self.pattern[:GUARD_BYTES])
        self.buf[GUARD_BYTES + self.n:].copy_(self.pattern[GUARD_BYTES:])
        self.buf[GUARD_BYTES:GUARD_BYTES + self.n].fill_(0xFF)
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + self.n].view(dtype).view(self.shape)

    def check(self, what: str) -> None:
        torch.cuda.synchronize()
        head = self.buf[:GUARD_BYTES]
        tail = self.buf[GUARD_BYTES + self.n:]
        assert torch.equal(head, self.pattern[:GUARD_BYTES]), f"{what}: bytes written before the output"
        assert torch.equal(tail, self.pattern[GUARD_BYTES:]), f"{what}: bytes written past the output"


def guarded(shape, dtype, device="cuda") -> Guarded:
    return Guarded(shape, dtype, device)


def check_guards(what: str, *gs) -> None:
    for i, g in enumerate(gs):
        if g is not None:
            g.check(f"{what} (output {i})")


def gamma(n: int, u: float = U32) -> float:
    return n * u / (1 - n * u)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def f64_of(bits_or_f32: np.ndarray) -> np.ndarray:
    if bits_or_f32.dtype == np.uint16:
        return synth.bf16_bits_to_f32(bits_or_f32).astype(np.float64)
    return bits_or_f32.astype(np.float64)


def assert_gates(y, r, dtype: str, what: str):
    """The stated gates: normwise relative error and (bf16) cosine."""
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    e = oracle.normwise_rel_err(y, r)
    c = oracle.cosine(y, r)
    if dtype == "f32":
        assert e <= 1e-5, f"{what}: normwise rel err {e:.3e} > 1e-5"
    else:
        assert e <= 2e-2, f"{what}: normwise rel err {e:.3e} > 2e-2"
        assert c >= 0.9999, f"{what}: cosine {c:.6f} < 0.9999"
    return e, c


def assert_within(y, r, bound, what: str):
    """Elementwise |y - r| <= bound; reports the worst ratio."""
    err = np.abs(y - r)
    ratio = np.max(err / np.maximum(bound, 1e-300))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements exceed the bound; first {bad[:3].tolist()}, "
                           f"worst ratio {ratio:.3g}")
    return ratio


def fwd_bound(x, wg, wu, dtype: str, rows=None, act: str = "silu", gate_mult: float = 1.0, up_mult: float = 1.0):
    """Elementwise error bound of the fused forward h = act(g) u on the given rows.

    g and u carry the fp32 accumulation error E = gamma_{K+1} sum|x||w| (the +1
    covers the rounding of fp32 products on the fp32 path; bf16 products are
    exact); it reaches h through |act'(g)| |u| E_g + |act(g)| E_u (|silu'| is
    below 1.1, |gelu_tanh'| below 1.13).  The activation itself is good to a
    few fp32 ulps (8 u |h| covers it) and the output rounding adds 2^-8 |h|
    (bf16) or u |h| (fp32).
    """
    xr = x if rows is None else x[rows]
    K = x.shape[1]
    # With multipliers the device forms fl(m * acc): the accumulation error
    # scales with |m| (so does sum|x||w|), and the extra rounding, u |m g|, is
    # below gamma_{K+1} sum|x||m w|, which the propagation term already holds.
    h = oracle.glu_fwd(xr, wg, wu, act, gate_mult, up_mult)
    ws, us = gate_mult * np.asarray(wg, np.float64), up_mult * np.asarray(wu, np.float64)
    g, u = oracle.gate_up(xr, ws, us)
    Sg = np.abs(xr) @ np.abs(ws).T
    Su = np.abs(xr) @ np.abs(us).T
    G = gamma(K + 1)
    a = oracle.ACTIVATIONS[act](g)
    prop = 1.2 * np.abs(u) * G * Sg + np.abs(a) * G * Su + G * Sg * G * Su
    out = BF16_HALF_ULP if dtype == "bf16" else U32
    return h, 2 * (prop + (8 * U32 + out) * np.abs(h)) + 1e-30


def dsw_terms(x, wg, wu, dh):
    g, u = oracle.gate_up(x, wg, wu)
    dg, du = oracle.dswiglu(g, u, dh)
    return g, u, dg, du
