"""GPU parity of the HIP path against the fp64 oracle (MI355X, through the C ABI).

Each case generates seeded synthetic inputs on the host, runs the library on
cuda:0 and compares element by element with the oracle on the same values:
the stated gates (normwise relative error, cosine) and an elementwise bound
derived from the arithmetic (parity_util).  Full-size cases compare every
element where the oracle is cheap, and sampled rows/columns where it is not.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (BF16_HALF_ULP, U32, assert_gates, assert_within, check_guards, dev_bf16, dev_f32, f64_of,
                         fwd_bound, gamma, guarded, host_f64)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the parity tests need the GPU; the CPU suite skips this file
    pytest.skip("no GPU visible", allow_module_level=True)

import swiglu_mlp_fwd_amd as S  # noqa: E402

DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def log(msg):
    print(msg, flush=True)


def to_dev(d: dict) -> dict:
    return {k: (dev_bf16(v) if v.dtype == np.uint16 else dev_f32(v)) for k, v in d.items()}


def to_f64(d: dict) -> dict:
    return {k: f64_of(v) for k, v in d.items()}


# ----------------------------------------------------------------- forward

def check_fwd(d, dtype, rows=None, what="fwd", via="dual", act="silu", mult=(1.0, 1.0)):
    t = to_dev(d)
    f = to_f64(d)
    M, N = t["x"].shape[0], t["wg"].shape[0]
    hg = guarded((M, N), t["x"].dtype)
    if via == "dual":
        h = S.fwd(t["x"], t["wg"], t["wu"], act=act, gate_mult=mult[0], up_mult=mult[1], out=hg.t)
    else:
        h = S.gemv_fwd(t["x"], t["wg"], t["wu"], act=act, gate_mult=mult[0], up_mult=mult[1], out=hg.t)
    torch.cuda.synchronize()
    check_guards(what, hg)
    y = host_f64(h if rows is None else h[torch.as_tensor(rows, device=DEV)])
    ref, bound = fwd_bound(f["x"], f["wg"], f["wu"], dtype, rows, act, mult[0], mult[1])
    e, c = assert_gates(y, ref, dtype, what)
    ratio = assert_within(y, ref, bound, what)
    log(f"{what}: normwise {e:.3e} cosine {c:.7f} bound-ratio {ratio:.3f}")
    return h


def test_fwd_tiny_fp32():
    d = synth.tiny_fp32(seed=0)
    d.pop("dh")
    check_fwd(d, "f32", what="fwd fp32 4x128x64")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 520, 264), (1, 1, 8), (129, 127, 72), (37, 300, 1032)])
def test_fwd_ragged(dt, shape):
    M, N, K = shape
    d = synth.train_bf16(M, N, K, seed=1, with_dh=False) if dt == "bf16" else synth.gemm_fp32(M, N, K, seed=1)
    check_fwd(d, dt, what=f"fwd {dt} {shape}")


def test_fwd_fp32_full_4001x3584x2048():
    """fp32 IEEE dual GEMM at M=4001, K=2048, N=3584, every element."""
    d = synth.gemm_fp32(4001, 3584, 2048, seed=0)
    check_fwd(d, "f32", what="fwd fp32 4001x3584x2048")


def test_fwd_bf16_full_8192x14336x4096_sampled_and_deterministic():
    M, N, K = 8192, 14336, 4096
    d = synth.train_bf16(M, N, K, seed=0, with_dh=False)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], np.random.default_rng(0).integers(0, M, 59)]))
    h = check_fwd(d, "bf16", rows=rows, what="fwd bf16 8192x14336x4096 (sampled rows)")
    t = to_dev(d)
    h2 = S.fwd(t["x"], t["wg"], t["wu"])
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), "forward is not deterministic"
    del h, h2, t
    torch.cuda.empty_cache()


def test_fwd_k_zero_gives_zero():
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((7, 0), dtype=torch.bfloat16, device=DEV)
    h = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device=DEV)
    S.fwd(x, w, w, out=h)
    torch.cuda.synchronize()
    assert torch.count_nonzero(h).item() == 0


def test_fwd_rank3_flatten_restore():
    d = synth.train_bf16(6, 40, 64, seed=3, with_dh=False)
    t = to_dev(d)
    x3 = t["x"].reshape(2, 3, 64)
    h3 = S.fwd(x3, t["wg"], t["wu"])
    h2 = S.fwd(t["x"], t["wg"], t["wu"])
    torch.cuda.synchronize()
    assert h3.shape == (2, 3, 40)
    assert torch.equal(h3.reshape(6, 40).view(torch.int16), h2.view(torch.int16))


# ---------------------------------------------------------------- backward

def bwd_bounds(f, dtype, rows=None, cols=None, mult=(1.0, 1.0), act="silu"):
    """Elementwise bounds for dX (rows) and dWg/dWu (cols) from |.| products.

    dg and du carry: the recompute error of g, u (gamma_{K+1} sum|x||w|)
    propagated through the dSwiGLU formula, a few fp32 ulps of the
    activation, and their rounding to the operand type (2^-8 for bf16).  The
    contractions add gamma_n of the absolute products and the output
    rounding.  A factor 2 of headroom is applied.

    With multipliers (mg, mu) the terms are those of the problem with weights
    mg Wg and mu Wu (the scaled projections are what the epilogue sees); dX is
    the same, dWg and dWu, and their bounds, carry the factor mg or mu.  The
    two extra roundings of the scaled dg, du sit inside the 16 ulps of the
    activation term.
    """
    mg, mu = mult
    x, dh = f["x"], f["dh"]
    wg, wu = mg * f["wg"], mu * f["wu"]
    M, K = x.shape
    N = wg.shape[0]
    op = BF16_HALF_ULP if dtype == "bf16" else 0.0
    out = BF16_HALF_ULP if dtype == "bf16" else U32
    GK = gamma(K + 1)

    # |act''| is below 0.5 (SiLU) and 0.8 (GELU-tanh); |act'| below 1.1 and 1.13.
    d2max, d1max = (0.5, 1.1) if act == "silu" else (0.85, 1.2)

    def terms(xs, wgs, wus, dhs):
        g, u = oracle.gate_up(xs, wgs, wus)
        dg, du = oracle.dswiglu(g, u, dhs) if act == "silu" else oracle.dglu(g, u, dhs, act)
        Eg = GK * (np.abs(xs) @ np.abs(wgs).T)
        Eu = GK * (np.abs(xs) @ np.abs(wus).T)
        d1 = np.abs(oracle.ACTIVATION_GRADS[act](g))
        ddg = np.abs(dh_ := dhs) * (d1 * Eu + d2max * np.abs(u) * Eg) + (op + 16 * U32) * np.abs(dg)
        ddu = np.abs(dh_) * d1max * Eg + (op + 16 * U32) * np.abs(du)
        return dg, du, ddg, ddu

    res = {}
    if rows is not None:
        dg, du, ddg, ddu = terms(x[rows], wg, wu, dh[rows])
        dx = dg @ wg + du @ wu
        absprod = np.abs(dg) @ np.abs(wg) + np.abs(du) @ np.abs(wu)
        b = ddg @ np.abs(wg) + ddu @ np.abs(wu) + gamma(2 * N + 1) * absprod * (1 + op) + out * np.abs(dx)
        res["dx"] = (dx, 2 * b + 1e-30)
    if cols is not None:
        dg, du, ddg, ddu = terms(x, wg[cols], wu[cols], dh[:, cols])
        dwg, dwu = dg.T @ x, du.T @ x
        bg = ddg.T @ np.abs(x) + gamma(M + 1) * (np.abs(dg).T @ np.abs(x)) * (1 + op) + out * np.abs(dwg)
        bu = ddu.T @ np.abs(x) + gamma(M + 1) * (np.abs(du).T @ np.abs(x)) * (1 + op) + out * np.abs(dwu)
        res["dwg"] = (mg * dwg, 2 * abs(mg) * bg + 1e-30)
        res["dwu"] = (mu * dwu, 2 * abs(mu) * bu + 1e-30)
    # The oracle's own multiplier backward gives the same references.
    if rows is not None:
        r = oracle.swiglu_bwd_dx_rows(f["x"], f["wg"], f["wu"], dh, rows, mg, mu, act)
        assert oracle.normwise_rel_err(r, res["dx"][0]) < 1e-12   # fp64 association only
    return res


def check_bwd(d, dtype, rows=None, cols=None, what="bwd", mult=(1.0, 1.0), act="silu"):
    M = d["x"].shape[0]
    N = d["wg"].shape[0]
    rows = np.arange(M) if rows is None else rows
    cols = np.arange(N) if cols is None else cols
    t = to_dev(d)
    f = to_f64(d)
    K = t["x"].shape[1]
    dt = t["x"].dtype
    outs = [guarded((M, K), dt), guarded((N, K), dt), guarded((N, K), dt)]
    ws = guarded((max(S.bwd_workspace_bytes(dt, M, N, K), 1),), torch.uint8)
    dx, dwg, dwu = S.bwd(t["x"], t["wg"], t["wu"], t["dh"], gate_mult=mult[0], up_mult=mult[1], act=act,
                         out=tuple(g.t for g in outs), workspace=ws.t)
    torch.cuda.synchronize()
    check_guards(what, *outs, ws)
    ref = bwd_bounds(f, dtype, rows, cols, mult, act)
    ri = torch.as_tensor(rows, device=DEV)
    ci = torch.as_tensor(cols, device=DEV)
    got = {"dx": host_f64(dx[ri]), "dwg": host_f64(dwg[ci]), "dwu": host_f64(dwu[ci])}
    for k in ("dx", "dwg", "dwu"):
        r, b = ref[k]
        e, c = assert_gates(got[k], r, dtype, f"{what} {k}")
        ratio = assert_within(got[k], r, b, f"{what} {k}")
        log(f"{what} {k}: normwise {e:.3e} cosine {c:.7f} bound-ratio {ratio:.3f}")
    return dx, dwg, dwu


def test_bwd_tiny_fp32():
    check_bwd(synth.tiny_fp32(seed=0), "f32", what="bwd fp32 4x128x64")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 520, 264), (1, 1, 8), (33, 17, 40), (129, 300, 136),
                                   (520, 700, 328), (257, 640, 520)])
def test_bwd_ragged(dt, shape):
    M, N, K = shape
    if dt == "bf16":
        d = synth.train_bf16(M, N, K, seed=2)
    else:
        d = synth.gemm_fp32(M, N, K, seed=2)
        d["dh"] = synth.normal_f32((M, N), 1.0, 2, synth.STREAM_DH)
    check_bwd(d, dt, what=f"bwd {dt} {shape}")


def test_bwd_bf16_full_8192x14336x4096_sampled():
    M, N, K = 8192, 14336, 4096
    d = synth.train_bf16(M, N, K, seed=0)
    rs = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, M - 1], rs.integers(0, M, 30)]))
    cols = np.unique(np.concatenate([[0, N - 1], rs.integers(0, N, 30)]))
    check_bwd(d, "bf16", rows=rows, cols=cols, what="bwd bf16 8192x14336x4096 (sampled)")
    torch.cuda.empty_cache()


def test_bwd_fp32_4001x3584x2048_sampled():
    """The IEEE-fp32 backward at the fp32 workload's size: 4001 tokens (a
    ragged last row tile), reductions of 2 x 3584 and 4001, on 32 sampled
    rows of dX and of dWg, dWu."""
    M, N, K = 4001, 3584, 2048
    d = synth.gemm_fp32(M, N, K, seed=5)
    d["dh"] = synth.normal_f32((M, N), 1.0, 5, synth.STREAM_DH)
    rs = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, M - 1], rs.integers(0, M, 30)]))
    cols = np.unique(np.concatenate([[0, N - 1], rs.integers(0, N, 30)]))
    check_bwd(d, "f32", rows=rows, cols=cols, what="bwd fp32 4001x3584x2048 (sampled)")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("shape", [(257, 136, 72), (24, 48, 64), (40, 8, 8), (300, 1032, 136)])
def test_bwd_dh_tile_edges(shape, act):
    """N % 8 == 0, so the recompute moves the dh tile to LDS by DMA: a column
    tail (chunks past N fixed in LDS), a row tail (rows past M read as zero),
    a single reduction step (K <= 64: the tile moves after the prologue) and
    two steps (it replaces the last refill)."""
    M, N, K = shape
    check_bwd(synth.train_bf16(M, N, K, seed=5), "bf16", act=act, what=f"bwd bf16 {act} {shape}")


def test_bwd_empty_sums_are_zero():
    K = 16
    x = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    w = torch.randn((5, K), device=DEV).to(torch.bfloat16)
    dh = torch.empty((0, 5), dtype=torch.bfloat16, device=DEV)
    dx, dwg, dwu = S.bwd(x, w, w, dh)
    torch.cuda.synchronize()
    assert dx.shape == (0, K) and torch.count_nonzero(dwg).item() == 0 and torch.count_nonzero(dwu).item() == 0
    x = torch.randn((3, K), device=DEV).to(torch.bfloat16)
    w0 = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    dh = torch.empty((3, 0), dtype=torch.bfloat16, device=DEV)
    dx, dwg, dwu = S.bwd(x, w0, w0, dh)
    torch.cuda.synchronize()
    assert dx.shape == (3, K) and torch.count_nonzero(dx).item() == 0


def test_autograd_matches_explicit_backward():
    d = synth.train_bf16(24, 48, 64, seed=4)
    t = to_dev(d)
    x = t["x"].reshape(2, 12, 64).clone().requires_grad_(True)
    wg = t["wg"].clone().requires_grad_(True)
    wu = t["wu"].clone().requires_grad_(True)
    h = S.swiglu(x, wg, wu)
    h.backward(t["dh"].reshape(2, 12, 48))
    dx, dwg, dwu = S.bwd(t["x"], t["wg"], t["wu"], t["dh"])
    torch.cuda.synchronize()
    assert torch.equal(x.grad.reshape(24, 64).view(torch.int16), dx.view(torch.int16))
    assert torch.equal(wg.grad.view(torch.int16), dwg.view(torch.int16))
    assert torch.equal(wu.grad.view(torch.int16), dwu.view(torch.int16))


# ----------------------------------------------------------------- decode

@pytest.mark.parametrize("M", [1, 2, 4, 8])
@pytest.mark.parametrize("NK", [(6912, 1536), (11008, 4096), (13824, 5120), (24576, 6144)])
def test_gemv_full(M, NK):
    """Every element, at the benchmark page's decode shapes: (6912, 1536), the
    LLaMA-7B-like (11008, 4096), and the wide LLaMA-2 13B (13824, 5120) and
    GPT-NeoX-20B (24576, 6144) up/gate shapes.  M = 1, 2 run the vector-ALU
    kernel, M = 4, 8 the matrix-core one."""
    N, K = NK
    d = synth.decode_bf16(M, N, K, seed=0)
    check_fwd(d, "bf16", what=f"gemv M={M} N={N} K={K}", via="gemv")


@pytest.mark.parametrize("M", [1, 3, 5, 6, 7, 8])
@pytest.mark.parametrize("NK", [(13, 8), (1, 64), (257, 520)])
def test_gemv_ragged(M, NK):
    N, K = NK
    d = synth.decode_bf16(M, N, K, seed=5)
    check_fwd(d, "bf16", what=f"gemv M={M} N={N} K={K}", via="gemv")


@pytest.mark.parametrize("M,N,K", [(8, 300, 20480), (5, 77, 16392), (8, 16, 4104), (3, 129, 10928),
                                   (1, 40, 40968), (2, 33, 32776)])
def test_gemv_long_reductions(M, N, K):
    """Long reductions through both decode kernels.  M >= 4 runs on the
    matrix cores, whose 8 waves split K into 128-wide slabs: 160 slabs, 20
    per wave; 129 slabs, the last holding one 16-byte chunk; 33 slabs.  M <=
    3 with x past 64 KiB stages x through LDS in phases along K: 3 rows of
    1366 chunks (phases of 704 and 662), 1 row of 5121 (three phases), 2 rows
    of 4097 (four phases, the last ragged)."""
    d = synth.decode_bf16(M, N, K, seed=7)
    check_fwd(d, "bf16", what=f"gemv M={M} N={N} K={K}", via="gemv")
    # the read-only twin walks the same loads and still reads every weight once
    t = to_dev(d)
    sink = torch.full((N + 64,), -1, dtype=torch.int32, device=DEV)
    S.probe_gemv_read(t["x"], t["wg"], t["wu"], sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = (np.bitwise_xor.reduce(d["wg"].view(np.uint32), axis=1) ^
            np.bitwise_xor.reduce(d["wu"].view(np.uint32), axis=1))
    assert np.array_equal(got[:N], want)
    assert np.all(got[N:] == np.uint32(0xFFFFFFFF))


@pytest.mark.parametrize("M,N,K", [(8, 200, 1664), (4, 77, 3968), (8, 33, 2048), (5, 130, 896), (8, 16, 1544),
                                   (6, 48, 3920), (8, 64, 2816), (4, 40, 1152), (7, 24, 2560), (8, 18, 384)])
def test_gemv_short_reductions(M, N, K):
    """Short reductions (fewer than 32 slabs of 128) on the matrix cores run
    as many waves as divide the slab count when that is 4 to 8, else 8 waves
    (one per slab below 8) with shares that differ by one slab, each wave
    taking its slabs two at a time: 13 slabs (8 waves of 1 or 2), 31 (8
    waves of 3 or 4), 16 (8 waves of a pair), 7 (7 waves of one slab), 13
    and 31 with a partial last slab (1 and 10 chunks), 22 (8 waves of 2 or
    3), 9 (8 waves of 1 or 2), 20 (5 waves of 4), 3 (3 waves of one slab).
    The read-only twin takes the same path and reads every weight once."""
    d = synth.decode_bf16(M, N, K, seed=9)
    check_fwd(d, "bf16", what=f"gemv M={M} N={N} K={K}", via="gemv")
    t = to_dev(d)
    sink = torch.full((N + 64,), -1, dtype=torch.int32, device=DEV)
    S.probe_gemv_read(t["x"], t["wg"], t["wu"], sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = (np.bitwise_xor.reduce(d["wg"].view(np.uint32), axis=1) ^
            np.bitwise_xor.reduce(d["wu"].view(np.uint32), axis=1))
    assert np.array_equal(got[:N], want)
    assert np.all(got[N:] == np.uint32(0xFFFFFFFF))


def test_gemv_rotated_copies_agree():
    """The bench rotates weight copies; every copy gives the same bits."""
    d = synth.decode_bf16(4, 6912, 1536, seed=0)
    t = to_dev(d)
    outs = []
    for _ in range(3):
        wg, wu = t["wg"].clone(), t["wu"].clone()
        outs.append(S.gemv_fwd(t["x"], wg, wu))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


# -------------------------------------------------------------- act_quant

def f32_ulp_distance(a, b):
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    oa = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ob = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(oa - ob)


H_ULP_MAX = 8   # the device activation is within this many fp32 ulps of the rounded exact value


def check_act_quant(gate, up, L, what, act="silu"):
    rows, cols = gate.shape
    gs = [guarded((rows, cols), torch.uint8), guarded((rows, cols // 32), torch.uint8),
          guarded((1,), torch.int64), guarded((rows, cols), torch.float32)]
    q, sc, cnt, h = S.act_quant(dev_f32(gate), dev_f32(up), L, act=act, out=tuple(g.t for g in gs))
    torch.cuda.synchronize()
    check_guards(what, *gs)
    q, sc, h = q.cpu().numpy(), sc.cpu().numpy(), h.cpu().numpy()
    rq, rs, rc, rh = oracle.act_quant(gate.astype(np.float64), up.astype(np.float64), L, act=act)
    # 1. clamp count: exact.
    assert int(cnt.item()) == rc, f"{what}: clamp count {int(cnt.item())} != {rc}"
    # 2. the activation h: same NaN/inf pattern, finite values within H_ULP_MAX ulps.
    nan_d, nan_r = np.isnan(h), np.isnan(rh)
    assert np.array_equal(nan_d, nan_r), f"{what}: NaN pattern of h differs"
    fin = ~nan_r
    assert np.array_equal(h[fin & np.isinf(rh)], rh[fin & np.isinf(rh)])
    ulp = f32_ulp_distance(h[fin], rh[fin])
    assert ulp.max() <= H_ULP_MAX, f"{what}: h off by {ulp.max()} ulps"
    # 3. same precision: the oracle's quantiser on the device's own h is bit-exact.
    oq, os_ = oracle.quantize_1x32(h)
    assert np.array_equal(sc, os_), f"{what}: scales differ from oracle(quantise(device h))"
    nq = (q & 0x7F) == 0x7F
    assert np.array_equal(nq, (oq & 0x7F) == 0x7F)
    assert np.array_equal(q[~nq], oq[~nq]), f"{what}: codes differ from oracle(quantise(device h))"
    # 4. against the oracle from the inputs: scales bit-exact except where the
    #    block amax sits within H_ULP_MAX ulps of a scale boundary 1.75 * 2^k.
    blocks = rh.astype(np.float64).reshape(rows, cols // 32, 32)
    amax = np.where(np.isnan(blocks), 0, np.abs(blocks)).max(axis=2)
    diff = sc != rs
    if diff.any():
        a = amax[diff]
        _, ex = np.frexp(a)
        bnd = 1.75 * np.exp2(ex - 1.0)
        near = np.abs(a - bnd) <= H_ULP_MAX * np.spacing(bnd.astype(np.float32)).astype(np.float64)
        assert near.all(), f"{what}: {int((~near).sum())} scale bytes differ away from a boundary"
    same = np.repeat(~diff, 32, axis=1)
    assert np.array_equal(((q & 0x7F) == 0x7F), ((rq & 0x7F) == 0x7F)), f"{what}: NaN code positions differ"
    ok = same & ~nq
    dist = np.abs(oracle.e4m3_ordinal(q[ok]) - oracle.e4m3_ordinal(rq[ok]))
    assert dist.max(initial=0) <= 1, f"{what}: code off by {dist.max()} ulps"
    log(f"{what}: count {rc}, h max ulp {ulp.max()}, scale diffs {int(diff.sum())}, "
        f"codes off by 1: {int((dist == 1).sum())} of {dist.size}")


@pytest.mark.parametrize("L", [math.inf, 7.0, 0.5])
def test_act_quant_full_4001x3584(L):
    d = synth.act_quant_f32(4001, 3584, seed=0)
    check_act_quant(d["gate"], d["up"], L, f"act_quant 4001x3584 L={L}")


@pytest.mark.parametrize("shape", [(1, 32), (3, 384), (7, 2048), (1, 96)])
def test_act_quant_ragged(shape):
    d = synth.act_quant_f32(*shape, seed=6)
    check_act_quant(d["gate"], d["up"], 7.0, f"act_quant {shape}")


def test_act_quant_adversarial_subnormal_and_huge():
    rs = np.random.default_rng(9)
    rows, cols = 64, 256
    mant = rs.integers(1, 1 << 23, rows * cols, dtype=np.uint32)
    gate = (mant | (rs.integers(0, 2, rows * cols, dtype=np.uint32) << 31)).view(np.float32).reshape(rows, cols)
    up = (rs.standard_normal((rows, cols)) * np.exp2(rs.integers(-20, 100, (rows, cols)))).astype(np.float32)
    check_act_quant(gate.copy(), up, math.inf, "act_quant subnormal gate, huge up")
    gate2 = rs.uniform(-30, 30, (rows, cols)).astype(np.float32)
    up2 = rs.uniform(-1e-30, 1e-30, (rows, cols)).astype(np.float32)
    check_act_quant(gate2, up2, math.inf, "act_quant tiny products")


def _load_cases():
    with open(os.path.join(GOLDEN, "act_quant_cases.json")) as f:
        return json.load(f)["cases"]


def _hexf(s):
    return float(s) if s in ("inf", "-inf", "nan") else float.fromhex(s)


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_act_quant_hand_cases_on_device(case):
    """The hand-derived cases (tests/golden) through the HIP kernel."""
    rows, cols = case["rows"], case["cols"]

    def fill(spec):
        a = np.full(rows * cols, _hexf(spec["fill"]), dtype=np.float64)
        for k, v in spec.get("set", {}).items():
            a[int(k)] = _hexf(v)
        return a.astype(np.float32).reshape(rows, cols)

    gate, up = fill(case["gate"]), fill(case["up"])
    q, sc, cnt, h = S.act_quant(dev_f32(gate), dev_f32(up), _hexf(case["clamp"]), h_out=True)
    torch.cuda.synchronize()
    q, sc, h = q.cpu().numpy(), sc.cpu().numpy(), h.cpu().numpy().reshape(-1)
    for k, v in case.get("expect_h", {}).items():
        want = _hexf(v)
        assert h[int(k)] == want and np.signbit(h[int(k)]) == np.signbit(want), (k, h[int(k)], want)
    np.testing.assert_array_equal(sc, np.array(case["expect_scale"], dtype=np.uint8))
    assert int(cnt.item()) == case["expect_count"]
    exp = case["expect_codes"]
    for i, c in enumerate(q.reshape(-1)):
        want = exp.get(str(i), exp["default"])
        if want == "nan":
            assert (c & 0x7F) == 0x7F, (i, hex(c))
        else:
            assert c == want, (i, hex(c), hex(want))


def test_act_quant_empty_and_count_reset():
    cnt = torch.full((1,), 12345, dtype=torch.int64, device=DEV)
    e = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    q = torch.empty((0, 64), dtype=torch.uint8, device=DEV)
    s = torch.empty((0, 2), dtype=torch.uint8, device=DEV)
    S.act_quant(e, e, 7.0, out=(q, s, cnt, None))
    torch.cuda.synchronize()
    assert cnt.item() == 0
    # With the clamp off the count is written as zero too.
    d = synth.act_quant_f32(4, 64, seed=1)
    cnt.fill_(777)
    q = torch.empty((4, 64), dtype=torch.uint8, device=DEV)
    s = torch.empty((4, 2), dtype=torch.uint8, device=DEV)
    S.act_quant(dev_f32(d["gate"]), dev_f32(d["up"]), math.inf, out=(q, s, cnt, None))
    torch.cuda.synchronize()
    assert cnt.item() == 0


def test_clamp_counts_over_many_calls():
    """Counting calls of act_quant and act_fwd take the 16 regions of the
    library's count slots in turn: 40 calls of different sizes and limits
    (more than two full turns), enqueued back to back before any is read,
    each with the oracle's count; the largest fills 8192 workgroups' slots."""
    calls = []
    for i in range(20):
        R, C = (4001, 3584) if i == 7 else (37 + 13 * i, 96)
        d = synth.act_quant_f32(R, C, seed=100 + i)
        L = 0.5 + 0.25 * i
        g, u = dev_f32(d["gate"]), dev_f32(d["up"])
        _, _, cq, _ = S.act_quant(g, u, L)
        _, cf = S.act_fwd(g, u, L, out_dtype=torch.bfloat16)
        calls.append((d, L, cq, cf))
    torch.cuda.synchronize()
    for d, L, cq, cf in calls:
        _, want = oracle.act_fwd(d["gate"], d["up"], L)
        assert cq.item() == want, (d["gate"].shape, L, cq.item(), want)
        assert cf.item() == want, (d["gate"].shape, L, cf.item(), want)


def test_act_quant_deterministic():
    d = synth.act_quant_f32(512, 1024, seed=2)
    g, u = dev_f32(d["gate"]), dev_f32(d["up"])
    a = S.act_quant(g, u, 7.0)
    b = S.act_quant(g, u, 7.0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and a[2].item() == b[2].item()


# ------------------------------------------------------------------ probe

def test_probe_mfma_runs():
    sink = torch.zeros(64, dtype=torch.float32, device=DEV)
    flops = S.probe_mfma(16, 64, sink)
    torch.cuda.synchronize()
    assert flops == 2 * 32 * 32 * 16 * 4 * 8 * 16 * 64
    assert torch.isfinite(sink).all() and torch.count_nonzero(sink).item() > 0


@pytest.mark.parametrize("M,N,K", [(1, 6912, 1536), (8, 11008, 4096), (8, 24576, 6144), (3, 257, 520),
                                   (6, 13, 8)])
def test_probe_gemv_read_reads_every_weight(M, N, K):
    """The decode kernel's read-only twin: column n's word is the XOR of every
    32-bit word of Wg[n, :] and Wu[n, :], so a skipped or repeated load shows."""
    d = synth.decode_bf16(M, N, K, seed=3)
    t = to_dev(d)
    sink = torch.full((N + 64,), -1, dtype=torch.int32, device=DEV)
    S.probe_gemv_read(t["x"], t["wg"], t["wu"], sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = (np.bitwise_xor.reduce(d["wg"].view(np.uint32), axis=1) ^
            np.bitwise_xor.reduce(d["wu"].view(np.uint32), axis=1))
    assert np.array_equal(got[:N], want), "the twin's fold differs from the weights' XOR"
    assert np.all(got[N:] == np.uint32(0xFFFFFFFF)), "the twin wrote past its N columns"


@pytest.mark.parametrize("shape", [(4001, 3584), (3, 384), (1, 32)])
def test_probe_act_quant_stream_moves_the_quantiser_bytes(shape):
    """The quantiser's twin writes, for each 4 consecutive elements, the XOR
    of their gate and up words (4 bytes of q), and for each 1x32 block the
    low byte of that fold of its first 4 elements: every input is read and
    exactly the quantiser's outputs written."""
    R, C = shape
    d = synth.act_quant_f32(R, C, seed=6)
    gs = [guarded((R, C), torch.uint8), guarded((R, C // 32), torch.uint8)]
    S.probe_act_quant_stream(dev_f32(d["gate"]), dev_f32(d["up"]), gs[0].t, gs[1].t)
    torch.cuda.synchronize()
    check_guards(f"act_quant twin {shape}", *gs)
    gw = d["gate"].view(np.uint32).reshape(-1, 4)
    uw = d["up"].view(np.uint32).reshape(-1, 4)
    fold = np.bitwise_xor.reduce(gw, axis=1) ^ np.bitwise_xor.reduce(uw, axis=1)      # [elements / 4]
    got = gs[0].t.cpu().numpy().reshape(-1).view(np.uint32)
    assert np.array_equal(got, fold)
    want_s = (fold.reshape(-1, 8)[:, 0] & 0xFF).astype(np.uint8)                      # first 4 of each block
    assert np.array_equal(gs[1].t.cpu().numpy().reshape(-1), want_s)


def _device_runs(kind, first, last, cap=8192):
    """The device's result as runs: sorted (start pattern, result) pairs."""
    out = torch.zeros(2 * cap, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    st = S.lib().swiglu_probe_fp8_transitions(kind, first, last, out.data_ptr(), cap, cnt.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    n = int(cnt.item())
    assert 0 < n <= cap
    pairs = out[:2 * n].cpu().numpy().view(np.uint32).reshape(n, 2)
    return pairs[np.argsort(pairs[:, 0])]


def _check_runs(runs, last, oracle_fn, what, canon=lambda c: c):
    """Each run [a, b] of constant device result c: the oracle at a and at b
    must be c (both through `canon`).  Over patterns of one sign the fp32
    value is monotone in the pattern and the oracle is a monotone step
    function of the value (nearest rounding on a sorted lattice, the overflow
    and NaN class above it; the smallest sufficient power of two for the
    scale), so equal ends mean the oracle is c on the whole run: every
    pattern of the range is compared."""
    starts = runs[:, 0].astype(np.int64)
    ends = np.append(starts[1:] - 1, last)
    codes = canon(runs[:, 1])
    for pts in (starts, ends):
        vals = pts.astype(np.uint32).view(np.float32)
        want = canon(oracle_fn(vals))
        bad = np.nonzero(want != codes)[0]
        assert bad.size == 0, (f"{what}: device {codes[bad[:4]]} vs oracle {want[bad[:4]]} at patterns "
                               f"{[hex(int(v)) for v in pts[bad[:4]]]}")


def test_e4m3_encoder_on_all_fp32_patterns():
    """The device E4M3 encoding (v_cvt_pk_fp8_f32 at scale 1, the path of every
    quantiser here) against the oracle's encoder on all 2^32 fp32 patterns:
    the device scans them in order and returns its runs of constant code, and
    the oracle is checked at both ends of every run.  Codes are compared
    exactly except that NaN is compared as a class: E4M3FN has two NaN codes
    (S.1111.111), any of which is a correct NaN (the oracle keeps the input's
    sign; the device writes 0xFF for some inputs of either sign, e.g. every
    positive NaN pattern, and 0x7F for others, as this test records).  Within one sign's range the oracle's raw codes are monotone,
    so equal classes at a run's ends still mean equal raw codes."""
    def oracle_codes(v):
        return oracle.e4m3_encode(v.astype(np.float64)).astype(np.uint32)

    def nan_class(c):
        c = np.asarray(c, np.uint32)
        return np.where((c & 0x7F) == 0x7F, np.uint32(0x7F), c)
    nan_codes = set()
    for first, last in ((0x00000000, 0x7FFFFFFF), (0x80000000, 0xFFFFFFFF)):
        runs = _device_runs(0, first, last)
        _check_runs(runs, last, oracle_codes, f"e4m3 patterns {first:#x}..{last:#x}", nan_class)
        nan_codes |= {int(c) for c in runs[:, 1] if (c & 0x7F) == 0x7F}
        log(f"e4m3 {first:#x}..{last:#x}: {len(runs)} runs, all equal to the oracle")
    log(f"device NaN codes: {sorted(hex(c) for c in nan_codes)}")


def test_ue8m0_scale_on_all_amax_patterns():
    """The device UE8M0 byte of a block amax (block_exponent) against the
    oracle's ue8m0_byte(ue8m0_exponent(amax)) on every non-negative fp32
    pattern up to +inf (amax ignores NaN, so it is never NaN)."""
    def oracle_bytes(v):
        return oracle.ue8m0_byte(oracle.ue8m0_exponent(v.astype(np.float64))).astype(np.uint32)
    runs = _device_runs(1, 0x00000000, 0x7F800000)
    _check_runs(runs, 0x7F800000, oracle_bytes, "ue8m0 amax patterns")
    log(f"ue8m0: {len(runs)} runs, all equal to the oracle")


def test_probe_read2_runs():
    a = torch.ones(1 << 20, dtype=torch.int32, device=DEV)
    b = torch.ones(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.zeros(4096, dtype=torch.int32, device=DEV)
    S.probe_read2(a, b, sink)
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(256, 1, 65535), (256, 8, 4096), (512, 1, 16384), (512, 2, 64), (512, 8, 1)])
def test_probe_read2_shapes_run(shape):
    """Every launch shape of the configurable read, on buffers that leave a
    grid-stride tail (1 MiB + 48 bytes); the sink stays untouched (no lane's
    fold of these words equals the marker)."""
    a = torch.ones((1 << 18) + 12, dtype=torch.int32, device=DEV)
    b = torch.full(((1 << 18) + 12,), 3, dtype=torch.int32, device=DEV)
    sink = torch.zeros(4096, dtype=torch.int32, device=DEV)
    S.probe_read2(a, b, sink, shape=shape)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


# ---------------------------------------------------------- act_bwd (next f1)

ULP32 = 2.0 ** -24
TINY32 = 2.0 ** -149


def bf16_rne_f64(r):
    """Round float64 values to bf16 (nearest, ties to even) and return
    (rounded, spacing at that value): 8 significant bits, subnormal spacing
    2^-133 below 2^-126."""
    a = np.abs(r)
    _, e = np.frexp(np.where(np.isfinite(a), a, 1.0))
    sp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.copysign(np.rint(a / sp) * sp, r), sp


def check_act_bwd(d, L, use_w, what):
    """fp32 or bf16 (d["gate"] holds bf16 bits) elementwise backward."""
    g, u, dy = d["gate"], d["up"], d["dy"]
    bf = g.dtype == np.uint16
    w = d["weights"] if use_w else None
    dev = dev_bf16 if bf else dev_f32
    tdt = torch.bfloat16 if bf else torch.float32
    R, C = g.shape
    gs = [guarded((R, C), tdt), guarded((R, C), tdt), guarded((R,), torch.float32)]
    gs2 = [guarded((R, C), tdt), guarded((R, C), tdt)]
    dg, du, wg = S.act_bwd(dev(g), dev(u), dev(dy), L, weights=None if w is None else dev_f32(w),
                           out=tuple(x.t for x in gs))
    # Without weight_grad the kernel walks the array flat instead of by rows;
    # every element goes through the same arithmetic, so the bits agree.
    dg2, du2, wg2 = S.act_bwd(dev(g), dev(u), dev(dy), L, weights=None if w is None else dev_f32(w),
                              out=(gs2[0].t, gs2[1].t, None))
    torch.cuda.synchronize()
    check_guards(what, *gs, *gs2)
    assert wg2 is None
    ibits = torch.int16 if bf else torch.int32
    assert torch.equal(dg2.view(ibits), dg.view(ibits)) and torch.equal(du2.view(ibits), du.view(ibits)), \
        f"{what}: flat mapping differs from the row mapping"
    assert dg.dtype == (torch.bfloat16 if bf else torch.float32)
    dg, du = dg.float().cpu().numpy().astype(np.float64), du.float().cpu().numpy().astype(np.float64)
    wg = wg.cpu().numpy().astype(np.float64)
    g, u, dy = f64_of(g), f64_of(u), f64_of(dy)
    rg, ru, rw = oracle.act_bwd(g, u, dy, L, None if w is None else w.astype(np.float64))
    # Term magnitudes the device error is bounded by (8 ulps of each, plus
    # the final rounding): |w dy u'| s (1 + |g'| (1 - s)) for dg, |w dy g' s| for du.
    gc = oracle.clamp_nan_preserving(g.astype(np.float64), L)
    uc = oracle.clamp_nan_preserving(u.astype(np.float64), L)
    wv = np.ones(g.shape[0]) if w is None else w.astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        s = oracle.sigmoid(gc)
        tg = np.abs(wv[:, None] * dy) * np.abs(uc) * s * (1.0 + np.abs(gc) * (1.0 - s))
        tu = np.abs(wv[:, None] * dy * gc * s)
        tw = np.sum(np.abs(dy * gc * s * uc), axis=1)
    for name, y, r, t in (("dgate", dg, rg, tg), ("dup", du, ru, tu), ("weight_grad", wg, rw, tw)):
        nan_y, nan_r = np.isnan(y), np.isnan(r)
        assert np.array_equal(nan_y, nan_r), f"{what} {name}: NaN pattern differs ({np.count_nonzero(nan_y != nan_r)})"
        inf_r = np.isinf(r)
        assert np.array_equal(y[inf_r], r[inf_r]) and not np.any(np.isinf(y[~inf_r & ~nan_r])), f"{what} {name}: inf"
        fin = ~nan_r & ~inf_r
        if not fin.any():
            continue
        with np.errstate(invalid="ignore"):
            # A term that is NaN (e.g. a NaN up value beside a clamped gate,
            # whose gradient is exactly 0 on both sides) bounds nothing.
            arith = np.nan_to_num(8 * ULP32 * t[fin], nan=np.inf) + TINY32
        out_u = BF16_HALF_ULP if (bf and name != "weight_grad") else ULP32
        bound = arith + out_u * np.abs(r[fin]) + (2.0 ** -133 if bf else 0.0)
        ratio = np.where(y[fin] == r[fin], 0.0, np.abs(y[fin] - r[fin]) / bound)
        assert ratio.max() <= 1.0, f"{what} {name}: worst error {ratio.max():.3f} of the bound"
        msg = f"{what} {name}: worst error {ratio.max():.4f} of the bound"
        if bf and name != "weight_grad":
            # One rounding: wherever the fp64 value is farther from a bf16
            # rounding midpoint than the arithmetic error, the output is the
            # round-to-nearest-even of the exact value.
            q, sp = bf16_rne_f64(r[fin])
            frac = np.abs(r[fin]) / sp
            to_mid = np.abs(frac - np.floor(frac) - 0.5) * sp
            safe = to_mid > arith
            assert np.array_equal(y[fin][safe], q[safe]), f"{what} {name}: not the single rounding of the exact value"
            msg += f", RNE-exact on {int(safe.sum())} of {safe.size}"
        log(msg)
    # Clamped positions carry exactly zero gradient.
    if np.isfinite(L):
        assert np.all(dg[np.abs(g) > L] == 0.0) and np.all(du[np.abs(u) > L] == 0.0)


@pytest.mark.parametrize("L,use_w", [(math.inf, True), (0.5, False), (7.0, True)])
def test_act_bwd_full_4001x3584(L, use_w):
    d = synth.act_bwd_f32(4001, 3584, seed=0)
    check_act_bwd(d, L, use_w, f"act_bwd 4001x3584 L={L} weights={use_w}")


@pytest.mark.parametrize("shape", [(1, 4), (3, 12), (7, 2052), (65, 260), (5, 0)])
def test_act_bwd_ragged_and_specials(shape):
    rows, cols = shape
    d = synth.act_bwd_f32(rows, cols, seed=3, specials=True)
    for L in (math.inf, 1.5):
        check_act_bwd(d, L, True, f"act_bwd {shape} L={L} specials")


@pytest.mark.parametrize("L,use_w", [(math.inf, True), (0.5, False)])
def test_act_bwd_bf16_full_4001x3584(L, use_w):
    d = synth.act_bwd_bf16(4001, 3584, seed=0)
    check_act_bwd(d, L, use_w, f"act_bwd bf16 4001x3584 L={L} weights={use_w}")


@pytest.mark.parametrize("shape", [(1, 8), (3, 24), (7, 2056), (65, 264), (5, 0)])
def test_act_bwd_bf16_ragged_and_specials(shape):
    rows, cols = shape
    d = synth.act_bwd_bf16(rows, cols, seed=3, specials=True)
    for L in (math.inf, 1.5):
        check_act_bwd(d, L, True, f"act_bwd bf16 {shape} L={L} specials")


# ------------------------------------- act_bwd with E4M3 outputs (next f1)

def check_act_bwd_fp8(d, L, use_w, what):
    """dgate and dup as 1x32 E4M3 blocks.

    1. same precision: the fp32-output backward on the same values (bf16
       inputs widened exactly) gives the once-rounded fp32 dgate and dup the
       quantiser works on; the oracle's 1x32 quantiser applied to them must
       give the device's scale bytes and codes bit for bit, and weight_grad
       must equal the fp32 path's bit for bit;
    2. from the inputs: against the oracle's E4M3 backward, scales bit-exact
       except blocks whose exact amax lies within the fp32 path's 8-ulp bound
       of a scale boundary 1.75 * 2^k, codes within 1 ulp elsewhere, NaN codes
       exactly where the oracle has them."""
    g, u, dy = d["gate"], d["up"], d["dy"]
    bf = g.dtype == np.uint16
    R, C = g.shape
    dev = dev_bf16 if bf else dev_f32
    w = d["weights"] if use_w else None
    gs = [guarded((R, C), torch.uint8), guarded((R, C // 32), torch.uint8), guarded((R, C), torch.uint8),
          guarded((R, C // 32), torch.uint8), guarded((R,), torch.float32)]
    S.act_bwd_fp8(dev(g), dev(u), dev(dy), L, weights=None if w is None else dev_f32(w),
                  out=(gs[0].t, gs[1].t, gs[2].t, gs[3].t, gs[4].t if use_w else None))
    # the flat mapping (no weight_grad) must give the same bytes
    gs2 = [guarded((R, C), torch.uint8), guarded((R, C // 32), torch.uint8), guarded((R, C), torch.uint8),
           guarded((R, C // 32), torch.uint8)]
    S.act_bwd_fp8(dev(g), dev(u), dev(dy), L, weights=None if w is None else dev_f32(w),
                  out=(gs2[0].t, gs2[1].t, gs2[2].t, gs2[3].t, None))
    f32 = {k: f64_of(d[k]).astype(np.float32) for k in ("gate", "up", "dy")}
    dg32, du32, wg32 = S.act_bwd(dev_f32(f32["gate"]), dev_f32(f32["up"]), dev_f32(f32["dy"]), L,
                                 weights=None if w is None else dev_f32(w), weight_grad=True)
    torch.cuda.synchronize()
    check_guards(what, *gs, *gs2)
    qg, sg, qu, su = (x.t.cpu().numpy() for x in gs[:4])
    for a, b in zip(gs[:4], gs2):
        assert torch.equal(a.t, b.t), f"{what}: the row and flat mappings differ"
    # 1. same precision
    for name, q, sc, v in (("dgate", qg, sg, dg32), ("dup", qu, su, du32)):
        oq, os_ = oracle.quantize_1x32(v.cpu().numpy())
        assert np.array_equal(sc, os_), f"{what} {name}: scales differ from quantise(fp32 backward)"
        nq = (oq & 0x7F) == 0x7F
        assert np.array_equal((q & 0x7F) == 0x7F, nq), f"{what} {name}: NaN codes differ"
        assert np.array_equal(q[~nq], oq[~nq]), f"{what} {name}: codes differ from quantise(fp32 backward)"
    if use_w:
        assert torch.equal(gs[4].t.view(torch.int32), wg32.view(torch.int32)), f"{what}: weight_grad differs"
    # 2. from the inputs
    g64, u64, dy64 = (f64_of(d[k]) for k in ("gate", "up", "dy"))
    w64 = None if w is None else w.astype(np.float64)
    rqg, rsg, rqu, rsu, _ = oracle.act_bwd_fp8(g64, u64, dy64, L, w64)
    rdg, rdu, _ = oracle.act_bwd(g64, u64, dy64, L, w64)
    for name, q, sc, rq, rs, rv in (("dgate", qg, sg, rqg, rsg, rdg), ("dup", qu, su, rqu, rsu, rdu)):
        nan = (rq & 0x7F) == 0x7F
        assert np.array_equal((q & 0x7F) == 0x7F, nan), f"{what} {name}: NaN positions differ from the oracle"
        diff = sc != rs
        if diff.any():
            blocks = rv.astype(np.float32).astype(np.float64).reshape(R, C // 32, 32)
            amax = np.where(np.isnan(blocks), 0, np.abs(blocks)).max(axis=2)[diff]
            _, ex = np.frexp(amax)
            bnd = 1.75 * np.exp2(ex - 1.0)
            near = np.abs(amax - bnd) <= H_ULP_MAX * np.spacing(bnd.astype(np.float32)).astype(np.float64)
            assert near.all(), f"{what} {name}: {int((~near).sum())} scale bytes differ away from a boundary"
        same = np.repeat(~diff, 32, axis=1) & ~nan
        dist = np.abs(oracle.e4m3_ordinal(q[same]) - oracle.e4m3_ordinal(rq[same]))
        assert dist.max(initial=0) <= 1, f"{what} {name}: a code is {dist.max()} ulps from the oracle's"
        log(f"{what} {name}: scale diffs {int(diff.sum())}, codes off by 1: {int((dist == 1).sum())} of {dist.size}")


@pytest.mark.parametrize("bf", [True, False])
@pytest.mark.parametrize("L,use_w", [(0.5, False), (math.inf, True), (7.0, True)])
def test_act_bwd_fp8_full_4001x3584(bf, L, use_w):
    d = (synth.act_bwd_bf16 if bf else synth.act_bwd_f32)(4001, 3584, seed=0)
    check_act_bwd_fp8(d, L, use_w, f"act_bwd_fp8 {'bf16' if bf else 'f32'} L={L} w={use_w}")


@pytest.mark.parametrize("bf", [True, False])
@pytest.mark.parametrize("shape", [(1, 32), (3, 384), (7, 2048), (65, 96)])
def test_act_bwd_fp8_ragged_and_specials(bf, shape):
    d = (synth.act_bwd_bf16 if bf else synth.act_bwd_f32)(*shape, seed=13, specials=True)
    for L, use_w in ((math.inf, True), (1.5, False)):
        check_act_bwd_fp8(d, L, use_w, f"act_bwd_fp8 {shape} {'bf16' if bf else 'f32'} L={L} specials")


def _load_bwd_fp8_cases():
    with open(os.path.join(GOLDEN, "act_bwd_fp8_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_bwd_fp8_cases(), ids=lambda c: c["name"])
def test_act_bwd_fp8_hand_cases_on_device(case):
    """The hand-derived cases of tests/golden/act_bwd_fp8_cases.json, fp32
    inputs, on the device: scales and codes as derived by hand."""
    rows, cols = case["rows"], case["cols"]

    def fill(spec):
        a = np.full(rows * cols, _hexf(spec["fill"]), dtype=np.float64)
        for k, v in spec.get("set", {}).items():
            a[int(k)] = _hexf(v)
        return a.astype(np.float32).reshape(rows, cols)
    g, u, dy = fill(case["gate"]), fill(case["up"]), fill(case["dy"])
    w = None if case["weights"] is None else dev_f32(np.array([_hexf(v) for v in case["weights"]], np.float32))
    qg, sg, qu, su, wg = S.act_bwd_fp8(dev_f32(g), dev_f32(u), dev_f32(dy), _hexf(case["clamp"]), weights=w,
                                       weight_grad=True)
    torch.cuda.synchronize()
    assert np.array_equal(sg.cpu().numpy(), np.array(case["expect_dgate_scale"], dtype=np.uint8))
    assert np.array_equal(su.cpu().numpy(), np.array(case["expect_dup_scale"], dtype=np.uint8))
    for q, exp in ((qg, case["expect_dgate_codes"]), (qu, case["expect_dup_codes"])):
        for i, c in enumerate(q.cpu().numpy().reshape(-1)):
            want = exp.get(str(i), exp["default"])
            if want == "nan":
                assert (c & 0x7F) == 0x7F, (case["name"], i, hex(c))
            else:
                assert c == want, (case["name"], i, hex(c), want)
    want = np.array([_hexf(v) for v in case["expect_weight_grad"]])
    got = wg.cpu().numpy().astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.allclose(got[~nan], want[~nan], rtol=2 ** -22, atol=0)


def test_act_bwd_without_weight_grad_and_empty():
    d = synth.act_bwd_f32(8, 64, seed=4)
    dg, du, wg = S.act_bwd(dev_f32(d["gate"]), dev_f32(d["up"]), dev_f32(d["dy"]), 7.0)
    torch.cuda.synchronize()
    assert wg is None
    rg, ru, _ = oracle.act_bwd(d["gate"].astype(np.float64), d["up"].astype(np.float64),
                               d["dy"].astype(np.float64), 7.0)
    # (elementwise error bounds are checked in check_act_bwd; here the
    # normwise error shows the outputs are right without a weight_grad)
    assert oracle.normwise_rel_err(dg.cpu().numpy(), rg) < 1e-6
    assert oracle.normwise_rel_err(du.cpu().numpy(), ru) < 1e-6
    e = torch.empty((0, 16), dtype=torch.float32, device=DEV)
    dg, du, wg = S.act_bwd(e, e, e, math.inf, weight_grad=True)
    torch.cuda.synchronize()
    assert dg.shape == (0, 16) and wg.shape == (0,)


# ------------------------------------------------------ GeGLU (next f2)

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 520, 264), (1, 1, 8), (129, 127, 72)])
def test_geglu_fwd_ragged(dt, shape):
    M, N, K = shape
    d = synth.train_bf16(M, N, K, seed=6, with_dh=False) if dt == "bf16" else synth.gemm_fp32(M, N, K, seed=6)
    check_fwd(d, dt, what=f"geglu fwd {dt} {shape}", act="gelu_tanh")


def test_geglu_fwd_fp32_full_4001x3584x2048():
    d = synth.gemm_fp32(4001, 3584, 2048, seed=0)
    check_fwd(d, "f32", what="geglu fwd fp32 4001x3584x2048", act="gelu_tanh")


def test_geglu_fwd_bf16_full_8192x14336x4096_sampled():
    M, N, K = 8192, 14336, 4096
    d = synth.train_bf16(M, N, K, seed=0, with_dh=False)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(2).integers(0, M, 62)]))
    check_fwd(d, "bf16", rows=rows, what="geglu fwd bf16 8192x14336x4096 (sampled rows)", act="gelu_tanh")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("L", [math.inf, 7.0])
def test_geglu_act_quant_full_4001x3584(L):
    d = synth.act_quant_f32(4001, 3584, seed=0)
    check_act_quant(d["gate"], d["up"], L, f"geglu act_quant 4001x3584 L={L}", act="gelu_tanh")


@pytest.mark.parametrize("shape", [(1, 32), (3, 384), (7, 2048)])
def test_geglu_act_quant_ragged(shape):
    d = synth.act_quant_f32(*shape, seed=6)
    check_act_quant(d["gate"], d["up"], 7.0, f"geglu act_quant {shape}", act="gelu_tanh")


def test_geglu_act_quant_tails_subnormal_and_huge():
    """The GELU tail (sigma of t ~ -100: the argument's rounding would cost
    hundreds of ulps in fp32), subnormal gates with huge up, tiny products."""
    rs = np.random.default_rng(10)
    rows, cols = 64, 256
    gate = rs.uniform(-13.0, 13.0, (rows, cols)).astype(np.float32)
    up = (rs.standard_normal((rows, cols)) * np.exp2(rs.integers(0, 120, (rows, cols)))).astype(np.float32)
    check_act_quant(gate, up, math.inf, "geglu act_quant tail", act="gelu_tanh")
    mant = rs.integers(1, 1 << 23, rows * cols, dtype=np.uint32)
    sub = (mant | (rs.integers(0, 2, rows * cols, dtype=np.uint32) << 31)).view(np.float32).reshape(rows, cols)
    big = (rs.standard_normal((rows, cols)) * np.exp2(rs.integers(-20, 100, (rows, cols)))).astype(np.float32)
    check_act_quant(sub.copy(), big, math.inf, "geglu act_quant subnormal gate, huge up", act="gelu_tanh")
    g2 = rs.uniform(-30, 30, (rows, cols)).astype(np.float32)
    u2 = rs.uniform(-1e-30, 1e-30, (rows, cols)).astype(np.float32)
    check_act_quant(g2, u2, math.inf, "geglu act_quant tiny products", act="gelu_tanh")


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("NK", [(6912, 1536), (257, 520)])
def test_geglu_gemv(M, NK):
    N, K = NK
    d = synth.decode_bf16(M, N, K, seed=7)
    check_fwd(d, "bf16", what=f"geglu gemv M={M} N={N} K={K}", via="gemv", act="gelu_tanh")


# ---------------------------------------- FP8-output forward (next f4)

def check_fwd_fp8(d, rows=None, act="silu", what="fwd_fp8"):
    """q, scale from the fused epilogue against the oracle.

    1. h (fp32, returned beside q) is within the forward's bound of the exact
       act(g) u;
    2. same precision: the oracle's 1x32 quantiser applied to that h gives
       exactly the device's scale bytes and codes;
    3. from the inputs: each scale byte lies between the UE8M0 bytes of the
       smallest and largest block amax that h's bound allows, and each code,
       at the device's scale, between the codes of h - bound and h + bound
       (encoding is monotone in the value, so this is the whole set of codes
       that some h within the bound would produce).
    """
    t = to_dev(d)
    f = to_f64(d)
    M, N = t["x"].shape[0], t["wg"].shape[0]
    gs = [guarded((M, N), torch.uint8), guarded((M, N // 32), torch.uint8), guarded((M, N), torch.float32)]
    gs2 = [guarded((M, N), torch.uint8), guarded((M, N // 32), torch.uint8)]
    q, sc, h = S.fwd_fp8(t["x"], t["wg"], t["wu"], act=act, out=tuple(g.t for g in gs))
    q2, sc2, none = S.fwd_fp8(t["x"], t["wg"], t["wu"], act=act, out=(gs2[0].t, gs2[1].t, None))
    torch.cuda.synchronize()
    check_guards(what, *gs, *gs2)
    assert none is None
    assert torch.equal(q, q2) and torch.equal(sc, sc2), f"{what}: output differs without h_out"
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=DEV)
    q, sc, h = q[sel].cpu().numpy(), sc[sel].cpu().numpy(), h[sel].cpu().numpy()
    ref, bound = fwd_bound(f["x"], f["wg"], f["wu"], "f32", rows, act)
    e, c = assert_gates(h.astype(np.float64), ref, "f32", what)
    ratio = assert_within(h.astype(np.float64), ref, bound, what + " h")
    # 2. same precision
    oq, os_ = oracle.quantize_1x32(h)
    assert np.array_equal(sc, os_), f"{what}: scales differ from oracle(quantise(device h))"
    assert np.array_equal(q, oq), f"{what}: codes differ from oracle(quantise(device h))"
    # 3. from the inputs
    R, N = ref.shape
    lo_mag = np.maximum(np.abs(ref) - bound, 0.0).reshape(R, N // 32, 32).max(axis=2)
    hi_mag = (np.abs(ref) + bound).reshape(R, N // 32, 32).max(axis=2)
    E_lo, E_hi = oracle.ue8m0_exponent(lo_mag), oracle.ue8m0_exponent(hi_mag)
    E = sc.astype(np.int64) - 127
    assert np.all((E_lo <= E) & (E <= E_hi)), f"{what}: a scale byte no h within the bound gives"
    Ee = np.repeat(E, 32, axis=1)
    o_lo = oracle.e4m3_ordinal(oracle.e4m3_encode(np.ldexp(ref - bound, -Ee)))
    o_hi = oracle.e4m3_ordinal(oracle.e4m3_encode(np.ldexp(ref + bound, -Ee)))
    o = oracle.e4m3_ordinal(q)
    bad = (o < o_lo) | (o > o_hi)
    assert not bad.any(), f"{what}: {int(bad.sum())} codes outside the bound's interval"
    exact_q, exact_s = oracle.quantize_1x32(ref.astype(np.float32))
    log(f"{what}: h normwise {e:.3e} cosine {c:.7f} bound-ratio {ratio:.3f}; vs exact h: "
        f"scale diffs {int((sc != exact_s).sum())}, code diffs {int((q != exact_q).sum())} of {q.size}")


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("shape", [(300, 544, 264), (1, 32, 8), (129, 96, 72), (37, 1056, 1032)])
def test_fwd_fp8_ragged(act, shape):
    M, N, K = shape
    d = synth.train_bf16(M, N, K, seed=8, with_dh=False)
    check_fwd_fp8(d, act=act, what=f"fwd_fp8 {act} {shape}")


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_fwd_fp8_full_8192x14336x4096_sampled(act):
    M, N, K = 8192, 14336, 4096
    d = synth.train_bf16(M, N, K, seed=0, with_dh=False)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(4).integers(0, M, 30)]))
    check_fwd_fp8(d, rows=rows, act=act, what=f"fwd_fp8 {act} 8192x14336x4096 (sampled rows)")
    torch.cuda.empty_cache()


def test_fwd_fp8_k_zero_and_empty():
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((64, 0), dtype=torch.bfloat16, device=DEV)
    q = torch.full((5, 64), 0x55, dtype=torch.uint8, device=DEV)
    s = torch.full((5, 2), 0x55, dtype=torch.uint8, device=DEV)
    h = torch.full((5, 64), 3.0, dtype=torch.float32, device=DEV)
    S.fwd_fp8(x, w, w, out=(q, s, h))
    torch.cuda.synchronize()
    assert torch.count_nonzero(q).item() == 0          # E4M3 +0
    assert torch.count_nonzero(s).item() == 0          # amax 0 -> E = -127 -> byte 0
    assert torch.count_nonzero(h).item() == 0
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((64, 64), dtype=torch.bfloat16, device=DEV)
    qq, ss, hh = S.fwd_fp8(e, w, w, h_out=True)
    torch.cuda.synchronize()
    assert qq.shape == (0, 64) and ss.shape == (0, 2) and hh.shape == (0, 64)



# ----------------------------------------------------- multipliers (next f3)

MULTS = [(0.7, 1.3), (-2.5, 0.125)]


@pytest.mark.parametrize("shape", [(300, 520, 264), (129, 300, 72)])   # N % 8 != 0: scalar-store epilogue
@pytest.mark.parametrize("mult", MULTS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_mult_fwd_ragged(shape, mult, dt, act):
    M, N, K = shape
    d = synth.train_bf16(M, N, K, seed=11, with_dh=False) if dt == "bf16" else synth.gemm_fp32(M, N, K, seed=11)
    check_fwd(d, dt, what=f"fwd {act} {dt} {shape} mult={mult}", act=act, mult=mult)


def test_mult_one_is_exactly_the_plain_forward_and_backward():
    d = synth.train_bf16(260, 384, 136, seed=12)
    t = to_dev(d)
    h0 = S.fwd(t["x"], t["wg"], t["wu"])
    h1 = S.fwd(t["x"], t["wg"], t["wu"], gate_mult=1.0, up_mult=1.0)
    b0 = S.bwd(t["x"], t["wg"], t["wu"], t["dh"])
    b1 = S.bwd(t["x"], t["wg"], t["wu"], t["dh"], gate_mult=1.0, up_mult=1.0)
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    for a, b in zip(b0, b1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mult_fwd_bf16_full_8192x14336x4096_sampled():
    M, N, K = 8192, 14336, 4096
    d = synth.train_bf16(M, N, K, seed=0, with_dh=False)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).integers(0, M, 30)]))
    check_fwd(d, "bf16", rows=rows, what="fwd bf16 8192x14336x4096 mult=(0.7, 1.3) (sampled rows)",
              mult=(0.7, 1.3))
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mult", MULTS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_mult_bwd_ragged(mult, dt):
    M, N, K = 257, 640, 520
    if dt == "bf16":
        d = synth.train_bf16(M, N, K, seed=13)
    else:
        d = synth.gemm_fp32(M, N, K, seed=13)
        d["dh"] = synth.normal_f32((M, N), 1.0, 13, synth.STREAM_DH)
    check_bwd(d, dt, what=f"bwd {dt} mult={mult}", mult=mult)


def test_mult_bwd_bf16_full_8192x14336x4096_sampled():
    M, N, K = 8192, 14336, 4096
    d = synth.train_bf16(M, N, K, seed=0)
    rs = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, M - 1], rs.integers(0, M, 20)]))
    cols = np.unique(np.concatenate([[0, N - 1], rs.integers(0, N, 20)]))
    check_bwd(d, "bf16", rows=rows, cols=cols, what="bwd bf16 8192x14336x4096 mult=(-2.5, 0.125) (sampled)",
              mult=(-2.5, 0.125))
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 8])
def test_mult_gemv(M):
    d = synth.decode_bf16(M, 6912, 1536, seed=14)
    for act in ("silu", "gelu_tanh"):
        check_fwd(d, "bf16", what=f"gemv {act} M={M} mult=(0.7, 1.3)", via="gemv", act=act, mult=(0.7, 1.3))


def test_mult_autograd():
    d = synth.train_bf16(24, 48, 64, seed=15)
    t = to_dev(d)
    x = t["x"].clone().requires_grad_(True)
    wg = t["wg"].clone().requires_grad_(True)
    wu = t["wu"].clone().requires_grad_(True)
    h = S.swiglu(x, wg, wu, 0.7, 1.3)
    h.backward(t["dh"])
    dx, dwg, dwu = S.bwd(t["x"], t["wg"], t["wu"], t["dh"], gate_mult=0.7, up_mult=1.3)
    torch.cuda.synchronize()
    assert torch.equal(x.grad.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(wg.grad.view(torch.int16), dwg.view(torch.int16))
    assert torch.equal(wu.grad.view(torch.int16), dwu.view(torch.int16))


# ------------------------------------------------------- GeGLU backward

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 520, 264), (33, 17, 40), (257, 640, 520)])
def test_geglu_bwd_ragged(dt, shape):
    M, N, K = shape
    if dt == "bf16":
        d = synth.train_bf16(M, N, K, seed=16)
    else:
        d = synth.gemm_fp32(M, N, K, seed=16)
        d["dh"] = synth.normal_f32((M, N), 1.0, 16, synth.STREAM_DH)
    check_bwd(d, dt, what=f"geglu bwd {dt} {shape}", act="gelu_tanh")
    check_bwd(d, dt, what=f"geglu bwd {dt} {shape} mult=(0.7, 1.3)", act="gelu_tanh", mult=(0.7, 1.3))


def test_geglu_bwd_bf16_full_8192x14336x4096_sampled():
    M, N, K = 8192, 14336, 4096
    d = synth.train_bf16(M, N, K, seed=0)
    rs = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, M - 1], rs.integers(0, M, 20)]))
    cols = np.unique(np.concatenate([[0, N - 1], rs.integers(0, N, 20)]))
    check_bwd(d, "bf16", rows=rows, cols=cols, what="geglu bwd bf16 8192x14336x4096 (sampled)", act="gelu_tanh")
    torch.cuda.empty_cache()


def test_geglu_autograd():
    d = synth.train_bf16(24, 48, 64, seed=17)
    t = to_dev(d)
    x = t["x"].clone().requires_grad_(True)
    wg = t["wg"].clone().requires_grad_(True)
    wu = t["wu"].clone().requires_grad_(True)
    h = S.swiglu(x, wg, wu, act="gelu_tanh")
    h.backward(t["dh"])
    dx, dwg, dwu = S.bwd(t["x"], t["wg"], t["wu"], t["dh"], act="gelu_tanh")
    torch.cuda.synchronize()
    assert torch.equal(x.grad.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(wg.grad.view(torch.int16), dwg.view(torch.int16))
    assert torch.equal(wu.grad.view(torch.int16), dwu.view(torch.int16))


# ------------------------------------------ non-quantised elementwise forward

def check_act_fwd(gate, up, L, act, out_dtype, what):
    gs = [guarded(gate.shape, out_dtype), guarded((1,), torch.int64)]
    h, cnt = S.act_fwd(dev_f32(gate), dev_f32(up), L, act=act, out=(gs[0].t, gs[1].t))
    torch.cuda.synchronize()
    check_guards(what, *gs)
    y = h.float().cpu().numpy().astype(np.float64)
    r, rc = oracle.act_fwd(gate.astype(np.float64), up.astype(np.float64), L, act)
    assert int(cnt.item()) == rc, f"{what}: clamp count {int(cnt.item())} != {rc}"
    bf = out_dtype == torch.bfloat16
    # The reference is the exact h rounded to the output type; NaN and
    # infinities (also from overflow of the rounding) must match.
    rr = bf16_rne_f64(r)[0] if bf else r.astype(np.float32).astype(np.float64)
    nan = np.isnan(rr)
    assert np.array_equal(np.isnan(y), nan), f"{what}: NaN pattern"
    inf = np.isinf(rr)
    assert np.array_equal(y[inf], rr[inf]) and not np.isinf(y[~inf & ~nan]).any(), f"{what}: inf pattern"
    fin = ~nan & ~inf
    if bf:
        # One rounding: equal to RNE(exact) wherever the exact value is
        # farther from a bf16 midpoint than the arithmetic error (8 fp32 ulps).
        q, sp = bf16_rne_f64(r[fin])
        frac = np.abs(r[fin]) / sp
        to_mid = np.abs(frac - np.floor(frac) - 0.5) * sp
        safe = to_mid > 8 * ULP32 * np.abs(r[fin]) + TINY32
        assert np.array_equal(y[fin][safe], q[safe]), f"{what}: not the single rounding of the exact value"
        assert np.all(np.abs(y[fin] - r[fin]) <= sp * (1 + 1e-9)), f"{what}: off by more than one bf16 step"
        log(f"{what}: count {rc}, RNE-exact on {int(safe.sum())} of {safe.size}")
    else:
        ulp = f32_ulp_distance(y[fin], rr[fin])
        assert ulp.max(initial=0) <= H_ULP_MAX, f"{what}: h off by {ulp.max()} ulps"
        log(f"{what}: count {rc}, max ulp {ulp.max(initial=0)}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("L", [math.inf, 7.0])
def test_act_fwd_full_4001x3584(out_dtype, act, L):
    d = synth.act_quant_f32(4001, 3584, seed=0)
    check_act_fwd(d["gate"], d["up"], L, act, out_dtype, f"act_fwd {act} {out_dtype} L={L}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 8), (3, 384), (7, 2056), (0, 64)])
def test_act_fwd_ragged_and_tails(out_dtype, shape):
    d = synth.act_quant_f32(*shape, seed=9)
    for act in ("silu", "gelu_tanh"):
        check_act_fwd(d["gate"], d["up"], 1.5, act, out_dtype, f"act_fwd {act} {shape} {out_dtype}")
    rs = np.random.default_rng(11)
    g = rs.uniform(-13.0, 13.0, (64, 256)).astype(np.float32)
    u = (rs.standard_normal((64, 256)) * np.exp2(rs.integers(-30, 120, (64, 256)))).astype(np.float32)
    for act in ("silu", "gelu_tanh"):
        check_act_fwd(g, u, math.inf, act, out_dtype, f"act_fwd {act} tails {out_dtype}")


def test_act_fwd_count_reset_without_clamp():
    d = synth.act_quant_f32(4, 64, seed=1)
    cnt = torch.full((1,), 99, dtype=torch.int64, device=DEV)
    h = torch.empty((4, 64), dtype=torch.float32, device=DEV)
    S.act_fwd(dev_f32(d["gate"]), dev_f32(d["up"]), math.inf, out=(h, cnt))
    torch.cuda.synchronize()
    assert cnt.item() == 0


@pytest.mark.parametrize("shape", [(37, 50, 36), (5, 129, 4), (130, 33, 260)])
def test_fp32_reduction_length_not_a_multiple_of_8(shape):
    """fp32 rows are 16-byte chunks of 4 values: K % 8 == 4 leaves a half
    chunk pair in the last k-step, for the forward and every backward GEMM."""
    M, N, K = shape
    d = synth.gemm_fp32(M, N, K, seed=18)
    check_fwd(d, "f32", what=f"fwd fp32 {shape}")
    check_fwd(d, "f32", what=f"geglu fwd fp32 {shape}", act="gelu_tanh")
    d["dh"] = synth.normal_f32((M, N), 1.0, 18, synth.STREAM_DH)
    check_bwd(d, "f32", what=f"bwd fp32 {shape}")


# --------------------------------------------------------- maximum sizes

BF16_MAX_LD = (1 << 22) - 64   # largest bf16 row length the 32-bit tile offsets allow


def test_bf16_forward_and_backward_at_the_longest_reduction():
    """K at the bf16 limit: the tile byte offsets of the DMA path reach their
    largest values (forward, recompute, dX over 2N and the transposes)."""
    M, N, K = 3, 5, BF16_MAX_LD
    d = synth.train_bf16(M, N, K, seed=19)
    check_fwd(d, "bf16", what=f"fwd bf16 K={K}")
    check_bwd(d, "bf16", what=f"bwd bf16 K={K}")
    assert S.lib().swiglu_fwd(1, M, N, K + 64, 0x10000, 0x10000, 0x10000, 0x10000, None) == 7   # UNSUPPORTED
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_full_tiles_at_the_longest_reduction(dt):
    """K at the limit with M and N large enough that an operand tile's buffer
    descriptor spans its full 512 bytes x K (128 fp32 rows, 256 bf16 rows):
    its size and the largest in-range offsets sit just below 2^31, with the
    out-of-range offset 2^31 right past them.  These descriptors are the
    forward's and the backward recompute's.  x, Wg, Wu in {-1, 0, 1}: every
    partial sum of g and u is an integer of magnitude <= K < 2^24, exact in
    fp32 whatever the order, so h must be within 8 fp32 ulps of the exact
    value (fp32) or its round-to-nearest-even (bf16, away from midpoints).
    dX (both types) and dWg, dWu (fp32) are held to the gates and to an
    elementwise bound of their reductions on sampled rows and columns."""
    K = BF16_MAX_LD
    M = N = 128 if dt == "f32" else 256
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    d = synth.small_int_i8(M, N, K, seed=22)
    dh = synth.normal_f32((M, N), 1.0, 22, synth.STREAM_DH)
    if dt == "bf16":
        dh = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(dh))
    # int8 -> fp32 / bf16 on the device is exact for these values
    t = {k: torch.from_numpy(v).to(DEV).to(tdt) for k, v in d.items()}
    t["dh"] = dev_f32(dh).to(tdt)
    log(f"limit {dt}: M=N={M} K={K}, inputs ready")
    hg = guarded((M, N), tdt)
    S.fwd(t["x"], t["wg"], t["wu"], out=hg.t)
    outs = [guarded((M, K), tdt), guarded((N, K), tdt), guarded((N, K), tdt)]
    ws = guarded((S.bwd_workspace_bytes(tdt, M, N, K),), torch.uint8)
    S.bwd(t["x"], t["wg"], t["wu"], t["dh"], out=tuple(g.t for g in outs), workspace=ws.t)
    torch.cuda.synchronize()
    check_guards(f"limit {dt}", hg, *outs, ws)
    rows = np.array([0, M // 2 + 1, M - 1])
    cols = np.array([0, N // 2 + 1, N - 1])
    ri, ci = torch.as_tensor(rows, device=DEV), torch.as_tensor(cols, device=DEV)
    y, dxd = host_f64(hg.t[ri]), host_f64(outs[0].t[ri])
    dwgd, dwud = host_f64(outs[1].t[ci]), host_f64(outs[2].t[ci])
    del t, hg, outs, ws
    torch.cuda.empty_cache()
    log(f"limit {dt}: device done")
    wg, wu = d["wg"].astype(np.float64), d["wu"].astype(np.float64)
    xr, dhf = d["x"][rows].astype(np.float64), dh.astype(np.float64)
    # forward: exact g, u on the sampled rows
    g, u = oracle.gate_up(xr, wg, wu)
    r = oracle.glu_fwd(xr, wg, wu)
    tail = oracle.sigmoid(g) < 2.0 ** -126
    assert np.all(np.abs(y[tail] - r[tail]) <= 2.0 ** -126 * np.abs(g[tail] * u[tail]) + 1e-45)
    keep = ~tail
    if dt == "f32":
        ulp = f32_ulp_distance(y[keep], r[keep].astype(np.float32).astype(np.float64))
        assert ulp.max(initial=0) <= H_ULP_MAX, f"limit fp32 h off by {ulp.max()} ulps"
    else:
        q, sp = bf16_rne_f64(r[keep])
        frac = np.abs(r[keep]) / sp
        safe = np.abs(frac - np.floor(frac) - 0.5) * sp > 2e-5 * np.abs(r[keep]) + 1e-30
        assert np.array_equal(y[keep][safe], q[safe]), "limit bf16 h is not the rounding of the exact value"
    # dX rows: dg, du carry a few fp32 ulps of the activation (and the bf16
    # operand rounding); the reduction over 2N adds gamma_{2N+1}.  With
    # |x|, |W| <= 1 the sums of |dg||W| (over n) and |dg||x| (over m) are at
    # most the sums of |dg|, which keeps the bounds free of K-long arrays.
    op = BF16_HALF_ULP if dt == "bf16" else 0.0
    outu = BF16_HALF_ULP if dt == "bf16" else U32
    checks = []
    dg, du = oracle.dswiglu(g, u, dhf[rows])
    dxr = oracle.swiglu_bwd_dx_rows(xr, wg, wu, dhf[rows], np.arange(len(rows)))
    absx = (np.abs(dg).sum(axis=1) + np.abs(du).sum(axis=1))[:, None]
    checks.append(("dx", dxd, dxr, 2 * ((gamma(2 * N + 1) + op + 16 * U32) * absx + outu * np.abs(dxr)) + 1e-30))
    if dt == "f32":
        del wg, wu
        x = d["x"].astype(np.float64)
        wgc, wuc = d["wg"][cols].astype(np.float64), d["wu"][cols].astype(np.float64)
        dwgr, dwur = oracle.swiglu_bwd_dw_rows(x, wgc, wuc, dhf[:, cols], np.arange(len(cols)))
        gc, uc = oracle.gate_up(x, wgc, wuc)
        dgc, duc = oracle.dswiglu(gc, uc, dhf[:, cols])
        for name, yv, rv, dd in (("dwg", dwgd, dwgr, dgc), ("dwu", dwud, dwur, duc)):
            b = 2 * ((gamma(M + 1) + 16 * U32) * np.abs(dd).sum(axis=0)[:, None] + outu * np.abs(rv)) + 1e-30
            checks.append((name, yv, rv, b))
    for name, yv, rv, b in checks:
        e, c = assert_gates(yv, rv, dt, f"limit {dt} {name}")
        ratio = assert_within(yv, rv, b, f"limit {dt} {name}")
        log(f"limit {dt} {name}: normwise {e:.3e} cosine {c:.7f} bound-ratio {ratio:.3f}")


def test_bf16_backward_at_the_largest_token_count():
    """M at the bf16 limit of the dW reduction (x^T and [dg | du]^T rows of
    round_up(M, 8) elements)."""
    M, N, K = BF16_MAX_LD, 3, 8
    d = synth.train_bf16(M, N, K, seed=20)
    rows = np.array([0, 1, M // 2, M - 1])
    check_bwd(d, "bf16", rows=rows, what=f"bwd bf16 M={M}")
    torch.cuda.empty_cache()


# ------------------------------------- exact accumulation: integer inputs

@pytest.mark.parametrize("shape", [(300, 520, 264), (129, 127, 4096)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_forward_on_small_integers_is_exact_up_to_the_activation(shape, dt):
    """x, W in {-3..3}: g and u are exact in fp32 whatever the summation
    order, so h differs from the exact act(g) u only by the activation and
    the output rounding: fp32 within 8 ulps of the rounded exact value;
    bf16 the round-to-nearest-even of the exact value wherever it is not
    within the short sigma's error of a rounding midpoint.  Where sigma(g)
    is below the smallest normal fp32 (g < -87.3), both sigma forms lose
    relative precision (the short one flushes to 0): there |h| < 2^-126 |g u|
    and only that absolute bound is required."""
    M, N, K = shape
    d = synth.small_int_bf16(M, N, K, seed=21)
    if dt == "f32":
        d = {k: synth.bf16_bits_to_f32(v) for k, v in d.items()}
    t = to_dev(d)
    f = to_f64(d)
    h = S.fwd(t["x"], t["wg"], t["wu"])
    torch.cuda.synchronize()
    y = host_f64(h)
    r = oracle.glu_fwd(f["x"], f["wg"], f["wu"])
    g, u = oracle.gate_up(f["x"], f["wg"], f["wu"])
    tail = oracle.sigmoid(g) < 2.0 ** -126
    assert np.all(np.abs(y[tail] - r[tail]) <= 2.0 ** -126 * np.abs(g[tail] * u[tail]) + 1e-45)
    keep = ~tail
    if dt == "f32":
        ulp = f32_ulp_distance(y[keep], r[keep].astype(np.float32).astype(np.float64))
        assert ulp.max() <= H_ULP_MAX, f"fp32 h off by {ulp.max()} ulps"
        log(f"small-integer fwd fp32 {shape}: max ulp {ulp.max()}, {int(tail.sum())} tail elements")
    else:
        yk, rk = y[keep], r[keep]
        q, sp = bf16_rne_f64(rk)
        frac = np.abs(rk) / sp
        to_mid = np.abs(frac - np.floor(frac) - 0.5) * sp
        safe = to_mid > 2e-5 * np.abs(rk) + 1e-30        # twice the short sigma's relative error bound
        assert np.array_equal(yk[safe], q[safe]), "bf16 h is not the rounding of the exact value"
        assert np.all(np.abs(yk - rk) <= sp * (1 + 1e-9)), "bf16 h off by more than one step"
        log(f"small-integer fwd bf16 {shape}: RNE-exact on {int(safe.sum())} of {safe.size}, "
            f"{int(tail.sum())} tail elements")


def _random_case(i):
    """Case i of the seeded random-shape sweep: sizes drawn so that the GEMM
    tiles (256 x 128, 256 x 256, 128 x 64), the 64-wide reduction steps and
    the decode slabs all see ragged tails."""
    rs = np.random.default_rng(20260 + i)
    M, N, K = int(rs.integers(1, 700)), int(rs.integers(1, 700)), 8 * int(rs.integers(1, 200))
    dt = "f32" if i % 3 == 0 else "bf16"
    act = "gelu_tanh" if i % 2 else "silu"
    mult = (1.0, 1.0) if i % 4 < 2 else (float(rs.uniform(0.5, 2.0)), float(rs.uniform(0.5, 2.0)))
    return M, N, K, dt, act, mult


@pytest.mark.parametrize("i", range(12))
def test_random_shapes_forward_and_backward(i):
    M, N, K, dt, act, mult = _random_case(i)
    what = f"random {i}: {dt} {act} mult={mult} ({M}, {N}, {K})"
    if dt == "bf16":
        d = synth.train_bf16(M, N, K, seed=30 + i)
    else:
        d = synth.gemm_fp32(M, N, K, seed=30 + i)
        d["dh"] = synth.normal_f32((M, N), 1.0, 30 + i, synth.STREAM_DH)
    fwd_d = {k: v for k, v in d.items() if k != "dh"}
    check_fwd(fwd_d, dt, what=what + " fwd", act=act, mult=mult)
    check_bwd(d, dt, what=what + " bwd", act=act, mult=mult)


@pytest.mark.parametrize("i", range(8))
def test_random_shapes_decode(i):
    rs = np.random.default_rng(30260 + i)
    M, N, K = int(rs.integers(1, 9)), int(rs.integers(1, 3000)), 8 * int(rs.integers(1, 1200))
    act = "gelu_tanh" if i % 2 else "silu"
    mult = (1.0, 1.0) if i % 4 < 2 else (float(rs.uniform(0.5, 2.0)), float(rs.uniform(0.5, 2.0)))
    d = synth.decode_bf16(M, N, K, seed=40 + i)
    check_fwd(d, "bf16", what=f"random decode {i}: {act} mult={mult} ({M}, {N}, {K})", via="gemv", act=act, mult=mult)
