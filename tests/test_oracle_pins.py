"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against mathematics, a library routine, brute
force, or a hand-derived value, so that a plausible mistake in the oracle (a
dropped term, a wrong sign or index, a transposed operand, a wrong rounding
direction) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- activation

def test_silu_closed_form_values():
    # sigma(0) = 1/2, silu(0) = 0, silu'(0) = 1/2.
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu_grad(0.0) == 0.5
    # sigma(ln 3) = 3/4 exactly, so silu(ln 3) = 0.75 ln 3 and silu(-ln 3) = -0.25 ln 3.
    l3 = math.log(3.0)
    assert math.isclose(oracle.silu(l3), 0.75 * l3, rel_tol=1e-15)
    assert math.isclose(oracle.silu(-l3), -0.25 * l3, rel_tol=1e-15)
    # silu'(ln 3) = s(1 + z(1 - s)) with s = 3/4: 0.75 * (1 + ln3/4).
    assert math.isclose(oracle.silu_grad(l3), 0.75 * (1 + l3 / 4), rel_tol=1e-14)


def test_silu_identities_on_grid():
    z = np.linspace(-30, 30, 6001)
    # sigma(z) + sigma(-z) = 1  =>  silu(z) - silu(-z) = z and silu'(z) + silu'(-z) = 1.
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.silu_grad(z) + oracle.silu_grad(-z), 1.0, rtol=0, atol=1e-13)
    # Tails: silu(z) -> z for z >> 0, -> -0 for z << 0.
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15 and math.copysign(1, oracle.silu(-800.0)) == -1


def test_silu_grad_matches_central_differences():
    z = np.linspace(-12, 12, 2401)
    eps = 1e-6
    fd = (oracle.silu(z + eps) - oracle.silu(z - eps)) / (2 * eps)
    np.testing.assert_allclose(oracle.silu_grad(z), fd, rtol=0, atol=1e-8)


def test_silu_special_values():
    assert oracle.silu(np.inf) == np.inf
    assert np.isnan(oracle.silu(-np.inf))
    assert np.isnan(oracle.silu(np.nan))


# ------------------------------------------------------------- GELU (tanh)

def test_gelu_tanh_matches_torch_library_routine():
    """torch's gelu(approximate='tanh') in float64 (a library routine) on a grid
    that spans the saturated tails."""
    z = np.concatenate([np.linspace(-40, 40, 40001), [0.0, -0.0, 1e-300, -1e-300, 5e5, -5e5]])
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    got = oracle.gelu_tanh(z)
    # torch evaluates 1 + tanh(y), which cancels in the negative tail, so the
    # comparison is absolute there (relative to |z|) and relative elsewhere.
    np.testing.assert_array_less(np.abs(got - ref), 1e-15 * np.maximum(1.0, np.abs(z)) + 1e-300)
    big = np.abs(ref) > 1e-3
    np.testing.assert_allclose(got[big], ref[big], rtol=1e-13)


def test_gelu_tanh_negative_tail_relative_accuracy():
    # In the tail the value is z * e^(2y) / (1 + e^(2y)); with log-space
    # arithmetic: log|h| = log|z| + 2y - log1p(e^(2y)).
    z = np.linspace(-30.0, -4.0, 261)
    y = oracle.GELU_C * (z + oracle.GELU_A * z ** 3)
    logh = np.log(-z) + 2 * y - np.log1p(np.exp(2 * y))
    got = oracle.gelu_tanh(z)
    ok = logh > -700
    np.testing.assert_allclose(np.log(-got[ok]), logh[ok], rtol=1e-13, atol=1e-13)


def test_gelu_tanh_identity_limits_and_erf_distance():
    z = np.linspace(-20, 20, 4001)
    # gelu(z) - gelu(-z) = z (tanh is odd), as for SiLU.
    np.testing.assert_allclose(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z), z, rtol=1e-14, atol=1e-14)
    # The tanh form stays within 5e-4 of the erf GELU z * Phi(z) everywhere.
    from scipy.special import erf
    exact = 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))
    assert np.max(np.abs(oracle.gelu_tanh(z) - exact)) < 5e-4
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    v = oracle.gelu_tanh(np.array([np.inf, -np.inf, np.nan]))
    assert v[0] == np.inf and np.isnan(v[1]) and np.isnan(v[2])


def test_gelu_tanh_grad_against_torch_autograd_and_differences():
    """The GELU-tanh derivative: torch's autograd of gelu(approximate="tanh")
    in float64 (a library routine), and central differences of the oracle's
    own gelu_tanh."""
    z = np.linspace(-12.0, 12.0, 24001)
    zt = torch.from_numpy(z.copy()).requires_grad_(True)
    torch.nn.functional.gelu(zt, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_grad(z), zt.grad.numpy(), rtol=1e-12, atol=1e-14)
    h = 1e-6
    fd = (oracle.gelu_tanh(z + h) - oracle.gelu_tanh(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(z), fd, rtol=0, atol=2e-9)
    assert oracle.gelu_tanh_grad(np.array([0.0]))[0] == 0.5          # sigma(0) = 1/2


def test_geglu_backward_matches_finite_differences():
    """Central differences of L = sum(dh * GELU(mg x Wg^T) * (mu x Wu^T)) w.r.t.
    every element of x, Wg, Wu against swiglu_bwd(act="gelu_tanh")."""
    d = synth.tiny_fp32(seed=7, M=3, N=10, K=12)
    x, wg, wu, dh = (d[k].astype(np.float64) for k in ("x", "wg", "wu", "dh"))
    for mg, mu in ((1.0, 1.0), (0.7, -1.3)):
        dx, dwg, dwu = oracle.swiglu_bwd(x, wg, wu, dh, mg, mu, act="gelu_tanh")

        def loss(x_, wg_, wu_):
            return float(np.sum(dh * oracle.glu_fwd(x_, wg_, wu_, "gelu_tanh", mg, mu)))

        eps = 1e-6
        for name, grad in (("x", dx), ("wg", dwg), ("wu", dwu)):
            args = {"x": x.copy(), "wg": wg.copy(), "wu": wu.copy()}
            t = args[name]
            fd = np.empty_like(t)
            for idx in np.ndindex(t.shape):
                v = t[idx]
                t[idx] = v + eps
                lp = loss(args["x"], args["wg"], args["wu"])
                t[idx] = v - eps
                lm = loss(args["x"], args["wg"], args["wu"])
                t[idx] = v
                fd[idx] = (lp - lm) / (2 * eps)
            err = np.max(np.abs(fd - grad) / np.maximum(1.0, np.abs(grad)))
            assert err < 1e-7, (mg, mu, name, err)


def test_geglu_forward_orientation_with_selection_weights():
    """The gated forward with GELU: g and u pick known x columns."""
    M, N, K = 4, 6, 9
    rs = np.random.default_rng(5)
    x = rs.standard_normal((M, K)) * 2
    pg = rs.integers(0, K, N)
    pu = rs.integers(0, K, N)
    wg = np.zeros((N, K)); wg[np.arange(N), pg] = 1.0
    wu = np.zeros((N, K)); wu[np.arange(N), pu] = 1.0
    h = oracle.glu_fwd(x, wg, wu, "gelu_tanh")
    ref = torch.nn.functional.gelu(torch.from_numpy(x[:, pg]), approximate="tanh").numpy() * x[:, pu]
    np.testing.assert_allclose(h, ref, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(oracle.glu_fwd(x, wg, wu, "silu"), oracle.swiglu_fwd(x, wg, wu))


# ------------------------------------------------------------------- forward

def test_forward_orientation_with_selection_weights():
    """One-hot weight rows select input columns: g[m,n] = x[m, pg[n]], u[m,n] = x[m, pu[n]].

    Fails on a transposed weight, a swapped gate/up pair, or a wrong axis.
    """
    M, N, K = 5, 7, 11
    rs = np.random.default_rng(3)
    x = rs.standard_normal((M, K))
    pg = rs.integers(0, K, N)
    pu = rs.integers(0, K, N)
    wg = np.zeros((N, K)); wg[np.arange(N), pg] = 1.0
    wu = np.zeros((N, K)); wu[np.arange(N), pu] = 1.0
    h = oracle.swiglu_fwd(x, wg, wu)
    expect = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            a, b = x[m, pg[n]], x[m, pu[n]]
            expect[m, n] = a / (1.0 + math.exp(-a)) * b
    np.testing.assert_allclose(h, expect, rtol=1e-15, atol=0)


def test_forward_against_exact_sum_loops():
    """Tiny shapes: each g/u dot product by math.fsum (exactly rounded) in plain loops."""
    d = synth.tiny_fp32(seed=1, M=3, N=9, K=16)
    x, wg, wu = (d[k].astype(np.float64) for k in ("x", "wg", "wu"))
    h = oracle.swiglu_fwd(x, wg, wu)
    for m in range(3):
        for n in range(9):
            g = math.fsum(x[m, k] * wg[n, k] for k in range(16))
            u = math.fsum(x[m, k] * wu[n, k] for k in range(16))
            assert math.isclose(h[m, n], g / (1 + math.exp(-g)) * u, rel_tol=1e-13, abs_tol=1e-15)


def test_row_helpers_agree_with_full():
    d = synth.tiny_fp32(seed=2, M=6, N=10, K=8)
    x, wg, wu, dh = (d[k].astype(np.float64) for k in ("x", "wg", "wu", "dh"))
    rows = np.array([0, 3, 5])
    cols = np.array([1, 4, 9])
    h = oracle.swiglu_fwd(x, wg, wu)
    np.testing.assert_array_equal(oracle.swiglu_fwd_rows(x, wg, wu, rows), h[rows])
    dx, dwg, dwu = oracle.swiglu_bwd(x, wg, wu, dh)
    np.testing.assert_allclose(oracle.swiglu_bwd_dx_rows(x, wg, wu, dh, rows), dx[rows], rtol=1e-14, atol=1e-15)
    a, b = oracle.swiglu_bwd_dw_rows(x, wg, wu, dh, cols)
    np.testing.assert_allclose(a, dwg[cols], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(b, dwu[cols], rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ backward

def test_backward_matches_finite_differences_everywhere():
    """Central differences of L = sum(dh * h) w.r.t. every element of x, Wg, Wu
    (4x64 input, 128x64 weights: 16,640 partials) against the closed-form backward."""
    d = synth.tiny_fp32(seed=0)
    x, wg, wu, dh = (d[k].astype(np.float64) for k in ("x", "wg", "wu", "dh"))
    dx, dwg, dwu = oracle.swiglu_bwd(x, wg, wu, dh)

    def loss(x_, wg_, wu_):
        g = x_ @ wg_.T
        u = x_ @ wu_.T
        return float(np.sum(dh * (g / (1.0 + np.exp(-g))) * u))

    eps = 1e-6
    worst = 0.0
    for name, grad in (("x", dx), ("wg", dwg), ("wu", dwu)):
        args = {"x": x.copy(), "wg": wg.copy(), "wu": wu.copy()}
        t = args[name]
        fd = np.empty_like(t)
        for idx in np.ndindex(t.shape):
            v = t[idx]
            t[idx] = v + eps
            lp = loss(args["x"], args["wg"], args["wu"])
            t[idx] = v - eps
            lm = loss(args["x"], args["wg"], args["wu"])
            t[idx] = v
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - grad) / np.maximum(1.0, np.abs(grad)))
        worst = max(worst, err)
        assert err < 1e-7, (name, err)
    assert worst < 1e-7


def test_multiplier_forward_is_weight_scaling():
    """The multipliers scale the projections: glu_fwd with (mg, mu) equals the
    plain (pinned) forward on mg * Wg and mu * Wu, for both activations."""
    d = synth.tiny_fp32(seed=5, M=5, N=12, K=16)
    x, wg, wu = (d[k].astype(np.float64) for k in ("x", "wg", "wu"))
    for act in ("silu", "gelu_tanh"):
        for mg, mu in ((0.7, 1.3), (-2.5, 0.125), (1.0, 1.0)):
            h = oracle.glu_fwd(x, wg, wu, act, mg, mu)
            ref = oracle.glu_fwd(x, mg * wg, mu * wu, act)
            np.testing.assert_allclose(h, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(oracle.glu_fwd(x, wg, wu, "silu", 1.0, 1.0), oracle.swiglu_fwd(x, wg, wu))


def test_multiplier_backward_matches_finite_differences():
    """Central differences of L = sum(dh * SiLU(mg x Wg^T) * (mu x Wu^T)) w.r.t.
    every element of x, Wg and Wu against swiglu_bwd with the multipliers;
    multipliers of 1 give the plain backward exactly; the row helpers agree."""
    d = synth.tiny_fp32(seed=6, M=3, N=10, K=12)
    x, wg, wu, dh = (d[k].astype(np.float64) for k in ("x", "wg", "wu", "dh"))
    mg, mu = 0.7, -1.3
    dx, dwg, dwu = oracle.swiglu_bwd(x, wg, wu, dh, mg, mu)

    def loss(x_, wg_, wu_):
        g = mg * (x_ @ wg_.T)
        u = mu * (x_ @ wu_.T)
        return float(np.sum(dh * (g / (1.0 + np.exp(-g))) * u))

    eps = 1e-6
    for name, grad in (("x", dx), ("wg", dwg), ("wu", dwu)):
        args = {"x": x.copy(), "wg": wg.copy(), "wu": wu.copy()}
        t = args[name]
        fd = np.empty_like(t)
        for idx in np.ndindex(t.shape):
            v = t[idx]
            t[idx] = v + eps
            lp = loss(args["x"], args["wg"], args["wu"])
            t[idx] = v - eps
            lm = loss(args["x"], args["wg"], args["wu"])
            t[idx] = v
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - grad) / np.maximum(1.0, np.abs(grad)))
        assert err < 1e-7, (name, err)
    for a, b in zip(oracle.swiglu_bwd(x, wg, wu, dh, 1.0, 1.0), oracle.swiglu_bwd(x, wg, wu, dh)):
        np.testing.assert_array_equal(a, b)
    rows, cols = np.array([0, 2]), np.array([1, 7, 9])
    np.testing.assert_allclose(oracle.swiglu_bwd_dx_rows(x, wg, wu, dh, rows, mg, mu), dx[rows], rtol=1e-14,
                               atol=1e-15)
    a, b = oracle.swiglu_bwd_dw_rows(x, wg, wu, dh, cols, mg, mu)
    np.testing.assert_allclose(a, dwg[cols], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(b, dwu[cols], rtol=1e-14, atol=1e-15)


def test_act_bwd_matches_finite_differences():
    """Elementwise backward: central differences of
    L = sum(dy * w * SiLU(clamp(g)) * clamp(u)) w.r.t. every g, u and w,
    with the clamp on (values kept at least 1e-3 away from +-L, where the
    clamp has its kinks) and off.  weight_grad is dL/dw."""
    rs = np.random.default_rng(11)
    rows, cols = 6, 40
    for L in (np.inf, 1.3):
        g = rs.normal(0.0, 2.0, (rows, cols))
        u = rs.normal(0.0, 2.0, (rows, cols))
        if np.isfinite(L):
            for a in (g, u):
                near = np.abs(np.abs(a) - L) < 1e-3
                a[near] += 3e-3
        dy = rs.normal(0.0, 1.0, (rows, cols))
        w = rs.uniform(0.1, 1.0, rows)

        def loss(g_, u_, w_):
            gc = np.clip(g_, -L, L)
            uc = np.clip(u_, -L, L)
            return float(np.sum(dy * w_[:, None] * (gc / (1.0 + np.exp(-gc))) * uc))

        dg, du, wgrad = oracle.act_bwd(g, u, dy, L, w)
        eps = 1e-6
        for name, grad in (("g", dg), ("u", du), ("w", wgrad)):
            args = {"g": g.copy(), "u": u.copy(), "w": w.copy()}
            t = args[name]
            fd = np.empty_like(t)
            for idx in np.ndindex(t.shape):
                v = t[idx]
                t[idx] = v + eps
                lp = loss(args["g"], args["u"], args["w"])
                t[idx] = v - eps
                lm = loss(args["g"], args["u"], args["w"])
                t[idx] = v
                fd[idx] = (lp - lm) / (2 * eps)
            err = np.max(np.abs(fd - grad) / np.maximum(1.0, np.abs(grad)))
            assert err < 1e-7, (L, name, err)
        if np.isfinite(L):
            # Clamped positions carry exactly zero gradient.
            assert np.all(dg[np.abs(g) > L] == 0.0) and np.all(du[np.abs(u) > L] == 0.0)
            assert np.count_nonzero(np.abs(g) > L) > 10


def test_act_bwd_special_cases():
    # Without weights the result is that of unit weights.
    rs = np.random.default_rng(12)
    g, u, dy = (rs.normal(0, 1.5, (3, 8)) for _ in range(3))
    a = oracle.act_bwd(g, u, dy)
    b = oracle.act_bwd(g, u, dy, np.inf, np.ones(3))
    for x_, y_ in zip(a, b):
        np.testing.assert_array_equal(x_, y_)
    # g = 0: SiLU(0) = 0 and SiLU'(0) = 1/2, so du = 0, dg = dy * u / 2, weight_grad = 0.
    z = np.zeros((2, 4))
    dg, du, wgrad = oracle.act_bwd(z, u[:2, :4], dy[:2, :4])
    np.testing.assert_array_equal(du, 0.0)
    np.testing.assert_allclose(dg, dy[:2, :4] * u[:2, :4] / 2, rtol=1e-15)
    np.testing.assert_array_equal(wgrad, 0.0)
    # A NaN gate passes the clamp (not clamped) and gives NaN gradients in its
    # element only; an infinite up value is clamped and stops its gradient.
    g2 = np.array([[np.nan, 0.5], [0.25, 1.0]])
    u2 = np.array([[1.0, np.inf], [2.0, -3.0]])
    dy2 = np.ones((2, 2))
    dg, du, wgrad = oracle.act_bwd(g2, u2, dy2, 2.0)
    assert np.isnan(dg[0, 0]) and np.isnan(du[0, 0]) and np.isnan(wgrad[0])
    assert du[0, 1] == 0.0 and dg[0, 1] > 0 and du[1, 1] == 0.0
    assert math.isclose(du[1, 0], 0.25 / (1 + math.exp(-0.25)), rel_tol=1e-15)


def test_dswiglu_reduces_to_product_rule_at_zero_gate():
    # At g = 0: silu(0) = 0 and silu'(0) = 1/2, so du = 0 and dg = dh * u / 2.
    g = np.zeros(4)
    u = np.array([1.0, -2.0, 3.0, 0.5])
    dh = np.array([2.0, 1.0, -1.0, 4.0])
    dg, du = oracle.dswiglu(g, u, dh)
    np.testing.assert_array_equal(du, 0.0)
    np.testing.assert_array_equal(dg, dh * u / 2)


# ------------------------------------------------------------- e4m3 encoding

def _decode_table_bruteforce():
    """All 256 codes decoded from the OCP E4M3FN field definition."""
    vals = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 0xF and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m / 8.0 * 2.0 ** (1 - 7)
        else:
            vals[c] = s * (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def test_e4m3_decode_table_and_known_points():
    t = _decode_table_bruteforce()
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(d), np.isnan(t))
    np.testing.assert_array_equal(d[~np.isnan(d)], t[~np.isnan(t)])
    assert oracle.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert oracle.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6
    assert oracle.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9
    assert oracle.e4m3_decode(np.uint8(0x38)) == 1.0


def _encode_bruteforce(v):
    """Nearest finite code by exhaustive search over all 256 codes, ties to the
    even code; NaN/inf -> NaN; a value nearer to 480 than to 448 -> NaN."""
    t = _decode_table_bruteforce()
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v.ravel()):
        if not np.isfinite(x):
            out.flat[i] = 0x7F
            continue
        if abs(x) > 464.0:
            out.flat[i] = 0x7F | (0x80 if x < 0 else 0)
            continue
        best, bestd = None, None
        for c in range(256):
            if np.isnan(t[c]) or (np.signbit(t[c]) != np.signbit(x) and t[c] != 0):
                continue
            if t[c] == 0 and (c & 0x80) != (0x80 if np.signbit(x) else 0):
                continue
            dist = abs(t[c] - x)
            if best is None or dist < bestd or (dist == bestd and c % 2 == 0 and best % 2 == 1):
                best, bestd = c, dist
        out.flat[i] = best
    return out


def _lattice_probe_values(rs, n_random):
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1000), pos, [464.0, 463.9, 464.1, 500.0]])
    rnd = rs.uniform(0, 470, n_random) * rs.choice([1, 2.0 ** -6, 2.0 ** -9, 1e-3], n_random)
    v = np.concatenate([near, -near, rnd, -rnd, [0.0, -0.0]])
    return v


def test_e4m3_encode_matches_bruteforce():
    rs = np.random.default_rng(7)
    v = _lattice_probe_values(rs, 300)
    got = oracle.e4m3_encode(v)
    ref = _encode_bruteforce(v)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_matches_torch_float8_cast():
    """Library pin: torch's float8_e4m3fn cast (round to nearest even, no saturation)."""
    rs = np.random.default_rng(11)
    v = np.concatenate([
        _lattice_probe_values(rs, 20000),
        rs.standard_normal(200000) * np.exp2(rs.integers(-14, 9, 200000)),
        [np.inf, -np.inf, np.nan, 1e30, -1e30, 2.0 ** -200],
    ]).astype(np.float32)
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v.astype(np.float64))
    nan_t = (t & 0x7F) == 0x7F
    nan_g = (got & 0x7F) == 0x7F
    np.testing.assert_array_equal(nan_g, nan_t)
    np.testing.assert_array_equal(got[~nan_g], t[~nan_t])


# ------------------------------------------------------------- UE8M0 exponent

def test_ue8m0_exponent_matches_linear_search():
    rs = np.random.default_rng(5)
    amax = np.concatenate([
        448.0 * np.exp2(np.arange(-140, 121, dtype=np.float64)),
        rs.uniform(0.5, 2, 2000) * np.exp2(rs.integers(-150, 120, 2000)),
        [0.0, 2.0 ** -149, 2.0 ** -126, 3.4e38],
    ])
    amax = amax[amax < 3.4e38].astype(np.float32).astype(np.float64)
    amax = np.concatenate([amax, np.nextafter(amax.astype(np.float32), np.float32(np.inf)).astype(np.float64)])
    amax = amax[np.isfinite(amax)]
    got = oracle.ue8m0_exponent(amax)
    for a, e in zip(amax, got):
        ref = 127
        for E in range(-127, 128):
            if a <= 448.0 * 2.0 ** E:
                ref = E
                break
        assert e == ref, (a, e, ref)
    assert oracle.ue8m0_exponent(np.array([np.inf]))[0] == 128
    assert oracle.ue8m0_byte(np.array([128]))[0] == 0xFF
    assert oracle.ue8m0_byte(np.array([-127]))[0] == 0


# --------------------------------------------------------- act_quant, by hand

def _hexf(s):
    return float(s) if s in ("inf", "-inf", "nan") else float.fromhex(s)


def _fill(spec, n):
    a = np.full(n, _hexf(spec["fill"]), dtype=np.float64)
    for k, v in spec.get("set", {}).items():
        a[int(k)] = _hexf(v)
    return a.astype(np.float32)


def load_act_quant_cases():
    with open(os.path.join(GOLDEN, "act_quant_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", load_act_quant_cases(), ids=lambda c: c["name"])
def test_act_quant_hand_cases(case):
    rows, cols = case["rows"], case["cols"]
    gate = _fill(case["gate"], rows * cols).reshape(rows, cols)
    up = _fill(case["up"], rows * cols).reshape(rows, cols)
    L = _hexf(case["clamp"])
    q, scale, count, h32 = oracle.act_quant(gate.astype(np.float64), up.astype(np.float64), L)
    for k, v in case.get("expect_h", {}).items():
        got = h32.reshape(-1)[int(k)]
        want = _hexf(v)
        assert got == want and np.signbit(got) == np.signbit(want), (k, got, want)
    np.testing.assert_array_equal(scale, np.array(case["expect_scale"], dtype=np.uint8))
    assert count == case["expect_count"]
    exp = case["expect_codes"]
    for i, c in enumerate(q.reshape(-1)):
        want = exp.get(str(i), exp["default"])
        if want == "nan":
            assert (c & 0x7F) == 0x7F, (i, hex(c))
        else:
            assert c == want, (i, hex(c), hex(want))


def load_act_bwd_fp8_cases():
    with open(os.path.join(GOLDEN, "act_bwd_fp8_cases.json")) as f:
        return json.load(f)["cases"]


def _expect_codes(q, exp, what):
    for i, c in enumerate(q.reshape(-1)):
        want = exp.get(str(i), exp["default"])
        if want == "nan":
            assert (c & 0x7F) == 0x7F, (what, i, hex(c))
        else:
            assert c == want, (what, i, hex(c), hex(want))


@pytest.mark.parametrize("case", load_act_bwd_fp8_cases(), ids=lambda c: c["name"])
def test_act_bwd_fp8_hand_cases(case):
    """The E4M3-output backward on hand-derived blocks (tests/golden): which
    output is which, the factor SiLU'(0) = 1/2, the row weight, the clamp's
    gradient stop, NaN passing, and the [rows, cols/32] scale layout."""
    rows, cols = case["rows"], case["cols"]
    gate = _fill(case["gate"], rows * cols).reshape(rows, cols).astype(np.float64)
    up = _fill(case["up"], rows * cols).reshape(rows, cols).astype(np.float64)
    dy = _fill(case["dy"], rows * cols).reshape(rows, cols).astype(np.float64)
    w = None if case["weights"] is None else np.array([_hexf(v) for v in case["weights"]])
    qg, sg, qu, su, wg = oracle.act_bwd_fp8(gate, up, dy, _hexf(case["clamp"]), w)
    np.testing.assert_array_equal(sg, np.array(case["expect_dgate_scale"], dtype=np.uint8))
    np.testing.assert_array_equal(su, np.array(case["expect_dup_scale"], dtype=np.uint8))
    _expect_codes(qg, case["expect_dgate_codes"], "dgate")
    _expect_codes(qu, case["expect_dup_codes"], "dup")
    want = np.array([_hexf(v) for v in case["expect_weight_grad"]])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(wg), nan)
    np.testing.assert_allclose(wg[~nan], want[~nan], rtol=1e-12, atol=0)


def test_act_bwd_fp8_is_the_quantised_fp32_backward_on_random_blocks():
    """On random inputs with specials the E4M3 backward equals, block by block,
    a linear-search UE8M0 exponent and an exhaustive nearest-code search on the
    once-rounded fp32 dgate and dup (brute force, not the oracle's encoder)."""
    d = synth.act_bwd_f32(3, 64, seed=12, specials=True)
    g, u, dy = (d[k].astype(np.float64) for k in ("gate", "up", "dy"))
    qg, sg, qu, su, _ = oracle.act_bwd_fp8(g, u, dy, 1.5, d["weights"].astype(np.float64))
    dg, du, _ = oracle.act_bwd(g, u, dy, 1.5, d["weights"].astype(np.float64))
    for q, sc, v in ((qg, sg, dg), (qu, su, du)):
        vb = v.astype(np.float32).astype(np.float64).reshape(3, 2, 32)
        for r in range(3):
            for b in range(2):
                blk = vb[r, b]
                fin = blk[~np.isnan(blk)]
                amax = np.max(np.abs(fin)) if fin.size else 0.0
                E = 128 if np.isinf(amax) else next(e for e in range(-127, 128) if amax <= 448.0 * 2.0 ** e)
                assert sc[r, b] == E + 127
                np.testing.assert_array_equal(q[r, b * 32:(b + 1) * 32], _encode_bruteforce(blk * 2.0 ** -E))


def test_act_quant_random_blocks_vs_bruteforce():
    """Random blocks: every scale by linear search and every code by exhaustive search."""
    d = synth.act_quant_f32(4, 64, seed=3, specials=True)
    g, u = d["gate"].astype(np.float64), d["up"].astype(np.float64)
    q, scale, count, h32 = oracle.act_quant(g, u, 3.0)
    hb = h32.astype(np.float64).reshape(4, 2, 32)
    for r in range(4):
        for b in range(2):
            blk = hb[r, b]
            fin = blk[~np.isnan(blk)]
            amax = np.max(np.abs(fin)) if fin.size else 0.0
            if np.isinf(amax):
                E = 128
            else:
                E = next(e for e in range(-127, 128) if amax <= 448.0 * 2.0 ** e)
            assert scale[r, b] == E + 127
            ref = _encode_bruteforce(blk * 2.0 ** -E)
            np.testing.assert_array_equal(q[r, b * 32:(b + 1) * 32], ref)
    assert count == int(np.sum(np.abs(g) > 3.0) + np.sum(np.abs(u) > 3.0))


def test_act_quant_geglu_variant_against_torch_gelu():
    """act="gelu_tanh": h is torch's tanh-form GELU (a library routine) of the
    clamped gate times the clamped up, then the same 1x32 quantiser."""
    d = synth.act_quant_f32(8, 64, seed=4)
    g, u = d["gate"].astype(np.float64), d["up"].astype(np.float64)
    L = 3.0
    q, scale, count, h32 = oracle.act_quant(g, u, L, act="gelu_tanh")
    gt = torch.clamp(torch.from_numpy(g), -L, L)
    ut = torch.clamp(torch.from_numpy(u), -L, L)
    ref = (torch.nn.functional.gelu(gt, approximate="tanh") * ut).numpy()
    # torch's float64 GELU and the oracle's sigma form agree to a few float64
    # ulps; rounded to fp32 they may differ only at a rounding boundary.
    # The inputs carry the specials (NaN, +-inf, subnormals): NaN must match.
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(h32), nan) and nan.any()
    diff = np.abs(h32[~nan].astype(np.float64) - ref[~nan])
    assert np.all(diff <= np.spacing(np.abs(ref[~nan]).astype(np.float32)).astype(np.float64))
    q2, s2 = oracle.quantize_1x32(h32)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(scale, s2)
    assert count == int(np.sum(np.abs(g) > L) + np.sum(np.abs(u) > L))
    _, _, _, h_silu = oracle.act_quant(g, u, L)
    assert not np.array_equal(h32, h_silu)


def test_act_fwd_against_torch_and_act_quant():
    """The non-quantised elementwise forward: torch's silu / tanh GELU (library
    routines) of the clamped gate times the clamped up; rounded to fp32 it is
    the h that act_quant quantises; the count is act_quant's."""
    d = synth.act_quant_f32(8, 64, seed=8)
    g, u = d["gate"].astype(np.float64), d["up"].astype(np.float64)
    for act, fn in (("silu", torch.nn.functional.silu),
                    ("gelu_tanh", lambda t: torch.nn.functional.gelu(t, approximate="tanh"))):
        h, count = oracle.act_fwd(g, u, 3.0, act)
        ref = (fn(torch.clamp(torch.from_numpy(g), -3.0, 3.0)) * torch.clamp(torch.from_numpy(u), -3.0, 3.0)).numpy()
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(h), nan)
        np.testing.assert_allclose(h[~nan], ref[~nan], rtol=1e-13, atol=1e-300)
        _, _, c2, h32 = oracle.act_quant(g, u, 3.0, act)
        assert count == c2
        assert np.array_equal(h.astype(np.float32), h32, equal_nan=True)


# ------------------------------------------------------------------- metrics

def test_metrics():
    r = np.array([1.0, -2.0, 4.0])
    assert oracle.normwise_rel_err(r, r) == 0.0
    assert oracle.normwise_rel_err(r + np.array([0, 0.4, 0]), r) == pytest.approx(0.1)
    assert oracle.cosine(r, 3 * r) == pytest.approx(1.0)
    assert oracle.cosine(np.array([1.0, 0]), np.array([0, 1.0])) == 0.0
    np.testing.assert_array_equal(oracle.e4m3_ordinal(np.array([0x00, 0x80, 0x01, 0x81], np.uint8)), [0, 0, 1, -1])


# ------------------------------------------------------- inputs and page facts

def test_bf16_rounding_matches_torch():
    rs = np.random.default_rng(1)
    a = (rs.standard_normal(100000) * np.exp2(rs.integers(-30, 30, 100000))).astype(np.float32)
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ours), torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_page_size_fact_pins_bf16_weight_pair_layout():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    N, K = facts["decode_pair_bytes"]["shape_NK"]
    d = synth.decode_bf16(1, N, K)
    assert d["wg"].shape == (N, K) and d["wu"].shape == (N, K)
    assert (d["wg"].nbytes + d["wu"].nbytes) / 2 ** 20 == facts["decode_pair_bytes"]["value_MB"]
    assert facts["scale_block"]["value"] == [1, 32]


def test_synth_is_deterministic_and_distributed_as_stated():
    a = synth.normal_f32((1000, 100), 0.02, 0, 2)
    b = synth.normal_f32((1000, 100), 0.02, 0, 2)
    np.testing.assert_array_equal(a, b)
    assert abs(a.std() - 0.02) < 0.001 and abs(a.mean()) < 0.001
    d = synth.act_quant_f32(400, 256, seed=0)
    g = d["gate"]
    nonfin = ~np.isfinite(g)
    sub = np.isfinite(g) & (g != 0) & (np.abs(g) < np.float32(2.0 ** -126))
    assert 0.0005 < nonfin.mean() < 0.0015
    assert 0.008 < sub.mean() < 0.012
