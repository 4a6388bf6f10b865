"""Pins for the oracle's squared-ReLU gating and its backward: exact
rational arithmetic with the stated roundings, the derivative by finite
differences of the forward in binary64, and the zero cases."""
from fractions import Fraction

import numpy as np

import oracle
from test_oracle_update import nearest_bf16_bits, nearest_f32


def rn_mul(a, b):
    """binary32 product of two binary32 values, rounded once: the exact
    rational product rounded to nearest-even; a zero product carries the
    xor of the operands' signs (the IEEE rule rational numbers lack)."""
    a, b = np.float32(a), np.float32(b)
    exact = Fraction(float(a)) * Fraction(float(b))
    if exact == 0:
        neg = bool(np.signbit(a)) != bool(np.signbit(b))
        return np.float32(-0.0) if neg else np.float32(0.0)
    return nearest_f32(exact)


def test_forward_matches_exact_rounding():
    rng = np.random.default_rng(11)
    g = rng.standard_normal(2000).astype(np.float32)
    u = rng.standard_normal(2000).astype(np.float32)
    h = oracle.relu2_gate(g, u)
    for i in range(0, 2000, 3):
        r = g[i] if g[i] > 0 else np.float32(0.0)
        hv = rn_mul(rn_mul(r, r), u[i])
        assert h[i] == nearest_bf16_bits(hv), i


def test_backward_matches_exact_rounding():
    rng = np.random.default_rng(12)
    g = rng.standard_normal(2000).astype(np.float32)
    u = rng.standard_normal(2000).astype(np.float32)
    d = rng.standard_normal(2000).astype(np.float32)
    dg, du = oracle.relu2_gate_bwd(d, g, u)
    for i in range(0, 2000, 3):
        r = g[i] if g[i] > 0 else np.float32(0.0)
        ref_du = rn_mul(d[i], rn_mul(r, r))
        ref_dg = rn_mul(rn_mul(d[i], u[i]), np.float32(2.0) * r)  # 2r is exact
        assert du[i] == nearest_bf16_bits(ref_du), i
        assert dg[i] == nearest_bf16_bits(ref_dg), i


def _bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_backward_is_the_derivative_of_the_forward():
    """Central differences of f(g, u) = relu(g)^2 u in binary64 against the
    oracle's gradients (bf16 outputs: about 3 significant digits)."""
    rng = np.random.default_rng(13)
    g = (rng.standard_normal(500) + np.sign(rng.standard_normal(500)) * 0.5).astype(np.float32)
    u = rng.standard_normal(500).astype(np.float32)
    d = rng.standard_normal(500).astype(np.float32)
    dg, du = oracle.relu2_gate_bwd(d, g, u)
    f = lambda gg, uu: np.maximum(gg, 0.0) ** 2 * uu
    eps = 1e-6
    g64, u64, d64 = g.astype(np.float64), u.astype(np.float64), d.astype(np.float64)
    num_dg = d64 * (f(g64 + eps, u64) - f(g64 - eps, u64)) / (2 * eps)
    num_du = d64 * (f(g64, u64 + eps) - f(g64, u64 - eps)) / (2 * eps)
    assert np.allclose(_bf16_values(dg), num_dg, rtol=1e-2, atol=1e-6)
    assert np.allclose(_bf16_values(du), num_du, rtol=1e-2, atol=1e-6)


def test_non_positive_gate_gives_zero_and_keeps_signs():
    g = np.array([0.0, -1.5, -0.0, -3.0], np.float32)
    u = np.array([2.0, -3.0, 1.0, 4.0], np.float32)
    d = np.array([1.0, 1.0, -1.0, -2.0], np.float32)
    h = oracle.relu2_gate(g, u)
    assert list(h) == [0x0000, 0x8000, 0x0000, 0x0000]  # +0 * (-3) = -0
    dg, du = oracle.relu2_gate_bwd(d, g, u)
    assert list(du) == [0x0000, 0x0000, 0x8000, 0x8000]  # dh * (+0)
    assert list(dg) == [0x0000, 0x8000, 0x8000, 0x8000]  # (dh u) * (+0)
