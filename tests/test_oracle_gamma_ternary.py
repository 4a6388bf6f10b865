"""Pins for the oracle's absmean scale and masked ternary codes
(BitNet b1.58 2B4T article §一: absmean ternary weights; Sparse-BitNet
article §六: quantise first, then sparsify).  The scale is checked against
Python's correctly rounded math.fsum and against exact Fractions; the codes
against exact-quotient rounding with Python's round-half-even."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_linear_layers_group_amd import synth


def vals(W):
    return synth.bf16_bits_to_f32(W).astype(np.float64)


def test_gamma_equals_fsum_on_workload_weights():
    W = synth.weights(256, 512, seed=4)
    a = np.abs(vals(W)).ravel()
    assert oracle.gamma(W) == math.fsum(a) / a.size


def test_gamma_exact_across_the_whole_bf16_range():
    # subnormals, tiny, large magnitudes in one tensor: a plain float sum
    # loses bits here, the exact sum rounded once does not.
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 0x7F80, size=(32, 128), dtype=np.uint16)  # all finite magnitudes
    bits |= (rng.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15)
    a = np.abs(vals(bits)).ravel()
    exact = sum(Fraction(float(x)) for x in a)
    assert oracle.gamma(bits) == float(exact) / a.size
    assert oracle.gamma(bits) == math.fsum(a) / a.size


def test_gamma_subnormal_and_tiny_magnitudes():
    # bf16 subnormals (exponent field 0) next to the smallest normals: each
    # must enter the sum with its exact value
    rng = np.random.default_rng(10)
    bits = rng.integers(1, 0x0200, size=(16, 128), dtype=np.uint16)
    a = np.abs(vals(bits)).ravel()
    assert np.count_nonzero(bits < 0x80) > 100
    assert oracle.gamma(bits) == math.fsum(a) / a.size
    only_sub = rng.integers(1, 0x80, size=(8, 128), dtype=np.uint16)
    b = np.abs(vals(only_sub)).ravel()
    assert oracle.gamma(only_sub) == math.fsum(b) / b.size > 0.0


def test_gamma_round_half_even_case():
    # 2^53 + 1 units of the last place: exact sum sits half-way between two
    # binary64 values; ties-to-even picks the even significand.
    big = np.float32(2.0 ** 60)
    small = np.float32(2.0 ** 7)  # 2^60 + 2^7 = 2^60 (1 + 2^-53): half an ulp
    W = synth.f32_to_bf16_bits(np.array([[big, small]], np.float32))
    expect = float(Fraction(2 ** 60) + Fraction(2 ** 7)) / 2.0
    assert oracle.gamma(W) == expect == 2.0 ** 59
    W3 = synth.f32_to_bf16_bits(np.array([[big, small, small, np.float32(0)]], np.float32))
    expect3 = float(Fraction(2 ** 60) + 2 * Fraction(2 ** 7)) / 4.0  # exactly representable
    assert oracle.gamma(W3) == expect3


def test_gamma_constant_magnitude():
    for c in (0.0078125, 0.019, 3.0):
        f = np.full((8, 128), np.float32(c))
        f[::2] *= -1
        W = synth.f32_to_bf16_bits(f)
        c_bf16 = abs(float(synth.bf16_bits_to_f32(W[0:1, 0:1])[0, 0]))
        assert oracle.gamma(W) == c_bf16


def test_gamma_zero_tensor():
    assert oracle.gamma(np.zeros((4, 128), np.uint16)) == 0.0


def test_gamma_statistics_match_half_normal_mean():
    W = synth.weights(1024, 2048, seed=0)
    g = oracle.gamma(W)
    mu = 0.02 * math.sqrt(2.0 / math.pi)
    sd = 0.02 * math.sqrt(1 - 2 / math.pi) / math.sqrt(W.size)
    assert abs(g - mu) < 6 * sd + 1e-6  # bf16 rounding bias is far below this


def test_gamma_masked_ablation():
    W = synth.weights(64, 256, seed=8)
    mb = oracle.mask(W, 6, 8)
    keep = np.unpackbits(mb, axis=1, bitorder="little").astype(bool)
    a = np.abs(vals(W))
    assert oracle.gamma(W, over_masked=True, mask_bits=mb) == math.fsum(a[keep]) / W.size
    assert oracle.gamma(W, over_masked=True, mask_bits=mb) < oracle.gamma(W)


def exact_code(w, g):
    """clip(round_half_even(w / g), -1, 1) on the exact quotient."""
    if g == 0:
        return 0
    q = Fraction(w) / Fraction(g)
    return max(-1, min(1, round(q)))  # round(Fraction) is ties-to-even


@pytest.mark.parametrize("n,m", [(8, 8), (6, 8), (4, 8), (2, 4), (3, 8), (2, 8)])
def test_ternary_matches_exact_quotient_rounding(n, m):
    W = synth.weights(24, 256, seed=12)
    mb = oracle.mask(W, n, m)
    g = oracle.gamma(W)
    T = oracle.ternary(W, mb, g)
    keep = np.unpackbits(mb, axis=1, bitorder="little")
    v = vals(W)
    for r in range(24):
        for c in range(256):
            expect = exact_code(v[r, c], g) if keep[r, c] else 0
            assert T[r, c] == expect


def test_ternary_half_way_rounds_to_zero():
    # equal counts of |W| = c and 3c: gamma = 2c, so c/gamma = 1/2 exactly
    # (ties to even -> 0) and 3c/gamma = 3/2 (-> 2, clipped to 1).
    c = np.float32(0.015625)
    row = np.array([c, -3 * c, -c, 3 * c] * 32, np.float32)
    W = synth.f32_to_bf16_bits(np.tile(row, (4, 1)))
    mb = oracle.mask(W, 8, 8)
    g = oracle.gamma(W)
    assert g == 2 * float(c)
    T = oracle.ternary(W, mb, g)
    assert list(T[0, :4]) == [0, -1, 0, 1]


def test_ternary_values_and_mask_zeros():
    W = synth.weights(64, 512, seed=13)
    mb = oracle.mask(W, 6, 8)
    T = oracle.ternary(W, mb, oracle.gamma(W))
    keep = np.unpackbits(mb, axis=1, bitorder="little").astype(bool)
    assert set(np.unique(T)) <= {-1, 0, 1}
    assert np.all(T[~keep] == 0)
    assert np.all(np.count_nonzero(T.reshape(64, 64, 8), axis=2) <= 6)
    # sign follows W wherever the code is nonzero
    v = vals(W)
    nz = T != 0
    assert np.all(np.sign(v[nz]) == T[nz])


def test_dense_pattern_is_plain_absmean_bitnet():
    W = synth.weights(32, 256, seed=14)
    g = oracle.gamma(W)
    T = oracle.ternary(W, oracle.mask(W, 8, 8), g)
    v = vals(W)
    dense = np.where(2 * np.abs(v) > g, np.sign(v), 0).astype(np.int8)
    assert np.array_equal(T, dense)


def test_no_dropped_weight_outranks_a_kept_code():
    W = synth.weights(64, 512, seed=15)
    mb = oracle.mask(W, 6, 8)
    g = oracle.gamma(W)
    T = oracle.ternary(W, mb, g)
    dense = oracle.ternary(W, oracle.mask(W, 8, 8), g)
    keep = np.unpackbits(mb, axis=1, bitorder="little").astype(bool)
    # a dropped entry that would have been nonzero implies every kept entry
    # of its group is nonzero too (kept magnitudes are at least as large)
    Tg = np.abs(T).reshape(64, 64, 8)
    Dg = np.abs(dense).reshape(64, 64, 8)
    Kg = keep.reshape(64, 64, 8)
    for r in range(64):
        for gi in range(64):
            if np.any(Dg[r, gi][~Kg[r, gi]] == 1):
                assert np.all(Tg[r, gi][Kg[r, gi]] == 1)


def test_zero_fraction_matches_closed_form():
    """Dense codes are zero where |W| <= gamma/2 = 0.02*sqrt(2/pi)/2, i.e.
    with probability 2*Phi(sqrt(1/(2 pi))) - 1 = 0.3101 for N(0, 0.02)."""
    W = synth.weights(512, 2048, seed=0)
    g = oracle.gamma(W)
    T = oracle.ternary(W, oracle.mask(W, 8, 8), g)
    p = math.erf(math.sqrt(1 / (2 * math.pi)) / math.sqrt(2))
    assert abs(np.mean(T == 0) - p) < 0.003


def test_all_zero_tensor_codes_are_zero():
    W = np.zeros((16, 128), np.uint16)
    T = oracle.ternary(W, oracle.mask(W, 6, 8), oracle.gamma(W))
    assert not T.any()
