"""Pins for the oracle's latent-weight update (plain gradient step on
binary32 latent weights, then bf16 nearest, ties to even): against exact
rational arithmetic and hand-made half-way cases, independent of the
oracle's own rounding code."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def nearest_f32(x: Fraction) -> np.float32:
    """binary32 nearest to the rational x, ties to the even significand."""
    f = np.float32(float(x))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def nearest_bf16_bits(x: np.float32) -> int:
    """bf16 bit pattern nearest to the binary32 x, ties to even, by exact
    comparison of the candidates' values."""
    v = Fraction(float(x))
    u = int(np.array(x, np.float32).view(np.uint32))
    if v == 0:
        return u >> 16  # signed zero
    cands = []
    for h in {u >> 16, (u >> 16) + 1, (u >> 16) - 1}:
        if not 0 <= h <= 0xFFFF:
            continue
        hv = np.array([h << 16], np.uint32).view(np.float32)[0]
        if np.isfinite(hv):
            cands.append((abs(Fraction(float(hv)) - v), h & 1, h))
    return min(cands)[2] & 0xFFFF


def test_update_matches_exact_rounding_random():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(3000) * 0.02).astype(np.float32)
    g = (rng.standard_normal(3000) * 1e-2).astype(np.float32)
    for lr in (np.float32(1e-3), np.float32(0.37), np.float32(3.0)):
        nw, hb = oracle.latent_update(w, g, lr)
        for i in range(0, 3000, 7):
            exact = Fraction(float(w[i])) - Fraction(float(lr)) * Fraction(float(g[i]))
            ref = nearest_f32(exact)
            assert nw[i].view(np.uint32) == np.array(ref, np.float32).view(np.uint32), (i, lr)
            assert hb[i] == nearest_bf16_bits(nw[i]), (i, lr)


def test_update_half_way_cases_round_to_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -23)
    half = np.float32(2.0 ** -24)
    w = np.array([one + ulp, one + 2 * ulp, one], np.float32)
    g = np.array([half, half, -half], np.float32)
    nw, _ = oracle.latent_update(w, g, 1.0)
    # 1 + 2^-24: between 1 (even) and 1 + 2^-23 (odd) -> 1
    # 1 + 1.5 * 2^-23: between 1 + 2^-23 (odd) and 1 + 2^-22 (even) -> 1 + 2^-22
    # 1 + 2^-24 again, from below -> 1
    assert list(nw) == [np.float32(1.0), np.float32(1.0 + 2.0 ** -22), np.float32(1.0)]


@pytest.mark.parametrize("value,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                 # half-way, even below
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # half-way, even above
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above half-way
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (0.0, 0x0000),
])
def test_bf16_of_updated_weights(value, bits):
    _, hb = oracle.latent_update(np.array([value], np.float32), np.zeros(1, np.float32), 0.0)
    assert hb[0] == bits


def test_zero_gradient_or_rate_leaves_weights():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal(64) * 0.02).astype(np.float32)
    nw, _ = oracle.latent_update(w, np.zeros(64, np.float32), 0.5)
    assert np.array_equal(nw.view(np.uint32), w.view(np.uint32))
    nw, _ = oracle.latent_update(w, rng.standard_normal(64).astype(np.float32), 0.0)
    assert np.array_equal(nw.view(np.uint32), w.view(np.uint32))
