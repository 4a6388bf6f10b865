"""Pins of the oracle's bf16-output forward (oracle.fwd_bf16), the optional
bf16 Y epilogue: Y16 = the bf16 nearest (ties to even) to the binary32 Y of
the epilogue, Y32 = f32(f32(acc) * f32(gamma * s32)).  The model here is
independent of oracle.c: exact integer sums, numpy binary32 arithmetic, and
the nearest bf16 found by comparing exact rational distances to the
neighbouring bf16 values."""
from fractions import Fraction

import numpy as np

import oracle


def _bf16_value(h):
    return float(np.array([(h & 0xFFFF) << 16], np.uint32).view(np.float32)[0])


def _nearest_bf16(y32):
    """bf16 bits nearest to the binary32 value y32, ties to an even last bit."""
    y = Fraction(float(y32))
    top = int(np.array([y32], np.float32).view(np.uint32)[0]) >> 16
    best = None
    for h in (top - 1, top, top + 1):
        h &= 0xFFFF
        v = _bf16_value(h)
        if not np.isfinite(v):
            continue
        d = abs(Fraction(v) - y)
        key = (d, h & 1)
        if best is None or key < best[0]:
            best = (key, h)
    return best[1]


def _model(xq, scale, T, g):
    acc = xq.astype(np.int64) @ T.astype(np.int64).T
    out = np.zeros(acc.shape, np.uint16)
    for t in range(acc.shape[0]):
        s32 = np.float32(scale[t])
        g32 = np.float32(g * float(s32))
        for r in range(acc.shape[1]):
            y32 = np.float32(np.float32(acc[t, r]) * g32)
            out[t, r] = _nearest_bf16(y32)
    return out


def _row_with_sum(total, k):
    """int8 activations whose sum is `total` (weights all +1)."""
    x = np.zeros(k, np.int8)
    sign = 1 if total >= 0 else -1
    left = abs(total)
    for c in range(k):
        step = min(127, left)
        x[c] = sign * step
        left -= step
    assert left == 0
    return x


def test_nearest_bf16_model_on_hand_values():
    # exact bf16 values stay; halfway cases go to the even neighbour
    assert _nearest_bf16(np.float32(1.0)) == 0x3F80
    assert _nearest_bf16(np.float32(1.0 + 2.0 ** -8)) == 0x3F80      # tie: 1.0 (even) vs 1.0078125
    assert _nearest_bf16(np.float32(1.0 + 3 * 2.0 ** -8)) == 0x3F82  # tie: 1.015625 (even)
    assert _nearest_bf16(np.float32(1.0 + 2.0 ** -8 + 2.0 ** -20)) == 0x3F81
    assert _nearest_bf16(np.float32(-(1.0 + 2.0 ** -8))) == 0xBF80


def test_bf16_y_exact_ties():
    """acc * 2^-7 exactly halfway between two bf16 values (9- and 10-bit
    sums), both signs: the even neighbour, as the model gives."""
    k = 128
    sums = [257, 259, -257, -259, 385, 513, 515, 771, -771, 1, 0, 255, 256]
    xq = np.stack([_row_with_sum(v, k) for v in sums])
    T = np.ones((1, k), np.int8)
    scale = np.full(len(sums), 2.0 ** -7)  # binary32 exactly
    got = oracle.fwd_bf16(xq, scale, T, 1.0)[:, 0]
    want = _model(xq, scale, T, 1.0)[:, 0]
    assert np.array_equal(got, want)
    # the ties themselves, by hand: 257/128 -> 256/128, 259/128 -> 260/128
    assert got[0] == 0x4000 and got[1] == 0x4002 and got[2] == 0xC000


def test_bf16_y_random_layers_match_model_and_bound():
    rng = np.random.default_rng(7)
    for tokens, k, n_out in [(3, 256, 40), (5, 384, 17), (1, 1024, 64)]:
        xq = rng.integers(-128, 128, size=(tokens, k), dtype=np.int8)
        T = rng.integers(-1, 2, size=(n_out, k), dtype=np.int8)
        a = rng.uniform(0.01, 8.0, size=tokens)
        scale = (a / 127.0).astype(np.float32).astype(np.float64)
        g = float(rng.uniform(0.001, 0.1))
        got = oracle.fwd_bf16(xq, scale, T, g)
        assert np.array_equal(got, _model(xq, scale, T, g))
        _, Y64 = oracle.fwd(xq, scale, T, g)
        Y16 = np.array([_bf16_value(int(h)) for h in got.ravel()]).reshape(got.shape)
        assert np.all(np.abs(Y16 - Y64) <= 2.0 ** -8 * np.abs(Y64) + 1e-30)


def _sensitive_cases(n_want, seed):
    """(acc, s32, gamma) where forming gamma * s in binary32, or rounding the
    binary64 product straight to bf16, changes the bf16 result."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_want:
        acc = rng.integers(-40000, 40000, size=20000)
        s = rng.uniform(1e-4, 5e-2, size=20000).astype(np.float32)
        g = rng.uniform(1e-3, 0.2, size=20000)
        g32 = (g * s.astype(np.float64)).astype(np.float32)
        g32_wrong = g.astype(np.float32) * s
        y = acc.astype(np.float32) * g32
        y_wrong = acc.astype(np.float32) * g32_wrong
        y64 = (acc.astype(np.float64) * g * s.astype(np.float64)).astype(np.float32)
        def b16(v):  # candidate search only; the pins use the exact model
            u = v.view(np.uint32).astype(np.uint64)
            return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        diff = (b16(y) != b16(y_wrong)) | (b16(y) != b16(y64))
        for i in np.flatnonzero(diff)[:n_want - len(cases)]:
            cases.append((int(acc[i]), float(s[i]), float(g[i])))
    return cases


def test_bf16_y_follows_the_binary32_epilogue():
    """Cases where a binary32 scale product, or rounding from binary64,
    would give another bf16: the oracle follows the stated binary32 steps."""
    k = 384
    T = np.ones((1, k), np.int8)
    for acc, s, g in _sensitive_cases(24, seed=11):
        xq = _row_with_sum(acc, k)[None, :]
        scale = np.array([s])
        got = oracle.fwd_bf16(xq, scale, T, g)
        assert got[0, 0] == _model(xq, scale, T, g)[0, 0], (acc, s, g)
