"""Pins of the MX-native FP4 oracle (E2M1 elements, E8M0 scale per 32) against a
hand-derived block, exact rational brute force, ties, saturation, round trips and the
error bound."""
from fractions import Fraction

import numpy as np
import pytest

import oracle

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _brute_block(xs):
    """Exact-rational MX quantization of one 32-element block: (codes, scale byte)."""
    fx = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in fx)
    if amax == 0:
        e = -127
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= amax:
            e += 1
        while Fraction(2) ** e > amax:
            e -= 1
        e = max(-127, min(127, e - 2))
    X = Fraction(2) ** e
    codes = []
    for v, raw in zip(fx, xs):
        q = abs(v) / X
        best = None
        for c, g in enumerate(GRID):  # nearest; ties to the even code (mantissa bit 0)
            d = abs(q - g)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        c = best[1]
        if q > 6:
            c = 7
        codes.append(c | (8 if np.signbit(float(raw)) else 0))  # sign of the float, -0 included
    return codes, e + 127


def test_hand_derived_block():
    # amax 2.5: floor(log2 2.5) = 1, e = -1, X = 1/2; q = 2 -> 2 (code 4); -5 is the tie
    # between 4 and 6 -> 4 (code 6, negative: 0xE); 0.6 -> 0.5 (code 1); 0.3 -> 0.5 (0.6
    # is nearer 0.5 than 1.0) code 1; scale byte 126
    x = np.zeros((1, 32))
    x[0, :4] = [1.0, -2.5, 0.3, 0.15]
    codes, scales = oracle.mx_quantize(x)
    assert list(codes[0, :4]) == [4, 0xE, 1, 1]  # 0.15 / 0.5 = 0.3 -> 0.5
    assert scales[0, 0] == 126
    assert np.array_equal(oracle.mx_dequantize(codes, scales)[0, :4], [1.0, -2.0, 0.25, 0.25])


def test_e8m0_anchors():
    assert oracle.e8m0_value(127) == 1.0 and oracle.e8m0_value(128) == 2.0
    assert oracle.e8m0_value(0) == 2.0 ** -127 and oracle.e8m0_value(254) == 2.0 ** 127
    v = oracle.e8m0_value(np.arange(255))
    assert np.all(v[1:] == 2 * v[:-1])
    assert np.isnan(oracle.e8m0_value(255))


def test_brute_force_random_blocks():
    rng = np.random.default_rng(91)
    x = (rng.standard_normal((6, 256)) * np.exp(rng.uniform(-30, 30, (6, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 32:64] = -0.0
    codes, scales = oracle.mx_quantize(x)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            bc, bs = _brute_block(x[r, 32 * b:32 * b + 32])
            assert list(codes[r, 32 * b:32 * b + 32]) == bc, (r, b)
            assert scales[r, b] == bs, (r, b)


def test_ties_and_saturation():
    # block max 4 -> X = 1: midpoints go to the even neighbour; 7.5 in a block of max 7.5
    # (e = 0) saturates to 6
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5]
    x = np.zeros((2, 32))
    x[0, :6] = mids
    x[0, 31] = 4.0
    x[1, 0] = 7.5
    x[1, 1] = 5.0  # tie between 4 and 6 at X = 1 -> 4
    codes, scales = oracle.mx_quantize(x)
    assert list(codes[0, :6]) == [0, 2, 2, 4, 4, 6]  # 0, 1, 1, 2, 2, 4
    assert scales[0, 0] == 127 and scales[1, 0] == 127
    assert codes[1, 0] == 7 and codes[1, 1] == 6


def test_round_trip_and_error_bound():
    rng = np.random.default_rng(92)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    exact = rng.choice(grid, (4, 128)) * rng.choice([-1, 1], (4, 128))
    exact[:, ::32] = 6.0
    exact *= np.ldexp(1.0, rng.integers(-20, 20, (4, 1)))
    assert np.array_equal(oracle.mx_dequantize(*oracle.mx_quantize(exact)), exact)
    x = rng.standard_normal((8, 512)) * 3
    codes, scales = oracle.mx_quantize(x)
    X = np.repeat(oracle.e8m0_value(scales), 32, axis=1)
    err = np.abs(oracle.mx_dequantize(codes, scales) - x)
    sat = np.abs(x) / X > 6
    assert np.all(err[~sat] <= X[~sat]) and np.all(err[sat] <= 2 * X[sat])
    assert np.all((X == 2.0 ** np.round(np.log2(X))))  # scales are powers of two


def test_product_brute_force():
    rng = np.random.default_rng(93)
    a = rng.standard_normal((3, 64))
    w = rng.standard_normal((5, 64))
    got = oracle.mx_gemm(a, w)
    ca, sa = oracle.mx_quantize(a)
    cw, sw = oracle.mx_quantize(w)
    da = [[Fraction(float(v)) for v in row] for row in oracle.mx_dequantize(ca, sa)]
    dw = [[Fraction(float(v)) for v in row] for row in oracle.mx_dequantize(cw, sw)]
    for i in range(3):
        for j in range(5):
            exact = sum(p * q for p, q in zip(da[i], dw[j]))
            assert abs(Fraction(got[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.mx_quantize(np.zeros((2, 48)))
    with pytest.raises(ValueError):
        oracle.mx_quantize(np.full((1, 32), np.inf))
