"""Pins of the sensitive-layer (W8A8) and static-activation-scale oracle functions against
the pinned dynamic quantizer, hand-derived values, saturation, exact-rational products and
the policy table."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_static_with_each_rows_own_macro_is_dynamic():
    rng = np.random.default_rng(111)
    x = rng.standard_normal((5, 512)) * 3
    x[:, 7] *= 40
    for elem in ("e2m1", "e4m3"):
        for r in range(5):
            d = oracle.quantize(x[r:r + 1], elem)
            s = oracle.quantize_static(x[r:r + 1], d.macro[0], elem)
            assert np.array_equal(d.codes, s.codes) and np.array_equal(d.micro, s.micro)
            assert np.array_equal(d.macro, s.macro)


def test_calibration_is_the_dynamic_rule_on_the_group_maximum():
    rng = np.random.default_rng(112)
    x = rng.standard_normal((6, 768))
    x[4, 300] = 90.0  # group 1's maximum sits in row 4
    x[2, 700] = -55.0  # group 2's in row 2
    x[0, 10] = 8.0  # group 0's in row 0
    for elem in ("e2m1", "e4m3"):
        cal = oracle.calibrate_macro(x, elem)
        assert cal[0] == oracle.quantize(x[0:1], elem).macro[0, 0]
        assert cal[1] == oracle.quantize(x[4:5], elem).macro[0, 1]
        assert cal[2] == oracle.quantize(x[2:3], elem).macro[0, 2]


def test_hand_derived_static_values_and_saturation():
    # M = 2^-10 (FP16 bits 0x1400); a block whose max is 1.5: mu = RNE_E4M3(1.5 / (6 * 2^-10))
    # = RNE(256) = 256 (E4M3 0x78); s = 0.25: x = 0.6 -> 2.4 -> 2 (code 4), x = -1.5 -> -6
    # (code 0xF)
    x = np.zeros((1, 256))
    x[0, 0], x[0, 1] = 0.6, -1.5
    q = oracle.quantize_static(x, [0x1400], "e2m1")
    codes4 = oracle.unpack_e2m1(q.codes)
    assert q.micro[0, 0] == 0x78 and codes4[0, 0] == 4 and codes4[0, 1] == 0xF
    # 1000x past the calibrated range: micro-scale saturates at 448 (0x7E), elements at 6
    big = np.full((1, 256), 1e3)
    big[0, 1::2] *= -1
    qb = oracle.quantize_static(big, [0x1400], "e2m1")
    assert np.all(qb.micro == 0x7E)
    assert np.all(np.abs(oracle.dequantize(qb)) == 6 * 448 * 2.0 ** -10)


def test_w8a8_product_exact_rational():
    rng = np.random.default_rng(113)
    a = rng.standard_normal((3, 256))
    w = rng.standard_normal((4, 256)) * 0.02
    w8 = oracle.quantize(w, "e4m3")
    got = oracle.gemm_w8a8(a, w8)
    da = oracle.activation_values(a, oracle.A8)
    dw = oracle.dequantize(w8)
    for i in range(3):
        for j in range(4):
            exact = sum(Fraction(float(p)) * Fraction(float(q)) for p, q in zip(da[i], dw[j]))
            assert abs(Fraction(got[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 45)
    with pytest.raises(ValueError):
        oracle.gemm_w8a8(a, oracle.quantize(w, "e2m1"))


def test_w8_round_trip_of_representable_weights():
    # w = e * mu * 2^-10 with e, mu E4M3 values, every block holding one e = 448 and every
    # group one block with mu = 448: group max 448 * 448 * 2^-10 -> M = 2^-10 exactly, block
    # max 448 * mu * 2^-10 -> that mu exactly, elements e exactly: the codec is lossless
    elems = np.array([0.0, 0.015625, 0.5, 1.0, 1.75, 3.0, 96.0, 448.0])
    mus = np.array([0.125, 1.0, 2.5, 13.0, 448.0])
    rng = np.random.default_rng(114)
    e = rng.choice(elems, (3, 512)) * rng.choice([-1, 1], (3, 512))
    e[:, ::16] = 448.0
    mu = rng.choice(mus, (3, 32))
    mu[:, ::16] = 448.0
    w = e * np.repeat(mu, 16, axis=1) * 2.0 ** -10
    q = oracle.quantize(w, "e4m3")
    assert np.all(q.macro == 0x1400)
    assert np.array_equal(oracle.dequantize(q), w)
    assert np.array_equal(oracle.dequantize(oracle.quantize_static(w, [0x1400, 0x1400], "e4m3")), w)


def test_policy_table():
    assert oracle.policy_select_ext(oracle.POLICY_SENSITIVE_W8, True) == oracle.W8A8
    assert oracle.policy_select_ext(oracle.POLICY_SENSITIVE_W8, False) == oracle.A4
    assert oracle.policy_select_ext(oracle.POLICY_STATIC, True) == oracle.A8S
    assert oracle.policy_select_ext(oracle.POLICY_STATIC, False) == oracle.A4S
    with pytest.raises(ValueError):
        oracle.policy_select_ext(7, True)


def test_static_product_matches_its_definition_on_a_tiny_case():
    rng = np.random.default_rng(115)
    a = rng.standard_normal((4, 256))
    w = oracle.quantize(rng.standard_normal((3, 256)) * 0.02)
    cal = oracle.calibrate_macro(a * 1.5, "e2m1")
    got = oracle.gemm_static(a, w, oracle.A4S, cal)
    av = oracle.dequantize(oracle.quantize_static(a, cal, "e2m1"))
    for i in range(4):
        for j in range(3):
            exact = sum(Fraction(float(p)) * Fraction(float(q))
                        for p, q in zip(av[i], oracle.dequantize(w)[j]))
            assert abs(Fraction(got[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 300)
