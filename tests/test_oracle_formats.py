"""Pins for oracle/formats.py: every codec is checked against something other than itself
(a hand-derived table, library casts, or an exact brute-force search over all values)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_e2m1_golden():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_codes.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c), float(v)))
    return rows


def test_e2m1_table_matches_golden():
    rows = _load_e2m1_golden()
    assert [c for c, _ in rows] == list(range(16))
    got = F.e2m1_decode(np.arange(16))
    for c, v in rows:
        assert got[c] == v and np.signbit(got[c]) == np.signbit(v), c


def test_e2m1_value_set():
    # The eight magnitudes of E2M1 with bias 1: {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
    mags = sorted(set(np.abs(F.e2m1_decode(np.arange(16))).tolist()))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_decode_all_bytes_vs_torch():
    b = np.array([x for x in range(256) if (x & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(b)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert F.e4m3_decode(np.array([0x7E]))[0] == 448.0


def test_e4m3_encode_roundtrip_all_bytes():
    b = np.arange(0, 0x7F, dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(b)), b)


def _grid(fmt):
    """All finite non-negative values of a format with their bit patterns, from libraries."""
    if fmt is F.E2M1:
        return np.abs(F.e2m1_decode(np.arange(8))), np.arange(8)
    if fmt is F.E4M3:
        b = np.arange(0, 0x7F, dtype=np.uint8)
        v = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return v, b.astype(np.int64)
    if fmt is F.FP16:
        b = np.arange(0, 0x7C00, dtype=np.uint16)
        return b.view(np.float16).astype(np.float64), b.astype(np.int64)
    raise ValueError


def _brute_round(t: Fraction, vals, bits, vmax):
    """Nearest grid value to the exact rational t, ties to the even bit pattern,
    saturating to the largest finite value."""
    if t >= Fraction(vmax):
        return float(vmax)
    i = int(np.searchsorted(vals, float(t)))
    best = None
    for j in (i - 1, i, i + 1):
        if 0 <= j < len(vals):
            d = abs(Fraction(vals[j]) - t)
            key = (d, int(bits[j]) & 1)
            if best is None or key < best[0]:
                best = (key, vals[j])
    return float(best[1])


@pytest.mark.parametrize("fmt", [F.E2M1, F.E4M3, F.FP16])
def test_round_to_grid_vs_bruteforce(fmt):
    vals, bits = _grid(fmt)
    rng = np.random.default_rng(123)
    # midpoints of neighbouring values (exact ties), points just off them, random points
    mids = (vals[:-1] + vals[1:]) / 2
    eps = np.abs(mids) * 2.0 ** -30
    cand = np.concatenate([vals, mids, mids + eps, mids - eps,
                           rng.uniform(0, vals[-1] * 1.2, 2000),
                           np.exp(rng.uniform(np.log(vals[1] / 4), np.log(vals[-1] * 1.1), 2000)),
                           [vals[-1] * 1.03, vals[-1] * 1.1, vals[-1] * 5]])
    cand = cand[cand >= 0]
    if fmt is F.FP16 and len(cand) > 4000:
        cand = np.concatenate([cand[:800], rng.choice(cand, 3000, replace=False)])
    got = F.round_to_grid(cand, fmt)
    for t, g in zip(cand, got):
        assert g == _brute_round(Fraction(float(t)), vals, bits, vals[-1]), (fmt.name, t)


def test_round_to_grid_exact_rational_quotients():
    """fl64(a/d) followed by rounding equals rounding the exact rational a/d, for the
    divisors the quantizer uses (2688 = 6*448, 6*M, 200704 = 448*448)."""
    rng = np.random.default_rng(7)
    vals, bits = _grid(F.FP16)
    for _ in range(3000):
        a = float(np.float32(rng.standard_normal() * 10 ** rng.uniform(-6, 3)))
        a = abs(a)
        got = F.round_to_grid(np.array([a / 2688.0]), F.FP16)[0]
        assert got == _brute_round(Fraction(a) / 2688, vals, bits, 65504.0)
    vals8, bits8 = _grid(F.E4M3)
    for _ in range(3000):
        a = abs(float(np.float32(rng.standard_normal())))
        M = float(np.float16(abs(rng.standard_normal()) * 1e-3 + 1e-6))
        if M == 0:
            continue
        got = F.round_to_grid(np.array([a / (6 * M)]), F.E4M3)[0]
        assert got == _brute_round(Fraction(a) / (6 * Fraction(M)), vals8, bits8, 448.0)


def test_e4m3_rounding_vs_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(0, 448, 20000), np.exp(rng.uniform(-12, 6, 20000))])
    x = np.minimum(x, 448.0).astype(np.float32).astype(np.float64)  # torch's cast does not saturate
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.round_to_grid(x, F.E4M3), ref)


def test_fp16_rounding_vs_numpy_cast():
    rng = np.random.default_rng(6)
    x = np.concatenate([np.exp(rng.uniform(-20, 11, 50000)), rng.uniform(0, 65504, 5000)])
    ref = x.astype(np.float16).astype(np.float64)   # numpy rounds float64->half to nearest even
    assert np.array_equal(F.round_to_grid(x, F.FP16), ref)


def test_bf16_rounding_vs_torch_cast():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(50000) * 10 ** rng.uniform(-30, 30, 50000),
                        rng.standard_normal(1000)]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_round(x), ref)
    assert np.array_equal(F.bf16_bits(ref),
                          torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
                          .view(torch.int16).numpy().view(np.uint16))


def test_fp16_bits_vs_numpy():
    v = np.array([2.0 ** -24, 2.0 ** -14, 2.0 ** -8, 1.0, 65504.0, 2.2351741790771484e-05])
    assert np.array_equal(F.fp16_bits(v), v.astype(np.float16).view(np.uint16))
    assert F.fp16_bits(np.array([2.0 ** -8]))[0] == 0x1C00
