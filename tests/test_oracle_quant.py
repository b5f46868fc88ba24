"""Pins for oracle/quant.py: the hand-worked group, exact round-trip of representable
values, the per-element error bound, invariants, and an exact-rational brute force."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F
from oracle.quant import quantize, dequantize, unpack_e2m1, pack_e2m1, element_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_worked_group():
    macro, blocks = None, []
    cur = {}
    with open(os.path.join(GOLDEN, "worked_group.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "macro":
                macro = int(vals[0], 16)
            elif key == "x":
                cur = {"x": [float(v) for v in vals]}
            elif key == "codes":
                cur["codes"] = [int(v) for v in vals]
            elif key == "mu":
                cur["mu"] = int(vals[0], 16)
                blocks.append(cur)
    return macro, blocks


def test_worked_group_golden():
    macro, blocks = _load_worked_group()
    x = np.zeros((1, 256))
    want_codes = np.zeros(256, dtype=np.uint8)
    want_mu = np.zeros(16, dtype=np.uint8)
    for b, blk in enumerate(blocks):
        x[0, 16 * b:16 * b + 16] = blk["x"]
        want_codes[16 * b:16 * b + 16] = blk["codes"]
        want_mu[b] = blk["mu"]
    q = quantize(x)
    assert q.macro[0, 0] == macro
    assert np.array_equal(q.micro[0], want_mu)
    assert np.array_equal(unpack_e2m1(q.codes)[0], want_codes)
    # packed byte order: even element in the low nibble
    assert q.codes[0, 0] == 0x10 and q.codes[0, 7] == 0xFE


def test_pack_order():
    c = np.array([[1, 2, 15, 0]], dtype=np.uint8)
    assert np.array_equal(pack_e2m1(c), np.array([[0x21, 0x0F]], dtype=np.uint8))
    assert np.array_equal(unpack_e2m1(pack_e2m1(c)), c)


def _representable_family(rng, rows, groups, elem="e2m1"):
    """x = value(code) * mu * M, with at least one max-magnitude element per block and
    the largest micro-scale (448) in every group, so quantize must return (code, mu, M)."""
    K = 256 * groups
    emax_code = 7 if elem == "e2m1" else 0x7E
    if elem == "e2m1":
        codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
        codes[:, ::16] = np.where(rng.random((rows, K // 16)) < 0.5, 7, 15)
        v = F.e2m1_decode(codes)
    else:
        codes = rng.integers(0, 0x7F, (rows, K)).astype(np.uint8)
        codes |= (rng.integers(0, 2, (rows, K)) << 7).astype(np.uint8)
        codes[:, ::16] = np.where(rng.random((rows, K // 16)) < 0.5, 0x7E, 0xFE)
        v = F.e4m3_decode(codes)
    mu_b = rng.integers(1, 0x7F, (rows, K // 16)).astype(np.uint8)
    mu_b[:, ::16] = 0x7E                              # 448 somewhere in each group
    mu = F.e4m3_decode(mu_b)
    # normal fp16 macro-scales within [2^-14, 2^5]
    Mv = (np.float16(1.0) * np.exp2(rng.integers(-14, 5, (rows, groups)))
          * (1 + rng.integers(0, 1024, (rows, groups)) / 1024.0))
    M = Mv.astype(np.float16).astype(np.float64)
    x = v * np.repeat(mu, 16, axis=1) * np.repeat(M, 256, axis=1)
    return x, codes, mu_b, M


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_roundtrip_representable(elem):
    rng = np.random.default_rng(11)
    x, codes, mu_b, M = _representable_family(rng, 6, 3, elem)
    assert np.all(np.abs(x) < 3.4e38)
    q = quantize(x, elem)
    got_codes = unpack_e2m1(q.codes) if elem == "e2m1" else q.codes
    # codes come back exactly, including the sign of zero (-0.0 inputs give the
    # negative-zero code because every block here has a nonzero scale)
    assert np.array_equal(got_codes, codes)
    assert np.array_equal(q.micro, mu_b)
    assert np.array_equal(F.fp16_from_bits(q.macro), M)
    xh = dequantize(q)
    assert np.array_equal(xh, x)
    assert np.array_equal(np.signbit(xh), np.signbit(x))


def test_error_bound_per_element():
    """|x - x_hat| <= s * h(|x|/s) with h = 1/4 (q<=2), 1/2 (q<=4), 1 (q<=6), q-6 above."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 1024)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    x[:, rng.choice(1024, 8, replace=False)] *= 100.0
    q = quantize(x)
    xh = dequantize(q)
    s = np.repeat(F.e4m3_decode(q.micro) * np.repeat(F.fp16_from_bits(q.macro), 16, axis=1),
                  16, axis=1)
    r = np.abs(x) / s
    h = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, np.where(r <= 6, 1.0, r - 6)))
    slack = 1e-12 * np.abs(x)  # float64 rounding of the test's own subtraction
    assert np.all(np.abs(x - xh) <= s * h + slack)
    # saturation stays small under max-abs scale selection
    assert r.max() <= 6.4
    assert np.all(np.abs(x - xh) <= np.maximum(s / 4, np.abs(x) / 4) + slack)


def test_error_magnitude_normal_data():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((256, 1024))
    rel = np.linalg.norm(dequantize(quantize(x)) - x) / np.linalg.norm(x)
    assert 0.07 < rel < 0.12
    rel8 = np.linalg.norm(dequantize(quantize(x, "e4m3")) - x) / np.linalg.norm(x)
    assert 0.01 < rel8 < 0.04


def test_invariants():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((4, 512))
    q = quantize(x)
    # sign symmetry: negating x flips bit 3 of every nonzero-scale code, nothing else
    qn = quantize(-x)
    assert np.array_equal(unpack_e2m1(qn.codes), unpack_e2m1(q.codes) ^ 8)
    assert np.array_equal(qn.micro, q.micro) and np.array_equal(qn.macro, q.macro)
    # power-of-two equivariance (macro stays normal and unclamped)
    for j in (-3, 1, 4):
        qj = quantize(x * 2.0 ** j)
        assert np.array_equal(qj.codes, q.codes) and np.array_equal(qj.micro, q.micro)
        assert np.array_equal(F.fp16_from_bits(qj.macro), F.fp16_from_bits(q.macro) * 2.0 ** j)
    # a permutation inside a block permutes that block's codes only
    perm = rng.permutation(16)
    xp = x.copy()
    xp[:, 32:48] = x[:, 32:48][:, perm]
    cp, c = unpack_e2m1(quantize(xp).codes), unpack_e2m1(q.codes)
    assert np.array_equal(cp[:, 32:48], c[:, 32:48][:, perm])
    assert np.array_equal(np.delete(cp, range(32, 48), 1), np.delete(c, range(32, 48), 1))
    # groups are independent: changing group 1 leaves group 0 untouched
    x2 = x.copy()
    x2[:, 256:] *= 1000.0
    q2 = quantize(x2)
    assert np.array_equal(q2.codes[:, :128], q.codes[:, :128])
    assert np.array_equal(q2.micro[:, :16], q.micro[:, :16])
    assert np.array_equal(q2.macro[:, 0], q.macro[:, 0])
    # rows are independent
    assert np.array_equal(quantize(x[2:3]).codes, q.codes[2:3])


def test_block_size_is_16():
    """Changing one element moves at most its own 16-block's micro-scale."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((1, 256))
    x[0, 0] = 3.0  # group max stays fixed
    base = quantize(x)
    y = x.copy()
    y[0, 37] = 2.9  # block 2 (elements 32..47)
    got = quantize(y)
    diff = np.nonzero(got.micro[0] != base.micro[0])[0]
    assert set(diff.tolist()) <= {2}
    assert got.macro[0, 0] == base.macro[0, 0]


def test_zero_and_tiny_edges():
    x = np.zeros((2, 256))
    x[1, 5] = -0.0
    q = quantize(x)
    assert not q.codes.any() and not q.micro.any() and not q.macro.any()
    # a group whose max is below the smallest macro-scale clamps M to 2^-24
    t = np.zeros((1, 256))
    t[0, 0] = 1e-12
    t[0, 17] = -1e-13
    qt = quantize(t)
    assert F.fp16_from_bits(qt.macro)[0, 0] == 2.0 ** -24
    # a block far below its group's max gets micro-scale 0 and codes 0
    u = np.zeros((1, 256))
    u[0, 0] = 1000.0
    u[0, 20] = 1e-6
    u[0, 21] = -1e-6
    qu = quantize(u)
    assert qu.micro[0, 1] == 0 and not unpack_e2m1(qu.codes)[0, 16:32].any()
    # inside a block with a nonzero scale, -0.0 and tiny negatives keep the sign bit
    v = np.zeros((1, 256))
    v[0, 0] = 6.0
    v[0, 1] = -0.0
    v[0, 2] = -1e-9
    cv = unpack_e2m1(quantize(v).codes)[0]
    assert cv[1] == 8 and cv[2] == 8 and cv[3] == 0
    # huge values saturate M at 65504 and stay finite
    w = np.full((1, 256), 3e38)
    qw = quantize(w)
    assert F.fp16_from_bits(qw.macro)[0, 0] == 65504.0
    assert np.all(np.isfinite(dequantize(qw)))
    with pytest.raises(ValueError):
        quantize(np.full((1, 256), np.inf))
    with pytest.raises(ValueError):
        quantize(np.zeros((1, 100)))


def _nearest(t: Fraction, grid):
    best = None
    for i, g in enumerate(grid):
        key = (abs(Fraction(g) - t), i & 1)
        if best is None or key < best[0]:
            best = (key, g)
    return best[1]


def _exact_quantize_group(xrow, emax, elem_grid):
    """Brute force over exact rationals for one 256-group of a row."""
    e4 = [float(v) for v in F.e4m3_decode(np.arange(0, 0x7F))]
    h = [float(v) for v in np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)]
    xs = [Fraction(float(v)) for v in xrow]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return 0.0, [0.0] * 16, [0.0] * 256
    t = amax / (emax * 448)
    M = 65504.0 if t >= 65504 else _nearest(t, h)
    M = min(max(M, 2.0 ** -24), 65504.0)
    mus, vals = [], []
    for b in range(16):
        blk = xs[16 * b:16 * b + 16]
        r = max(abs(v) for v in blk) / (emax * Fraction(M))
        mu = 448.0 if r >= 448 else _nearest(r, e4)
        mus.append(mu)
        s = Fraction(mu) * Fraction(M)
        for v in blk:
            if s == 0:
                vals.append(0.0)
                continue
            qv = abs(v) / s
            mag = elem_grid[-1] if qv >= elem_grid[-1] else _nearest(qv, elem_grid)
            vals.append(-mag if v < 0 else mag)
    return M, mus, vals


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_quantize_vs_exact_bruteforce(elem):
    """Tiny adversarial inputs: points exactly on and next to every tie point t*s."""
    rng = np.random.default_rng(16)
    emax = 6.0 if elem == "e2m1" else 448.0
    elem_grid = ([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0] if elem == "e2m1"
                 else [float(v) for v in F.e4m3_decode(np.arange(0, 0x7F))])
    rows = []
    for trial in range(6):
        x = rng.standard_normal(256).astype(np.float32).astype(np.float64)
        x *= 10.0 ** rng.integers(-4, 4)
        q = quantize(x[None, :], elem)
        s = np.repeat(F.e4m3_decode(q.micro[0]) * F.fp16_from_bits(q.macro[0, 0]), 16)
        ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) if elem == "e2m1" else \
            np.array(elem_grid[:-1]) + np.diff(elem_grid) / 2
        pick = rng.choice(len(ties), 256)
        nudge = rng.choice([-1, 0, 0, 1], 256) * 2.0 ** -22
        y = ties[pick] * s * (1 + nudge) * np.sign(x)
        y = y.astype(np.float32).astype(np.float64)
        # keep every block's largest element (so s is unchanged) and stay below it
        bmax = np.repeat(np.abs(x).reshape(16, 16).max(1), 16)
        is_max = np.zeros(256, bool)
        is_max[np.arange(16) * 16 + np.abs(x).reshape(16, 16).argmax(1)] = True
        keep = (~is_max) & (np.abs(y) < bmax)
        x[keep] = y[keep]
        rows.append(x)
    x = np.array(rows)
    q = quantize(x, elem)
    got_vals = element_values(q)
    for r in range(x.shape[0]):
        M, mus, vals = _exact_quantize_group(x[r], emax, elem_grid)
        assert F.fp16_from_bits(q.macro[r, 0]) == M
        assert np.array_equal(F.e4m3_decode(q.micro[r]), np.array(mus))
        assert np.array_equal(got_vals[r], np.array(vals)), r


def test_micro_scale_ties_vs_exact_bruteforce():
    """Block maxima placed exactly on (and 2^-22 around) midpoints between neighbouring
    E4M3 micro-scales; the group max pins M = 2^-8 so amax_b / (6 M) is the tie itself."""
    e4 = F.e4m3_decode(np.arange(0, 0x7F))
    mids = (e4[:-1] + e4[1:]) / 2
    rng = np.random.default_rng(17)
    emax, elem_grid = 6.0, [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rows = []
    for trial in range(8):
        x = np.zeros(256)
        x[0] = 10.5                       # 10.5 / 2688 = 2^-8 exactly
        for b in range(1, 16):
            t = mids[rng.integers(8, len(mids))] * (1 + rng.choice([-1, 0, 1]) * 2.0 ** -22)
            amax = np.float64(np.float32(t * 6 * 2.0 ** -8))
            x[16 * b] = amax * rng.choice([-1, 1])
            x[16 * b + 1:16 * b + 16] = rng.uniform(-1, 1, 15) * amax
        rows.append(x.astype(np.float32).astype(np.float64))
    x = np.array(rows)
    q = quantize(x)
    for r in range(x.shape[0]):
        M, mus, vals = _exact_quantize_group(x[r], emax, elem_grid)
        assert F.fp16_from_bits(q.macro[r, 0]) == M == 2.0 ** -8
        assert np.array_equal(F.e4m3_decode(q.micro[r]), np.array(mus)), r
        assert np.array_equal(element_values(q)[r], np.array(vals)), r
