"""Number formats used by two-level block-scaled FP4, written out from their definitions.

TEST INFRASTRUCTURE ONLY. This package is the slow CPU oracle that the HIP path is
checked against. Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it; the product path never does.

Sources
-------
* "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200",
  section "The Mathematical Breakthrough of Microscopic FP4 Scaling": elements are
  E2M1 (one sign bit, two exponent bits, one mantissa bit); micro-scales are FP8;
  macro-scales are FP16.
* Readings where that page is silent (kept in one place so they can be audited):
  - E2M1 has exponent bias 1, a subnormal step of 0.5 at exponent field 0, no Inf/NaN,
    so the magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; conversion saturates at 6.
  - the FP8 micro-scale is OCP E4M3 (bias 7, max 448, 0x7F/0xFF are NaN and never
    produced).
  - every conversion is round-to-nearest, ties to the even significand, with
    saturation to the largest finite value (never Inf/NaN).

Everything here is float64 numpy; all values handled are exactly representable in
float64, so the only rounding is the explicit one in ``round_to_grid``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "FloatFormat", "E2M1", "E4M3", "FP16", "BF16",
    "round_to_grid", "e2m1_decode", "e2m1_encode_magnitude",
    "e4m3_decode", "e4m3_encode", "fp16_bits", "fp16_from_bits",
    "bf16_round", "bf16_bits",
]


class FloatFormat:
    """A binary floating-point format described by its significand width and range.

    ``mant_bits``  fraction bits of a normal number (the leading 1 is implicit)
    ``emin``       exponent of the smallest normal number; below it the spacing is
                   fixed at 2**(emin - mant_bits) (gradual underflow)
    ``max_finite`` largest finite magnitude; rounding saturates here
    """

    def __init__(self, name: str, mant_bits: int, emin: int, max_finite: float):
        self.name = name
        self.mant_bits = mant_bits
        self.emin = emin
        self.max_finite = float(max_finite)

    def __repr__(self) -> str:  # pragma: no cover - debugging aid
        return f"FloatFormat({self.name})"


# E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit. Normal exponents 0..2 -> 1..6.
E2M1 = FloatFormat("e2m1", mant_bits=1, emin=0, max_finite=6.0)
# OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 15 with
# mantissa 7 is NaN, so the largest finite value is 1.75 * 2**8 = 448.
E4M3 = FloatFormat("e4m3", mant_bits=3, emin=-6, max_finite=448.0)
# IEEE binary16.
FP16 = FloatFormat("fp16", mant_bits=10, emin=-14, max_finite=65504.0)
# bfloat16 (8 exponent bits, 7 fraction bits).
BF16 = FloatFormat("bf16", mant_bits=7, emin=-126, max_finite=float.fromhex("0x1.fep127"))


def round_to_grid(t, fmt: FloatFormat) -> np.ndarray:
    """Round non-negative reals ``t`` to the nearest value of ``fmt``.

    Ties go to the value whose significand is even; results above ``fmt.max_finite``
    saturate to it.  ``t`` must be finite and >= 0 (signs are handled by callers).

    The grid spacing at ``t`` is 2**q with q = max(floor(log2 t), emin) - mant_bits;
    ``t / 2**q`` is exact in float64 (a power-of-two scaling) and ``np.rint`` rounds
    half to even, which is exactly ties-to-even on the significand.
    """
    t = np.asarray(t, dtype=np.float64)
    if np.any(~np.isfinite(t)) or np.any(t < 0):
        raise ValueError("round_to_grid expects finite, non-negative input")
    out = np.zeros_like(t)
    nz = t > 0
    tn = t[nz]
    _, e2 = np.frexp(tn)            # tn = m * 2**e2 with m in [0.5, 1)
    floor_log2 = e2 - 1
    q = np.maximum(floor_log2, fmt.emin) - fmt.mant_bits
    n = np.rint(np.ldexp(tn, -q))   # integer count of grid steps, half-to-even
    out[nz] = np.minimum(np.ldexp(n, q), fmt.max_finite)
    return out


# --- E2M1 --------------------------------------------------------------------------

_E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes: bit 3 is the sign, bits 2..1 the exponent field e,
    bit 0 the mantissa m.  e == 0 -> m * 0.5 (subnormal); else 2**(e-1) * (1 + m/2)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes are 4-bit")
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(c & 8, -mag, mag)


def e2m1_encode_magnitude(v) -> np.ndarray:
    """3-bit magnitude code of an E2M1 value already on the grid (|v| in the table)."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.searchsorted(_E2M1_MAGNITUDES, v)
    idx = np.minimum(idx, 7)
    if not np.all(_E2M1_MAGNITUDES[idx] == v):
        raise ValueError("value is not an E2M1 magnitude")
    return idx.astype(np.uint8)


# --- E4M3 --------------------------------------------------------------------------

def e4m3_decode(byte) -> np.ndarray:
    """Value of OCP E4M3 bytes: s = bit 7, e = bits 6..3, m = bits 2..0.
    e == 0 -> m * 2**-9; else 2**(e-7) * (1 + m/8).  0x7F/0xFF (NaN) are rejected."""
    b = np.asarray(byte).astype(np.int64)
    if np.any((b & 0x7F) == 0x7F):
        raise ValueError("E4M3 NaN encoding")
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(b & 0x80, -mag, mag)


def e4m3_encode(v) -> np.ndarray:
    """Byte of non-negative values that are already on the E4M3 grid."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    nz = v > 0
    x = v[nz]
    _, e2 = np.frexp(x)
    e = e2 - 1
    normal = e >= -6
    byte = np.where(normal,
                    ((e + 7) << 3) + np.rint((np.ldexp(x, -np.where(normal, e, 0)) - 1.0) * 8),
                    np.rint(np.ldexp(x, 9)))
    out[nz] = byte.astype(np.uint8)
    if not np.all(e4m3_decode(out) == v):
        raise ValueError("value is not on the E4M3 grid")
    return out


# --- FP16 / BF16 -------------------------------------------------------------------

def fp16_bits(v) -> np.ndarray:
    """IEEE binary16 bit pattern of values that are already on the FP16 grid."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    if not np.all(h.astype(np.float64) == v):
        raise ValueError("value is not on the FP16 grid")
    return h.view(np.uint16)


def fp16_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round signed reals to bfloat16 (ties to even, saturating at the largest finite)."""
    x = np.asarray(x, dtype=np.float64)
    mag = round_to_grid(np.abs(x), BF16)
    return np.where(np.signbit(x), -mag, mag)


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit pattern of values already on the bf16 grid (sign kept for -0.0)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.all(f.astype(np.float64) == x):
        raise ValueError("value is not representable")
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value is not on the bf16 grid")
    return (u >> 16).astype(np.uint16)
