"""MX-native FP4 (E2M1 elements, one E8M0 power-of-two scale per 32 elements) and its
matrix product, on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is not the pages' two-level format. It is the block format that CDNA4's scaled FP4
matrix instructions consume natively, kept beside the pages' format so that the speed of
that path and its accuracy against the two-level format can be measured. Reading used
(the public OCP microscaling definition for MXFP4):
  * blocks are 32 consecutive elements of a row (along K);
  * the block's scale is X = 2^e with e = floor(log2(max |x|)) - 2 (2 being the exponent of
    E2M1's largest value, 6 = 1.5 * 2^2), clamped to [-127, 127]; stored as the E8M0 byte
    e + 127; an all-zero block stores e = -127 (byte 0);
  * each element is x / X rounded to the nearest E2M1 value, ties to even, saturating at
    +-6 (block maxima in (6X, 8X) clamp to 6X); the sign bit is kept for negative values
    that round to 0 (code 0x8), as in the two-level codec;
  * dequantized value = code value * X; the product is C = A_hat . W_hat^T, float64 here.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1, round_to_grid

__all__ = ["MX_BLOCK", "e8m0_value", "mx_quantize", "mx_dequantize", "mx_gemm"]

MX_BLOCK = 32


def e8m0_value(byte):
    """E8M0 scale byte -> 2^(byte - 127) (255 is NaN and never produced)."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0, exactly (frexp gives a = f * 2^e with f in [0.5, 1))."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


def mx_quantize(x):
    """x [R, K] (K % 32 == 0) -> (codes uint8 [R, K] as 4-bit E2M1 codes, scales uint8
    [R, K/32] E8M0 bytes)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("x must be [rows, k] with k % 32 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    R, K = x.shape
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.clip(_floor_log2(amax[nz]) - 2, -127, 127)
    X = np.ldexp(1.0, e)[:, :, None]
    q = blocks / X  # exact: division by a power of two
    mag = np.minimum(round_to_grid(np.abs(q), E2M1), 6.0)  # RNE, then saturate
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = np.zeros(mag.shape, dtype=np.uint8)
    for c, v in enumerate(grid):
        codes[mag == v] = c
    codes |= np.signbit(q).astype(np.uint8) << 3  # sign kept, also for values rounding to 0
    return codes.reshape(R, K), (e + 127).astype(np.uint8)


def mx_dequantize(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    X = np.repeat(e8m0_value(scales), MX_BLOCK, axis=1)
    return val * X


def mx_gemm(a, w) -> np.ndarray:
    """C = mx(A) . mx(W)^T in float64 for A [M, K], W [N, K]."""
    ca, sa = mx_quantize(a)
    cw, sw = mx_quantize(w)
    return mx_dequantize(ca, sa) @ mx_dequantize(cw, sw).T
