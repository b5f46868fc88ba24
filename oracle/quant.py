"""Two-level block-scaled quantization, step by step, on the CPU (float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200",
section "The Mathematical Breakthrough of Microscopic FP4 Scaling", item 2: a tensor is
cut into micro-vectors of 16 consecutive elements, each with its own FP8 scale, and
each run of 16 micro-vectors (256 elements) shares one FP16 macro-scale.

Readings where the page is silent (each is also listed in the design notes):
* blocks run along the last (contiguous, reduction) axis of a row; a 256-group is 16
  consecutive blocks of the same row;
* scale selection is max-abs based: the group max maps onto (element max) * 448, the
  block max onto the element max;
      M_g  = RNE_fp16(amax_g / (emax * 448)), kept in [2**-24, 65504] when amax_g > 0
      mu_b = RNE_e4m3(amax_b / (emax * M_g))
      code = RNE_elem(|x| / (mu_b * M_g)), sign copied from x
  where emax = 6 for E2M1 elements and 448 for E4M3 elements (the 8-bit activation
  variant used by W4A8 layers, from "llama.cpp Put Precision Policy Inside the Model",
  section "One model can need more than one precision");
* an all-zero group gets M = 0, mu = 0 and code 0; a block whose scale is 0 gets code 0;
  otherwise the sign bit of x is kept, so -0.0 and tiny negatives give the "negative
  zero" code (0x8 for E2M1, 0x80 for E4M3);
* inputs must be finite.

Storage (row-major, "canonical"): E2M1 codes two per byte with the even element in the
low nibble; E4M3 codes one per byte; micro-scales one E4M3 byte per block; macro-scales
the FP16 bit pattern per group.
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1, E4M3, FP16, round_to_grid, e2m1_decode, e2m1_encode_magnitude,
                      e4m3_decode, e4m3_encode, fp16_bits, fp16_from_bits)

BLOCK = 16
GROUP = 256
E4M3_MAX = 448.0
ELEM_MAX = {"e2m1": 6.0, "e4m3": 448.0}
M_MIN = 2.0 ** -24
M_MAX = 65504.0

__all__ = ["quantize", "dequantize", "unpack_e2m1", "pack_e2m1", "QuantizedTensor",
           "BLOCK", "GROUP"]


class QuantizedTensor:
    """codes: uint8 [R, K/2] (e2m1, packed) or [R, K] (e4m3); micro: uint8 [R, K/16];
    macro: uint16 [R, K/256] (FP16 bits)."""

    def __init__(self, codes, micro, macro, elem: str, k: int):
        self.codes = codes
        self.micro = micro
        self.macro = macro
        self.elem = elem
        self.k = k

    @property
    def rows(self) -> int:
        return self.micro.shape[0]


def pack_e2m1(codes4: np.ndarray) -> np.ndarray:
    """[R, K] 4-bit codes -> [R, K/2] bytes, even element in the low nibble."""
    c = codes4.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] 4-bit codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def _check_input(x) -> np.ndarray:
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] array")
    if x.shape[1] % GROUP:
        raise ValueError("K must be a multiple of 256")
    x = x.astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    return x


def quantize(x, elem: str = "e2m1") -> QuantizedTensor:
    """Quantize each row of ``x`` [R, K] (K % 256 == 0) with two-level scaling."""
    if elem not in ELEM_MAX:
        raise ValueError(elem)
    x = _check_input(x)
    R, K = x.shape
    emax = ELEM_MAX[elem]
    ax = np.abs(x)

    # Step 1: group and block maxima of |x| (exact).
    amax_g = ax.reshape(R, K // GROUP, GROUP).max(axis=2)
    amax_b = ax.reshape(R, K // BLOCK, BLOCK).max(axis=2)

    # Step 2: FP16 macro-scale per 256-group.
    M = round_to_grid(amax_g / (emax * E4M3_MAX), FP16)
    M = np.where(amax_g > 0, np.clip(M, M_MIN, M_MAX), 0.0)

    # Step 3: E4M3 micro-scale per 16-block, relative to its group's macro-scale.
    M_of_block = np.repeat(M, GROUP // BLOCK, axis=1)
    ratio = np.divide(amax_b, emax * M_of_block, out=np.zeros_like(amax_b),
                      where=M_of_block > 0)
    mu = round_to_grid(ratio, E4M3)

    # Step 4: element codes against the effective scale s = mu * M (exact product).
    s = np.repeat(mu * M_of_block, BLOCK, axis=1)
    q = np.divide(ax, s, out=np.zeros_like(ax), where=s > 0)
    sign = np.signbit(x) & (s > 0)
    if elem == "e2m1":
        mag = e2m1_encode_magnitude(round_to_grid(q, E2M1))
        codes4 = (mag | (sign.astype(np.uint8) << 3)).astype(np.uint8)
        codes = pack_e2m1(codes4)
    else:
        mag = e4m3_encode(round_to_grid(q, E4M3))
        codes = (mag | (sign.astype(np.uint8) << 7)).astype(np.uint8)

    return QuantizedTensor(codes=codes, micro=e4m3_encode(mu), macro=fp16_bits(M),
                           elem=elem, k=K)


def element_values(qt: QuantizedTensor) -> np.ndarray:
    """Element values before scaling: E2M1 or E4M3 decode of the codes, [R, K]."""
    if qt.elem == "e2m1":
        return e2m1_decode(unpack_e2m1(qt.codes))
    return e4m3_decode(qt.codes)


def dequantize(qt: QuantizedTensor) -> np.ndarray:
    """x_hat = value(code) * mu * M, float64 [R, K] (every product is exact)."""
    v = element_values(qt)
    mu = e4m3_decode(qt.micro)
    M = fp16_from_bits(qt.macro)
    return v * np.repeat(mu, BLOCK, axis=1) * np.repeat(M, GROUP, axis=1)
