"""Precision for sensitive layers and calibrated activation scales, on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:
* "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200", section
  "Deployment Guidelines and Production Safeguards", item 2: layer 0 and the output heads
  are more sensitive, and FP8 precision can be kept on those layers while the rest runs in
  FP4; section "Step 2: Executing FP4 Calibration and Engine Compilation" and item 1 of
  the guidelines: activation ranges are calibrated ahead of deployment on data that
  matches production traffic.
* The ClusterBid FP4 inference cost guide, section "FP4 Migration Checklist That Prevents
  Rollbacks": when FP4 regresses, a few sensitive layers go back to FP8.
* "llama.cpp Put Precision Policy Inside the Model. That Matters More Than W4A4", section
  "Local inference is becoming a policy engine": the runtime picks precision per layer
  (q4 / q8 / auto).

The pages fix no FP8 weight format and no calibration procedure. Plain readings used here:
  * W8A8: weights in the same two-level format with E4M3 elements (E4M3 micro-scale per 16,
    FP16 macro-scale per 256), activations quantized dynamically as for W4A8;
  * static activation macro-scales: one FP16 macro-scale per 256-group of columns, shared
    by every row (token), calibrated as the dynamic rule applied to the group's maximum
    over the calibration rows; at run time the micro-scales stay per 16 elements and per
    row, computed against that fixed macro-scale; values beyond its range saturate;
  * two more policy modes: "sensitive-w8" runs flagged layers W8A8 and the others W4A4;
    "static" runs A8 on flagged layers and A4 elsewhere, both with static macro-scales.
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1, E4M3, FP16, round_to_grid, fp16_bits, fp16_from_bits, e4m3_encode,
                      e2m1_encode_magnitude)
from .quant import (QuantizedTensor, dequantize, pack_e2m1, BLOCK, GROUP, E4M3_MAX, ELEM_MAX,
                    M_MIN, M_MAX, _check_input)
from .gemm import A4, A8, activation_values

__all__ = ["W8A8", "A4S", "A8S", "POLICY_SENSITIVE_W8", "POLICY_STATIC", "calibrate_macro",
           "quantize_static", "activation_values_static", "gemm_w8a8", "gemm_static",
           "policy_select_ext"]

W8A8, A4S, A8S = 88, 40, 80  # precision codes beyond A4 / A8 / A16
POLICY_SENSITIVE_W8, POLICY_STATIC = 1, 2


def calibrate_macro(a_calib, elem: str) -> np.ndarray:
    """FP16 bits [K/256] of the static macro-scales: the dynamic macro rule on each group's
    maximum |x| over all calibration rows."""
    x = _check_input(a_calib)
    R, K = x.shape
    amax = np.abs(x).reshape(R, K // GROUP, GROUP).max(axis=(0, 2))
    M = round_to_grid(amax / (ELEM_MAX[elem] * E4M3_MAX), FP16)
    M = np.where(amax > 0, np.clip(M, M_MIN, M_MAX), 0.0)
    return fp16_bits(M)


def quantize_static(x, macro_bits, elem: str = "e2m1") -> QuantizedTensor:
    """Two-level quantization of each row of x with the given macro-scales (FP16 bits per
    group, shared by all rows): micro-scales RNE_E4M3sat(amax_16 / (emax * M)), elements
    RNE to the element format, saturating."""
    x = _check_input(x)
    R, K = x.shape
    emax = ELEM_MAX[elem]
    M = np.broadcast_to(fp16_from_bits(np.asarray(macro_bits, dtype=np.uint16)), (R, K // GROUP))
    ax = np.abs(x)
    amax_b = ax.reshape(R, K // BLOCK, BLOCK).max(axis=2)
    M_of_block = np.repeat(M, GROUP // BLOCK, axis=1)
    ratio = np.divide(amax_b, emax * M_of_block, out=np.zeros_like(amax_b), where=M_of_block > 0)
    mu = round_to_grid(ratio, E4M3)  # saturates at 448
    s = np.repeat(mu * M_of_block, BLOCK, axis=1)
    q = np.divide(ax, s, out=np.zeros_like(ax), where=s > 0)
    sign = np.signbit(x) & (s > 0)
    if elem == "e2m1":
        mag = e2m1_encode_magnitude(round_to_grid(q, E2M1))
        codes = pack_e2m1((mag | (sign.astype(np.uint8) << 3)).astype(np.uint8))
    else:
        mag = e4m3_encode(round_to_grid(q, E4M3))
        codes = (mag | (sign.astype(np.uint8) << 7)).astype(np.uint8)
    return QuantizedTensor(codes=codes, micro=e4m3_encode(mu),
                           macro=np.ascontiguousarray(fp16_bits(M)), elem=elem, k=K)


def activation_values_static(a, act: int, macro_bits) -> np.ndarray:
    elem = {A4S: "e2m1", A8S: "e4m3"}[act]
    return dequantize(quantize_static(a, macro_bits, elem))


def gemm_w8a8(a, w8: QuantizedTensor) -> np.ndarray:
    """C = A8(a) . W_hat^T, W quantized with E4M3 elements (float64)."""
    if w8.elem != "e4m3":
        raise ValueError("W8A8 weights are E4M3")
    return activation_values(a, A8) @ dequantize(w8).T


def gemm_static(a, w: QuantizedTensor, act: int, macro_bits) -> np.ndarray:
    """C = A_static(a) . W_hat^T for act A4S / A8S, W E2M1 (float64)."""
    if w.elem != "e2m1":
        raise ValueError("weights are E2M1")
    return activation_values_static(a, act, macro_bits) @ dequantize(w).T


def policy_select_ext(mode: int, layer_flag: bool) -> int:
    """sensitive-w8: flagged -> W8A8, else A4; static: flagged -> A8S, else A4S."""
    if mode == POLICY_SENSITIVE_W8:
        return W8A8 if layer_flag else A4
    if mode == POLICY_STATIC:
        return A8S if layer_flag else A4S
    raise ValueError(f"unknown policy mode {mode}")
