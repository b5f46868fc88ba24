"""Quantized matrix products on the CPU: C = A_hat . W_hat^T accumulated in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:
* "llama.cpp Put Precision Policy Inside the Model. That Matters More Than W4A4",
  intro and section "One model can need more than one precision": 4-bit weights with
  4-bit activations (W4A4), 8-bit activations for layers marked in the model's metadata
  (W4A8), layers "closer to W4A16"; the same routing for dense and mixture-of-experts
  products; section "Local inference is becoming a policy engine": modes q4 (force
  W4A4), q8 (force W4A8) and auto (follow the per-layer metadata).
* "NVIDIA Ships TensorRT-LLM 0.16 ...", item 3 of the scaling section: the scales are
  applied before the dot products, i.e. the product is taken of the dequantized values.

Definitions used here (plain readings):
  W_hat = dequantize(quantize(W, e2m1))                      (weights, always FP4)
  A_hat = A                                    for W4A16
        = dequantize(quantize(A, e2m1))        for W4A4
        = dequantize(quantize(A, e4m3))        for W4A8
  C     = A_hat @ W_hat^T, exact products, float64 sums; no bias, no activation.
  A bf16 result is C rounded to bfloat16 (ties to even).
A grouped (mixture-of-experts) product applies expert e's weights to the rows
``offsets[e] .. offsets[e+1]`` of the routed activation list.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_round
from .quant import QuantizedTensor, quantize, dequantize

A16, A8, A4 = 16, 8, 4
POLICY_AUTO, POLICY_Q4, POLICY_Q8 = 0, 4, 8

__all__ = ["activation_values", "gemm", "gemm_bf16", "grouped_gemm", "policy_select",
           "A16", "A8", "A4", "POLICY_AUTO", "POLICY_Q4", "POLICY_Q8"]


def activation_values(a, act: int) -> np.ndarray:
    """A_hat for the given activation precision (float64)."""
    a = np.asarray(a).astype(np.float64)
    if act == A16:
        return a
    if act == A4:
        return dequantize(quantize(a, "e2m1"))
    if act == A8:
        return dequantize(quantize(a, "e4m3"))
    raise ValueError(f"unknown activation precision {act}")


def gemm(a, w: QuantizedTensor, act: int) -> np.ndarray:
    """C[m, n] = sum_k A_hat[m, k] * W_hat[n, k] in float64."""
    if w.elem != "e2m1":
        raise ValueError("weights are E2M1")
    a_hat = activation_values(a, act)
    w_hat = dequantize(w)
    if a_hat.shape[1] != w_hat.shape[1]:
        raise ValueError("K mismatch")
    return a_hat @ w_hat.T


def gemm_bf16(a, w: QuantizedTensor, act: int) -> np.ndarray:
    return bf16_round(gemm(a, w, act))


def grouped_gemm(a, row_token, offsets, w_stacked: QuantizedTensor, n_experts: int,
                 act: int, experts=None) -> dict:
    """Per-expert products over routed rows.

    ``a``         [T, K] token activations
    ``row_token`` [R] source token of each routed row, or None when ``a`` already holds
                  the R routed rows in expert order
    ``offsets``   [E + 1] non-decreasing, offsets[0] = 0, offsets[E] = R
    ``w_stacked`` expert weights stacked along rows: expert e owns rows e*N .. e*N+N-1
    ``experts``   optional subset of expert ids to evaluate (all when None)
    Returns {e: C_e [rows_e, N] float64}.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    a = np.asarray(a).astype(np.float64)
    rows = a if row_token is None else a[np.asarray(row_token, dtype=np.int64)]
    n_total = w_stacked.rows
    if n_total % n_experts:
        raise ValueError("stacked rows not divisible by expert count")
    N = n_total // n_experts
    out = {}
    for e in (range(n_experts) if experts is None else experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sl = slice(e * N, (e + 1) * N)
        w_e = QuantizedTensor(w_stacked.codes[sl], w_stacked.micro[sl],
                              w_stacked.macro[sl], w_stacked.elem, w_stacked.k)
        out[e] = gemm(rows[lo:hi], w_e, act)
    return out


def policy_select(mode: int, layer_flag: bool) -> int:
    """q4 -> W4A4, q8 -> W4A8, auto -> W4A8 where the layer is marked, else W4A4."""
    if mode == POLICY_Q4:
        return A4
    if mode == POLICY_Q8:
        return A8
    if mode == POLICY_AUTO:
        return A8 if layer_flag else A4
    raise ValueError(f"unknown policy mode {mode}")
