"""The mixture-of-experts layer around the grouped product, on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:
* "llama.cpp Put Precision Policy Inside the Model. That Matters More Than W4A4", section
  "One model can need more than one precision": the W4A4 / W4A8 routing covers mixture-of-
  experts operations as well as dense ones.
* The ClusterBid FP4 inference cost guide, section "Where Does FP4 Hurt Accuracy?": the
  router is among the parts that quantization hurts most, so it stays in float32 here and
  is never quantized.

The pages fix no routing details. Plain readings used here:
  * each token goes to the top_k experts with the largest router logits; equal logits
    go to the lower expert id first;
  * the token's combine weights are the softmax over its top_k selected logits (the full
    softmax restricted to the selected experts and renormalized);
  * routed rows are ordered by (expert, token): expert e owns rows
    offsets[e] .. offsets[e+1], its tokens in increasing order;
  * the gate/up product's output row holds gate in columns [0, I) and up in [I, 2I);
    the down product's input is h = silu(gate) * up, silu(x) = x / (1 + exp(-x)), rounded
    to bfloat16 (the activation dtype of every product here) before its own dynamic
    quantization;
  * the layer output for token t is the sum over its top_k choices j (in rank order) of
    weight[t, j] * down_output[row(t, j)].
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_round

__all__ = ["route", "silu_gate", "combine"]


def route(logits, top_k: int):
    """Top-k routing of float router logits [T, E].

    Returns (topk_ids int32 [T, k], weights float64 [T, k], offsets int32 [E + 1],
    row_token int32 [R], token_rows int32 [T, k]) with R = T * k; row_token[r] is the
    token of routed row r and token_rows[t, j] the routed row of token t's j-th choice."""
    logits = np.asarray(logits, dtype=np.float64)
    t_count, e_count = logits.shape
    if not 1 <= top_k <= e_count:
        raise ValueError("top_k must be in [1, n_experts]")
    topk_ids = np.zeros((t_count, top_k), dtype=np.int32)
    weights = np.zeros((t_count, top_k), dtype=np.float64)
    for t in range(t_count):
        # largest logit first; among equal logits the lower expert id first
        order = sorted(range(e_count), key=lambda e: (-logits[t, e], e))[:top_k]
        topk_ids[t] = order
        sel = logits[t, order]
        ex = np.exp(sel - sel.max())
        weights[t] = ex / ex.sum()
    counts = np.zeros(e_count, dtype=np.int64)
    for t in range(t_count):
        for e in topk_ids[t]:
            counts[e] += 1
    offsets = np.zeros(e_count + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_token = np.zeros(t_count * top_k, dtype=np.int32)
    token_rows = np.zeros((t_count, top_k), dtype=np.int32)
    fill = offsets[:-1].astype(np.int64).copy()
    for t in range(t_count):  # tokens in increasing order: rows of each expert sorted by token
        for e in sorted(topk_ids[t]):
            r = fill[e]
            fill[e] += 1
            row_token[r] = t
            token_rows[t, list(topk_ids[t]).index(e)] = r
    return topk_ids, weights, offsets, row_token, token_rows


def silu_gate(y1, inter: int, precision=np.float64) -> np.ndarray:
    """h = silu(gate) * up for gate = y1[:, :inter], up = y1[:, inter:2*inter], evaluated in
    the given float precision and rounded to bfloat16 (returned as float64 values)."""
    y1 = np.asarray(y1, dtype=precision)
    g, u = y1[:, :inter], y1[:, inter:2 * inter]
    one = precision(1.0)
    h = (g / (one + np.exp(-g))) * u
    return bf16_round(h.astype(np.float64))


def combine(y2, token_rows, weights) -> np.ndarray:
    """out[t] = sum_j weights[t, j] * y2[token_rows[t, j]] (float64, j in rank order)."""
    y2 = np.asarray(y2, dtype=np.float64)
    token_rows = np.asarray(token_rows)
    weights = np.asarray(weights, dtype=np.float64)
    out = np.zeros((token_rows.shape[0], y2.shape[1]), dtype=np.float64)
    for j in range(token_rows.shape[1]):
        out += weights[:, j:j + 1] * y2[token_rows[:, j]]
    return out
