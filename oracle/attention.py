"""Decode attention over a KV cache stored in the two-level block-scaled FP4 format, on the
CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:
* "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200", section
  "The Mathematical Breakthrough of Microscopic FP4 Scaling" (the codec).
* "The FP4 Inflection: Rethinking AI Inference Architecture", section "What does this
  mean for model serving engines?": keeping the KV cache in FP4 cuts its memory footprint
  and bandwidth, and needs new attention kernels.
* "AdaLLM Breakthrough: First NVFP4-Only Inference Engine for RTX 4090 Unveiled": a
  quantized KV cache read by a dedicated decode kernel (FP8 there), with grouped-query
  models (Qwen3, Gemma3).

The pages fix no attention details. Plain readings used here:
  * the cache holds, per token, the key (and value) vector of every KV head; each token's
    vector [kv_heads * head_dim] is one row of the codec (blocks of 16 and groups of 256
    along it), quantized once when the token is appended;
  * decode attention for query head h of a sequence with L cached tokens uses KV head
    h // (q_heads // kv_heads) (grouped-query attention):
        out[h] = sum_t softmax_t(scale * q[h] . K_hat[t]) * V_hat[t],   t < L,
    with K_hat, V_hat the dequantized cache and scale usually 1/sqrt(head_dim).
"""
from __future__ import annotations

import numpy as np

from .quant import quantize, dequantize

__all__ = ["kv_quantize_rows", "kv_dequantize_rows", "attention_decode"]


def kv_quantize_rows(rows):
    """Quantize token rows [n, kv_heads * head_dim] with the two-level E2M1 codec."""
    return quantize(np.asarray(rows, dtype=np.float64))


def kv_dequantize_rows(rows) -> np.ndarray:
    """The values the cache holds for token rows: dequantize(quantize(rows)), float64."""
    return dequantize(kv_quantize_rows(rows))


def attention_decode(q, k_hat, v_hat, lengths, scale: float) -> np.ndarray:
    """q [B, Hq, D]; k_hat, v_hat [B, T, Hkv, D] (cache values); lengths [B] (1 <= L <= T).
    Returns out [B, Hq, D] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    n_seq, q_heads, _ = q.shape
    kv_heads = k_hat.shape[2]
    if q_heads % kv_heads:
        raise ValueError("q_heads must be a multiple of kv_heads")
    group = q_heads // kv_heads
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(n_seq):
        length = int(lengths[b])
        if not 1 <= length <= k_hat.shape[1]:
            raise ValueError("every sequence needs 1 <= length <= cache tokens")
        for h in range(q_heads):
            kvh = h // group
            s = scale * (k_hat[b, :length, kvh, :] @ q[b, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, h] = p @ v_hat[b, :length, kvh, :]
    return out
