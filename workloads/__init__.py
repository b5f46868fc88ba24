"""Seeded synthetic inputs for the five workloads (shared by the oracle tests and the
GPU harness as *input data only*; nothing here quantizes or multiplies).

The shapes and value distributions stand in for the 8B-70B-class LLM linear layers the
FP4 pages discuss (no weights or datasets are used):
* weights ~ N(0, 0.02), activations ~ N(0, 1);
* a few input channels scaled up to model activation outliers, which the TensorRT-LLM
  FP4 page ("The Mathematical Breakthrough of Microscopic FP4 Scaling") describes as
  features "up to 100x" the mean magnitude;
* bf16 values are produced by torch's round-to-nearest-even cast.

Every array is drawn from ``numpy.random.default_rng`` (PCG64). Large workloads are
generated piecewise (one layer / one expert at a time) from child generators seeded by
``(seed, stream_id, index)`` so any piece can be regenerated alone.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["normal", "to_bf16_values", "outlier_channels", "tiny", "decode", "prefill",
           "policy_flags", "policy_outliers", "policy_layer", "policy_calibration",
           "moe_router_logits", "moe_tokens",
           "moe_expert_weights", "moe_down_inputs", "kv_lengths", "kv_key_outliers", "kv_queries",
           "kv_rows_device", "WORKLOADS"]

WORKLOADS = {
    "tiny_w4a16": dict(seed=0, m=16, k=512, n=256),
    "decode_w4a16": dict(seed=1, m=8, k=4096, n=14336, outlier_frac=0.001, outlier_gain=100.0),
    "prefill_w4a4": dict(seed=2, m=2048, k=4096, n=4096, outlier_frac=0.005, outlier_gain=50.0),
    "policy_stack": dict(seed=3, layers=8, flagged=2, m=512, k=5120, n=5120,
                         outlier_frac=0.005, outlier_gain=50.0, calib_rows=512),
    "decode_attention_fp4kv": dict(seed=5, n_seq=32, q_heads=32, kv_heads=8, head_dim=128,
                                   max_tokens=16384, min_len=8192, max_len=16383),
    "moe_w4a4": dict(seed=4, experts=128, top_k=8, tokens=4096, hidden=2048,
                     inter=768, outlier_frac=0.005, outlier_gain=50.0),
}


def normal(rng: np.random.Generator, sigma: float, shape) -> np.ndarray:
    return (sigma * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16 round-to-nearest-even of ``x``."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def outlier_channels(rng: np.random.Generator, k: int, frac: float) -> np.ndarray:
    count = int(math.floor(frac * k + 0.5))
    return np.sort(rng.choice(k, count, replace=False))


def _child(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng((seed, stream, index))


def tiny(m=16, k=512, n=256, seed=0):
    """fp32 A [m, k] then fp32 W [n, k], both N(0, 1)."""
    rng = np.random.default_rng(seed)
    a = normal(rng, 1.0, (m, k))
    w = normal(rng, 1.0, (n, k))
    return a, w


def decode(m=8, k=4096, n=14336, seed=1, outlier_frac=0.001, outlier_gain=100.0):
    """W [n, k] ~ N(0, 0.02) with a few input channels x gain; A bf16 [m, k] ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    w = normal(rng, 0.02, (n, k))
    ch = outlier_channels(rng, k, outlier_frac)
    w[:, ch] *= np.float32(outlier_gain)
    a = to_bf16_values(normal(rng, 1.0, (m, k)))
    return a, w, ch


def prefill(m=2048, k=4096, n=4096, seed=2, outlier_frac=0.005, outlier_gain=50.0):
    """A bf16 [m, k] ~ N(0, 1) with outlier channels x gain; W [n, k] ~ N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    a = normal(rng, 1.0, (m, k))
    ch = outlier_channels(rng, k, outlier_frac)
    a[:, ch] *= np.float32(outlier_gain)
    a = to_bf16_values(a)
    w = normal(rng, 0.02, (n, k))
    return a, w, ch


def policy_flags(layers=8, flagged=2, seed=3) -> np.ndarray:
    """Boolean flag per layer: exactly ``flagged`` layers are marked for 8-bit activations."""
    rng = np.random.default_rng(seed)
    idx = rng.choice(layers, flagged, replace=False)
    flags = np.zeros(layers, dtype=bool)
    flags[idx] = True
    return flags


def policy_outliers(k=5120, seed=3, outlier_frac=0.005) -> np.ndarray:
    return outlier_channels(_child(seed, 1), k, outlier_frac)


def policy_layer(layer: int, m=512, k=5120, n=5120, seed=3, outlier_frac=0.005,
                 outlier_gain=50.0):
    """(W_l [n, k] ~ N(0, 0.02), x_l bf16 [m, k] ~ N(0, 1) with the shared outliers)."""
    w = normal(_child(seed, 2, layer), 0.02, (n, k))
    x = normal(_child(seed, 3, layer), 1.0, (m, k))
    x[:, policy_outliers(k, seed, outlier_frac)] *= np.float32(outlier_gain)
    return w, to_bf16_values(x)


def policy_calibration(layer: int, rows=512, k=5120, seed=3, outlier_frac=0.005,
                       outlier_gain=50.0) -> np.ndarray:
    """A separate calibration batch for layer ``layer``, bf16 [rows, k], drawn like x_l (same
    outlier channels): the data static activation scales are calibrated on."""
    x = normal(_child(seed, 4, layer), 1.0, (rows, k))
    x[:, policy_outliers(k, seed, outlier_frac)] *= np.float32(outlier_gain)
    return to_bf16_values(x)


def moe_router_logits(tokens=4096, experts=128, seed=4):
    """Router logits fp32 [tokens, experts] ~ N(0, 1). (The routing itself, top-k with its
    softmax weights and the permutation of routed rows, is a step of the layer: the oracle
    and the library each compute it from these logits.)"""
    return normal(_child(seed, 0), 1.0, (tokens, experts))


def moe_tokens(tokens=4096, hidden=2048, seed=4, outlier_frac=0.005, outlier_gain=50.0):
    """Token activations bf16 [tokens, hidden] ~ N(0, 1) with outlier channels x gain."""
    rng = _child(seed, 1)
    x = normal(rng, 1.0, (tokens, hidden))
    ch = outlier_channels(rng, hidden, outlier_frac)
    x[:, ch] *= np.float32(outlier_gain)
    return to_bf16_values(x)


def moe_expert_weights(expert: int, hidden=2048, inter=768, seed=4):
    """(W1_e [2*inter, hidden] fused gate/up, W2_e [hidden, inter]), both N(0, 0.02)."""
    rng = _child(seed, 2, expert)
    w1 = normal(rng, 0.02, (2 * inter, hidden))
    w2 = normal(rng, 0.02, (hidden, inter))
    return w1, w2


def moe_down_inputs(rows: int, inter=768, seed=4):
    """Stand-in inputs of the down projection alone, bf16 [rows, inter] ~ N(0, 1) (for
    tests of the plain grouped product; the layer itself feeds it silu(gate) * up)."""
    return to_bf16_values(normal(_child(seed, 3), 1.0, (rows, inter)))


def kv_lengths(n_seq=32, min_len=8192, max_len=16383, seed=5) -> np.ndarray:
    """Cached tokens per sequence before the decode step, int32 uniform in [min_len, max_len]."""
    return _child(seed, 0).integers(min_len, max_len + 1, size=n_seq).astype(np.int32)


def kv_key_outliers(width=1024, frac=0.005, seed=5) -> np.ndarray:
    """Key channels (of the kv_heads * head_dim row) scaled up: 0.5% of them."""
    return outlier_channels(_child(seed, 1), width, frac)


def kv_queries(n_seq=32, q_heads=32, head_dim=128, seed=5) -> np.ndarray:
    """Decode queries, bf16 values of N(0, 1) [n_seq, q_heads, head_dim]."""
    return to_bf16_values(normal(_child(seed, 2), 1.0, (n_seq, q_heads, head_dim)))


def kv_rows_device(torch, rows: int, width: int, seed: int, stream: int, outliers=None,
                   gain: float = 20.0, device="cuda"):
    """Cache rows bf16 [rows, width] ~ N(0, 1) from torch's seeded generator on the device
    (about 10^9 values at full size are too many to draw on the host); ``outliers``
    channels scaled by ``gain``. Tests copy the rows they check back to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    x = torch.randn(rows, width, generator=g, device=device, dtype=torch.float32)
    if outliers is not None and len(outliers):
        x[:, torch.as_tensor(np.asarray(outliers), device=device)] *= gain
    return x.to(torch.bfloat16)
