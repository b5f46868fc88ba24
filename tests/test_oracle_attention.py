"""Pins of the decode-attention oracle against a library routine (torch's scaled dot-product
attention in float64), closed forms, the grouped-query head mapping and the length bound."""
import numpy as np
import pytest
import torch

import oracle


def _sdpa(q, k, v, lengths, scale):
    """torch.nn.functional.scaled_dot_product_attention per sequence, KV heads repeated
    for grouped-query attention."""
    n_seq, q_heads, d = q.shape
    group = q_heads // k.shape[2]
    out = np.zeros(q.shape)
    for b in range(n_seq):
        length = int(lengths[b])
        kk = torch.from_numpy(k[b, :length]).permute(1, 0, 2).repeat_interleave(group, dim=0)
        vv = torch.from_numpy(v[b, :length]).permute(1, 0, 2).repeat_interleave(group, dim=0)
        qq = torch.from_numpy(q[b]).unsqueeze(1)  # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
        out[b] = o[:, 0, :].numpy()
    return out


def test_matches_torch_sdpa_with_gqa_and_ragged_lengths():
    rng = np.random.default_rng(61)
    n_seq, t_max, kv_heads, q_heads, d = 3, 70, 2, 8, 16
    q = rng.standard_normal((n_seq, q_heads, d))
    k = rng.standard_normal((n_seq, t_max, kv_heads, d))
    v = rng.standard_normal((n_seq, t_max, kv_heads, d))
    lengths = np.array([70, 1, 33])
    scale = 1.0 / np.sqrt(d)
    got = oracle.attention_decode(q, k, v, lengths, scale)
    ref = _sdpa(q, k, v, lengths, scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value_and_equal_keys_average():
    rng = np.random.default_rng(62)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 5, 1, 8))
    v = rng.standard_normal((1, 5, 1, 8))
    one = oracle.attention_decode(q, k, v, [1], 0.3)
    assert np.array_equal(one[0], np.repeat(v[0, 0, 0][None, :], 4, axis=0))
    k_same = np.repeat(k[:, :1], 5, axis=1)  # every key equal: uniform weights
    avg = oracle.attention_decode(q, k_same, v, [5], 0.3)
    assert np.allclose(avg[0], np.repeat(v[0, :, 0].mean(axis=0)[None, :], 4, axis=0), rtol=0, atol=1e-14)
    zero_scale = oracle.attention_decode(q, k, v, [4], 0.0)  # scale 0: uniform too
    assert np.allclose(zero_scale[0, 2], v[0, :4, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(63)
    q = np.zeros((1, 2, 4))
    q[0, :, 0] = 1.0
    k = rng.standard_normal((1, 9, 1, 4)) * 0.01
    k[0, 6, 0, 0] = 100.0  # score 100 against ~0: weight 1 - O(e^-99)
    v = rng.standard_normal((1, 9, 1, 4))
    out = oracle.attention_decode(q, k, v, [9], 1.0)
    assert np.max(np.abs(out[0, 0] - v[0, 6, 0])) <= 8 * np.exp(-99) * np.abs(v).max()


def test_grouped_query_head_mapping():
    n_seq, t_max, kv_heads, q_heads, d = 2, 6, 4, 12, 8
    rng = np.random.default_rng(64)
    q = rng.standard_normal((n_seq, q_heads, d))
    k = rng.standard_normal((n_seq, t_max, kv_heads, d))
    v = np.zeros((n_seq, t_max, kv_heads, d))
    for kvh in range(kv_heads):
        v[:, :, kvh, :] = kvh  # a head's output is its KV head's constant value
    out = oracle.attention_decode(q, k, v, [6, 3], 0.5)
    for h in range(q_heads):
        assert np.allclose(out[:, h], h // 3, rtol=0, atol=1e-12)


def test_tokens_past_the_length_are_ignored():
    rng = np.random.default_rng(65)
    q = rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((1, 10, 1, 8))
    v = rng.standard_normal((1, 10, 1, 8))
    ref = oracle.attention_decode(q, k, v, [4], 0.4)
    k[0, 4:], v[0, 4:] = np.nan, np.inf
    assert np.array_equal(oracle.attention_decode(q, k, v, [4], 0.4), ref)


def test_kv_rows_use_the_pinned_codec_per_token():
    """Cache values are the two-level codec applied to each token row; a row of exactly
    representable values is kept: E2M1 codes times 448 * 2^-10, every block reaching code
    6, so that M = 2688 * 448 * 2^-10 / 2688 / 448 = 2^-10 (an FP16 value) and mu = 448 (an
    E4M3 value) exactly."""
    rng = np.random.default_rng(66)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    row = rng.choice(grid, size=(3, 512)) * rng.choice([-1, 1], size=(3, 512))
    row[:, ::16] = 6.0
    scaled = row * 448.0 * 2.0 ** -10
    assert np.array_equal(oracle.kv_dequantize_rows(scaled), scaled)
    # a different power of two per group is kept as well (groups are independent)
    scaled2 = scaled.copy()
    scaled2[:, 256:] *= 2.0 ** 5
    assert np.array_equal(oracle.kv_dequantize_rows(scaled2), scaled2)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.attention_decode(np.zeros((1, 3, 4)), np.zeros((1, 2, 2, 4)), np.zeros((1, 2, 2, 4)), [1], 1.0)
    with pytest.raises(ValueError):
        oracle.attention_decode(np.zeros((1, 2, 4)), np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1, 4)), [3], 1.0)
