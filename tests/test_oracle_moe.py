"""Pins of the mixture-of-experts oracle steps (routing, gated activation, combine)
against library routines, closed forms and brute force."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def test_top1_is_argmax_lower_id_on_ties():
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((64, 10)).astype(np.float32)
    logits[3, [2, 7]] = 5.0  # tie: expert 2 must win
    ids, w, *_ = oracle.route(logits, 1)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))  # argmax returns the first max
    assert ids[3, 0] == 2
    assert np.all(w == 1.0)


def test_topk_order_matches_lexsort_and_full_softmax():
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((40, 16)).astype(np.float32)
    logits[5, :] = 0.25  # all tied: ids in increasing order
    ids, w, *_ = oracle.route(logits, 16)
    for t in range(logits.shape[0]):
        ref = np.lexsort((np.arange(16), -logits[t].astype(np.float64)))
        assert np.array_equal(ids[t], ref)
    assert np.array_equal(ids[5], np.arange(16))
    # k = E: the weights are the full softmax, in the selected order
    sm = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(sm, ids.astype(np.int64), axis=1), rtol=0, atol=1e-15)


def test_topk_weights_closed_form():
    logits = np.array([[0.5, 2.0, -1.0, 2.0, 1.5]], dtype=np.float32)
    ids, w, *_ = oracle.route(logits, 3)
    assert list(ids[0]) == [1, 3, 4]  # the tie 2.0 / 2.0 goes to the lower id first
    den = math.exp(2.0) + math.exp(2.0) + math.exp(1.5)
    assert np.allclose(w[0], [math.exp(2.0) / den, math.exp(2.0) / den, math.exp(1.5) / den],
                       rtol=1e-15, atol=0)


def test_routed_rows_bruteforce():
    rng = np.random.default_rng(13)
    t_count, e_count, k = 37, 9, 3
    logits = rng.standard_normal((t_count, e_count)).astype(np.float32)
    ids, w, offsets, row_token, token_rows = oracle.route(logits, k)
    pairs = sorted((int(e), t) for t in range(t_count) for e in ids[t])  # (expert, token)
    assert [t for _, t in pairs] == list(row_token)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(ids.ravel(), minlength=e_count))]))
    for t in range(t_count):
        for j in range(k):
            r = token_rows[t, j]
            assert row_token[r] == t
            assert offsets[ids[t, j]] <= r < offsets[ids[t, j] + 1]
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_silu_gate_library_and_closed_form():
    rng = np.random.default_rng(14)
    inter = 24
    y1 = (3 * rng.standard_normal((7, 2 * inter))).astype(np.float32)
    y1[0, 0], y1[0, inter] = 1.0, 1.0  # silu(1) * 1 = 1 / (1 + e^-1)
    y1[0, 1], y1[0, inter + 1] = 0.0, 5.0  # silu(0) = 0
    h = oracle.silu_gate(y1, inter)
    g, u = y1[:, :inter].astype(np.float64), y1[:, inter:].astype(np.float64)
    ref = scipy.special.expit(g) * g * u
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(h, ref_bf16)
    assert h[0, 0] == torch.tensor(1.0 / (1.0 + math.exp(-1.0))).to(torch.bfloat16).item()
    assert h[0, 1] == 0.0


def test_combine_one_hot_and_linearity():
    rng = np.random.default_rng(15)
    y2 = rng.standard_normal((12, 5))
    rows = np.array([[3, 7], [0, 11], [5, 5]])
    onehot = np.array([[1.0, 0.0], [0.0, 1.0], [0.5, 0.5]])
    out = oracle.combine(y2, rows, onehot)
    assert np.array_equal(out[0], y2[3]) and np.array_equal(out[1], y2[11])
    assert np.array_equal(out[2], y2[5])
    w = rng.random((3, 2))
    full = oracle.combine(y2, rows, w)
    assert np.allclose(full, oracle.combine(y2, rows[:, :1], w[:, :1]) +
                       oracle.combine(y2, rows[:, 1:], w[:, 1:]), rtol=0, atol=1e-14)


def test_route_rejects_bad_topk():
    with pytest.raises(ValueError):
        oracle.route(np.zeros((2, 4), np.float32), 5)
