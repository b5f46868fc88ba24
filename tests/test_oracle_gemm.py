"""Pins for oracle/gemm.py: exact rational products on tiny shapes, W4A16 on representable
weights against a plain matmul, the policy table, the grouped product's row routing, and
the two quality directions the pages state."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F
from oracle.quant import quantize, dequantize
import workloads


def _exact_matmul(a, w):
    """sum_k a[m,k] * w[n,k] over exact rationals."""
    M, K = a.shape
    N = w.shape[0]
    out = np.empty((M, N))
    fa = [[Fraction(float(v)) for v in row] for row in a]
    fw = [[Fraction(float(v)) for v in row] for row in w]
    for i in range(M):
        for j in range(N):
            out[i, j] = float(sum(x * y for x, y in zip(fa[i], fw[j])))
    return out


@pytest.mark.parametrize("act", [oracle.A16, oracle.A8, oracle.A4])
@pytest.mark.parametrize("shape", [(4, 8, 256), (3, 5, 512)])
def test_gemm_vs_exact_rational(act, shape):
    M, N, K = shape
    rng = np.random.default_rng(21 + M)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, 7] *= 50
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    wq = quantize(w)
    got = oracle.gemm(a, wq, act)
    a_hat = oracle.activation_values(a, act)
    want = _exact_matmul(a_hat, dequantize(wq))
    assert got.shape == (M, N)
    assert np.allclose(got, want, rtol=2.0 ** -40, atol=2.0 ** -40 * np.abs(want).max())


def test_w4a16_representable_weights_is_plain_matmul():
    rng = np.random.default_rng(22)
    N, K, M = 24, 512, 5
    codes = rng.integers(0, 16, (N, K))
    codes[:, ::16] = 7
    mu = F.e4m3_decode(rng.integers(1, 0x7F, (N, K // 16)))
    mu[:, ::16] = 448.0
    Mg = np.exp2(rng.integers(-12, -6, (N, K // 256))).astype(np.float64)
    w = F.e2m1_decode(codes) * np.repeat(mu, 16, 1) * np.repeat(Mg, 256, 1)
    a = rng.standard_normal((M, K))
    assert np.array_equal(dequantize(quantize(w)), w)
    got = oracle.gemm(a, quantize(w), oracle.A16)
    np.testing.assert_allclose(got, a @ w.T, rtol=1e-13, atol=1e-13)
    # operand order: C is [M, N], row m uses A row m, column n uses W row n
    got2 = oracle.gemm(a[::-1], quantize(w[::-1]), oracle.A16)
    np.testing.assert_allclose(got2, (a @ w.T)[::-1, ::-1], rtol=1e-13, atol=1e-13)


def test_bf16_output_rounding():
    rng = np.random.default_rng(23)
    a = rng.standard_normal((3, 256))
    wq = quantize(rng.standard_normal((7, 256)))
    c = oracle.gemm(a, wq, oracle.A16)
    import torch
    ref = torch.from_numpy(c).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.gemm_bf16(a, wq, oracle.A16), ref)


def test_policy_select_table():
    assert oracle.policy_select(oracle.POLICY_Q4, True) == oracle.A4
    assert oracle.policy_select(oracle.POLICY_Q4, False) == oracle.A4
    assert oracle.policy_select(oracle.POLICY_Q8, False) == oracle.A8
    assert oracle.policy_select(oracle.POLICY_Q8, True) == oracle.A8
    assert oracle.policy_select(oracle.POLICY_AUTO, True) == oracle.A8
    assert oracle.policy_select(oracle.POLICY_AUTO, False) == oracle.A4
    with pytest.raises(ValueError):
        oracle.policy_select(3, False)


def test_grouped_gemm_routes_rows():
    rng = np.random.default_rng(24)
    T, K, N, E = 10, 256, 16, 3
    a = rng.standard_normal((T, K))
    w = rng.standard_normal((E * N, K)) * 0.02
    wq = quantize(w)
    row_token = np.array([3, 1, 4, 1, 5, 9, 2], dtype=np.int32)
    offsets = np.array([0, 3, 3, 7], dtype=np.int32)  # expert 1 gets no rows
    out = oracle.grouped_gemm(a, row_token, offsets, wq, E, oracle.A4)
    assert out[1].shape == (0, N)
    for e, (lo, hi) in enumerate(zip(offsets[:-1], offsets[1:])):
        rows = a[row_token[lo:hi]]
        want = oracle.activation_values(rows, oracle.A4) @ dequantize(wq)[e * N:(e + 1) * N].T
        np.testing.assert_allclose(out[e], want, rtol=1e-13, atol=1e-13)


def _rel(x, ref):
    return np.linalg.norm(x - ref) / np.linalg.norm(ref)


def test_direction_w4a8_beats_w4a4_on_outliers():
    """llama.cpp precision-policy page, "The fastest kernel can be the wrong kernel":
    routing marked layers through W4A8 improved quality over native W4A4."""
    a, w, _ = workloads.prefill(m=64, k=1024, n=128, seed=31)
    wq = quantize(w)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    e16 = _rel(oracle.gemm(a, wq, oracle.A16), ref)
    e8 = _rel(oracle.gemm(a, wq, oracle.A8), ref)
    e4 = _rel(oracle.gemm(a, wq, oracle.A4), ref)
    assert e16 <= e8 < e4


def test_direction_micro_scaling_protects_outliers():
    """TensorRT-LLM FP4 page: per-16 micro-scales keep "up to 100x" outliers from
    clipping the rest; a single per-tensor FP4 scale does much worse."""
    rng = np.random.default_rng(32)
    x = rng.standard_normal((64, 1024))
    x[:, rng.choice(1024, 4, replace=False)] *= 100.0
    two_level = _rel(dequantize(quantize(x)), x)
    s = np.abs(x).max() / 6.0
    single = np.sign(x) * F.round_to_grid(np.abs(x) / s, F.E2M1) * s
    assert two_level < 0.5 * _rel(single, x)


def test_workload_generators_are_deterministic():
    a1, w1 = workloads.tiny()
    a2, w2 = workloads.tiny()
    assert a1.dtype == np.float32 and a1.shape == (16, 512) and w1.shape == (256, 512)
    assert np.array_equal(a1, a2) and np.array_equal(w1, w2)
    l1 = workloads.moe_router_logits(tokens=64, experts=16)
    assert l1.dtype == np.float32 and l1.shape == (64, 16)
    assert np.array_equal(l1, workloads.moe_router_logits(tokens=64, experts=16))
