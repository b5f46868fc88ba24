"""GPU parity of the MX-native FP4 path (quantize_mxfp4, gemm_mxfp4) against the CPU oracle,
through the C ABI.

Gates: codes and E8M0 scales bit-exact (integer work); float32 products within 1e-5
relative Frobenius error (every element product is exact, the matrix core accumulates in
float32); bf16 products through the bf16 gate."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._util import host, bf16_values, bf16_gate, f32_gate, mx_tiled_to_canonical

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _inputs(rng, rows, k):
    x = (rng.standard_normal((rows, k)) * np.exp(rng.uniform(-8, 8, (rows, 1)))).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 50  # outlier channels
    x[0, :32] = 0.0
    x[1 % rows, 32:64] = -0.0
    x[2 % rows, 64:96] = 1e-42  # float32 subnormals
    return x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,k", [(37, 384), (16, 128), (1, 256)])
def test_quantize_bit_exact(dtype, rows, k):
    rng = np.random.default_rng(101 + rows + k)
    x = _inputs(rng, rows, k)
    if dtype == torch.bfloat16:
        x = workloads.to_bf16_values(x)
    print(f"[case] quantize_mxfp4 {rows}x{k} {dtype}", flush=True)
    q = fp4.quantize_mxfp4(torch.from_numpy(x).cuda().to(dtype))
    codes, scales, pad_c, pad_s = mx_tiled_to_canonical(q)
    rc, rs = oracle.mx_quantize(x.astype(np.float64))
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales, rs)
    assert not pad_c.any() and not pad_s.any()


def test_quantize_full_prefill_weight():
    _, w, _ = workloads.prefill()
    print("[case] quantize_mxfp4 4096x4096 weight", flush=True)
    q = fp4.quantize_mxfp4(torch.from_numpy(w).cuda())
    codes, scales, _, _ = mx_tiled_to_canonical(q)
    rc, rs = oracle.mx_quantize(w.astype(np.float64))
    assert np.array_equal(codes, rc) and np.array_equal(scales, rs)


# 128-k stages: 3 and 1 (only the last partial pass), 8 (two whole passes over the four-slot
# ring), 5, 6 and 7 (a whole pass, then 1, 2 or 3 stages)
@pytest.mark.parametrize("m,n,k", [(37, 300, 384), (128, 128, 128), (200, 136, 1024), (64, 200, 640),
                                   (130, 96, 768), (96, 150, 896)])
def test_gemm_small(m, n, k):
    rng = np.random.default_rng(m + n + k)
    a = workloads.to_bf16_values(_inputs(rng, m, k))
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm_mxfp4 {m}x{n}x{k}", flush=True)
    aq = fp4.quantize_mxfp4(torch.from_numpy(a).cuda().to(torch.bfloat16))
    wq = fp4.quantize_mxfp4(torch.from_numpy(w).cuda())
    ref = oracle.mx_gemm(a.astype(np.float64), w.astype(np.float64))
    got = host(fp4.gemm_mxfp4(aq, wq, out_dtype=torch.float32)).astype(np.float64)
    rel = f32_gate(got, ref, rel_frob=1e-5)
    print(f"  relative Frobenius error {rel:.2e}", flush=True)
    bf16_gate(bf16_values(fp4.gemm_mxfp4(aq, wq)), oracle.formats.bf16_round(ref))


def test_gemm_prefill_full_size_sampled():
    a, w, _ = workloads.prefill()
    print("[case] gemm_mxfp4 2048x4096x4096 sampled", flush=True)
    aq = fp4.quantize_mxfp4(torch.from_numpy(a).cuda().to(torch.bfloat16))
    wq = fp4.quantize_mxfp4(torch.from_numpy(w).cuda())
    got = host(fp4.gemm_mxfp4(aq, wq, out_dtype=torch.float32)).astype(np.float64)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(2048, 64, replace=False))
    cols = np.sort(rng.choice(4096, 256, replace=False))
    ca, sa = oracle.mx_quantize(a[rows].astype(np.float64))
    cw, sw = oracle.mx_quantize(w[cols].astype(np.float64))
    ref = oracle.mx_dequantize(ca, sa) @ oracle.mx_dequantize(cw, sw).T
    f32_gate(got[np.ix_(rows, cols)], ref, rel_frob=1e-5)
    again = host(fp4.gemm_mxfp4(aq, wq, out_dtype=torch.float32)).astype(np.float64)
    assert np.array_equal(got, again)


def test_rejects_bad_shapes():
    with pytest.raises(fp4.Fp4Error):
        fp4.quantize_mxfp4(torch.zeros(4, 96, device="cuda"))
