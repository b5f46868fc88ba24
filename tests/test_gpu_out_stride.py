"""Products written into a padded output (row stride ldc > n): every product form stores
through the row stride it is given, writes nothing between column n and the stride, and
gives the same bits as with contiguous rows.

The stores address rows through ldc (a raw buffer over the tile's rows, a scalar row
offset per store), so these cases take the forms the shapes select (the 128-row-wave
dense form, the 64-row forms, the grouped form, the MX-native product) with ragged m and
n, bf16 and float32 outputs."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as fp4
import oracle
import workloads
from tests._util import host, to_device_bf16

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A  # bf16 / half of a float32 word: a value no product here writes


def _padded(rows, n, ldc, dtype):
    """A [rows x ldc] buffer of sentinel bits and its [rows x n] view."""
    words = 1 if dtype == torch.bfloat16 else 2
    big = torch.full((rows, ldc * words), SENTINEL, dtype=torch.int16, device="cuda")
    view = big.view(dtype)[:, :n]
    return big, view


def _check(big, view, ref, n, dtype):
    words = 1 if dtype == torch.bfloat16 else 2
    pad = host(big[:, n * words:])
    assert np.all(pad == np.int16(SENTINEL)), "a store landed between column n and the row stride"
    assert np.array_equal(host(view.contiguous().view(torch.int16)), host(ref.view(torch.int16))), \
        "padded output differs from the contiguous one"


@pytest.mark.parametrize("act,m,n,k,dtype", [
    (4, 2043, 4080, 256, torch.bfloat16),   # 128-row-wave form
    (4, 300, 1040, 512, torch.float32),     # 64-row forms
    (16, 97, 272, 768, torch.bfloat16),
    (8, 512, 5120, 1024, torch.bfloat16),   # ten-wave form
])
def test_gemm_padded_output(act, m, n, k, dtype):
    rng = np.random.default_rng(m + n + k)
    a = workloads.to_bf16_values(rng.standard_normal((m, k)).astype(np.float32))
    w = (0.05 * rng.standard_normal((n, k))).astype(np.float32)
    wq = fp4.quantize_fp4(torch.from_numpy(w).cuda(), layout=fp4.LAYOUT_TILED)
    ad = to_device_bf16(a)
    name = fp4.fp4_product_kernel(act, torch.bfloat16, m, n, k)
    ldc = n + 48
    print(f"[case] padded output act={act} {m}x{n}x{k} {dtype} ldc={ldc} ({name})", flush=True)
    ref = fp4.gemm_w4aX(act, ad, wq, out_dtype=dtype)
    big, view = _padded(m, n, ldc, dtype)
    fp4.gemm_w4aX(act, ad, wq, out=view)
    torch.cuda.synchronize()
    _check(big, view, ref, n, dtype)


def test_w8a8_padded_output():
    m, n, k = 512, 5120, 1024
    rng = np.random.default_rng(17)
    a = to_device_bf16(workloads.to_bf16_values(rng.standard_normal((m, k)).astype(np.float32)))
    w = torch.from_numpy((0.05 * rng.standard_normal((n, k))).astype(np.float32)).cuda()
    wq = fp4.quantize_fp4(w, elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
    name = fp4.fp4_product_kernel(fp4.W8A8, torch.bfloat16, m, n, k, w_e4m3=True)
    print(f"[case] W8A8 padded output {m}x{n}x{k} ({name})", flush=True)
    ref = fp4.gemm_w8a8(a, wq, out_dtype=torch.bfloat16)
    big, view = _padded(m, n, n + 32, torch.bfloat16)
    fp4.gemm_w8a8(a, wq, out=view)
    torch.cuda.synchronize()
    _check(big, view, ref, n, torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_grouped_padded_output(dtype):
    tokens, experts, top_k, k, n = 300, 6, 2, 512, 272
    logits = workloads.moe_router_logits(tokens=tokens, experts=experts, seed=5)
    _, _, offsets, row_token, _ = oracle.route(logits, top_k)
    R = int(offsets[-1])
    rng = np.random.default_rng(5)
    a = workloads.to_bf16_values(rng.standard_normal((tokens, k)).astype(np.float32))
    w = (0.05 * rng.standard_normal((experts * n, k))).astype(np.float32)
    wq = fp4.quantize_fp4(torch.from_numpy(w).cuda(), layout=fp4.LAYOUT_TILED)
    off = torch.from_numpy(offsets).cuda()
    tok = torch.from_numpy(row_token).cuda()
    print(f"[case] grouped padded output {dtype} R={R}", flush=True)
    ref = fp4.grouped_gemm_w4aX(fp4.A4, to_device_bf16(a), tok, off, experts, R, wq, out_dtype=dtype)
    big, view = _padded(R, n, n + 16, dtype)
    fp4.grouped_gemm_w4aX(fp4.A4, to_device_bf16(a), tok, off, experts, R, wq, out=view)
    torch.cuda.synchronize()
    _check(big, view, ref, n, dtype)


@pytest.mark.parametrize("m,n,k,dtype", [(200, 300, 256, torch.bfloat16), (129, 130, 384, torch.float32)])
def test_mx_padded_output(m, n, k, dtype):
    rng = np.random.default_rng(m * n)
    a = torch.from_numpy(workloads.to_bf16_values(rng.standard_normal((m, k)).astype(np.float32))).cuda()
    w = torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).cuda()
    aq, wq = fp4.quantize_mxfp4(a.to(torch.bfloat16)), fp4.quantize_mxfp4(w)
    ldc = n + 40
    print(f"[case] MX padded output {m}x{n}x{k} {dtype} ldc={ldc}", flush=True)
    ref = fp4.gemm_mxfp4(aq, wq, out_dtype=dtype)
    big, view = _padded(m, n, ldc, dtype)
    fp4.gemm_mxfp4(aq, wq, out=view)
    torch.cuda.synchronize()
    _check(big, view, ref, n, dtype)


def test_out_shape_is_checked():
    a = torch.zeros(8, 256, dtype=torch.bfloat16, device="cuda")
    wq = fp4.quantize_fp4(torch.zeros(32, 256, device="cuda"), layout=fp4.LAYOUT_TILED)
    with pytest.raises(ValueError):
        fp4.gemm_w4aX(fp4.A4, a, wq, out=torch.empty(8, 48, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fp4.gemm_w4aX(fp4.A4, a, wq, out=torch.empty(32, 8, dtype=torch.bfloat16, device="cuda").t())


@pytest.mark.parametrize("kind", ["gemm", "mx"])
def test_largest_row_stride(kind):
    """Row stride at the boundary's limit, FP4_MAX_LDC = 2^21 float32 elements (8 MiB per
    row, 512 MiB for 64 rows): the 32-bit byte offsets of a tile's stores stay in range,
    and the results equal the contiguous ones bit for bit (ragged second row tile)."""
    m, n, k = 70, 272, 256
    ldc = 1 << 21
    rng = np.random.default_rng(3)
    print(f"[case] largest row stride {kind} {m}x{n}x{k} ldc={ldc}", flush=True)
    a = workloads.to_bf16_values(rng.standard_normal((m, k)).astype(np.float32))
    w = (0.05 * rng.standard_normal((n, k))).astype(np.float32)
    if kind == "gemm":
        wq = fp4.quantize_fp4(torch.from_numpy(w).cuda(), layout=fp4.LAYOUT_TILED)
        run = lambda out=None: fp4.gemm_w4aX(fp4.A4, to_device_bf16(a), wq, out_dtype=torch.float32, out=out)
    else:
        aq = fp4.quantize_mxfp4(to_device_bf16(a))
        wq = fp4.quantize_mxfp4(torch.from_numpy(w).cuda())
        run = lambda out=None: fp4.gemm_mxfp4(aq, wq, out_dtype=torch.float32, out=out)
    ref = run()
    big = torch.full((m, ldc), 3.0, dtype=torch.float32, device="cuda")
    view = big[:, :n]
    run(view)
    torch.cuda.synchronize()
    assert np.array_equal(host(view.contiguous()).view(np.uint32), host(ref).view(np.uint32))
    assert bool(torch.all(big[:, n:n + 4096] == 3.0)) and bool(torch.all(big[:, -4096:] == 3.0))
    del big
    torch.cuda.empty_cache()
