"""GPU parity of repack_fp4 (canonical <-> tiled layout, E2M1 and E4M3 elements) through
the C ABI.

Gates (integer work, so bit-exact throughout):
  - canonical -> tiled equals the tiled layout's definition (include/fp4_e2m1.h, written
    out as index maps in tests/_util.py) applied to the canonical bytes, for codes, micro-
    and macro-scales; tiled -> canonical is its inverse; a round trip returns the
    original bytes;
  - on the decode weights (14336 x 4096, 0.1% outlier input channels) and on outlier-heavy
    data, repacking quantize_fp4's canonical output gives quantize_fp4's tiled output
    byte for byte, while re-quantizing the dequantized tensor does not (the reason the
    repack exists: bf16 dequantized values are re-rounded, and with E4M3 elements a
    block maximum that rounds down changes the micro-scale);
  - a W4A4 product on repacked weights passes the bf16 gate against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._util import host, tiled_index_maps, tiled8_code_index, to_device_bf16, bf16_values, bf16_gate

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _random_qtensor(rng, rows, k, elem, layout):
    ncodes = rows * k // 2 if elem == fp4.ELEM_E2M1 else rows * k
    u8 = lambda n: torch.from_numpy(rng.integers(0, 256, n, dtype=np.uint8)).cuda()
    macro = torch.from_numpy(rng.integers(-32768, 32768, rows * k // 256, dtype=np.int16)).cuda()
    return fp4.QTensor(u8(ncodes), u8(rows * k // 16), macro, rows, k, elem, layout)


def _maps(rows, k, elem):
    ci, mi, gi = tiled_index_maps(rows, k)
    if elem == fp4.ELEM_E4M3:
        ci = tiled8_code_index(rows, k)
    return ci, mi, gi


@pytest.mark.parametrize("elem", [0, 1])
@pytest.mark.parametrize("rows,k", [(16, 256), (48, 768), (32, 1280), (1040, 4096)])
def test_repack_is_the_documented_permutation(elem, rows, k):
    rng = np.random.default_rng(900 + 7 * elem + rows + k)
    print(f"[case] repack elem={elem} rows={rows} k={k}", flush=True)
    can = _random_qtensor(rng, rows, k, elem, fp4.LAYOUT_CANONICAL)
    til = fp4.repack_fp4(can, fp4.LAYOUT_TILED)
    ci, mi, gi = _maps(rows, k, elem)
    codes_c, micro_c, macro_c = host(can.codes), host(can.micro), host(can.macro)
    codes_t, micro_t, macro_t = host(til.codes), host(til.micro), host(til.macro)
    # canonical = tiled[I]: every canonical byte sits where the definition puts it
    assert np.array_equal(codes_t[ci].reshape(-1), codes_c)
    assert np.array_equal(micro_t[mi].reshape(-1), micro_c)
    assert np.array_equal(macro_t[gi].reshape(-1), macro_c)
    # and back: tiled -> canonical is the inverse, so the round trip is the identity
    back = fp4.repack_fp4(til, fp4.LAYOUT_CANONICAL)
    for a, b in ((back.codes, can.codes), (back.micro, can.micro), (back.macro, can.macro)):
        assert torch.equal(a, b)
    # tiled -> canonical -> tiled from a random tiled tensor
    til2 = _random_qtensor(rng, rows, k, elem, fp4.LAYOUT_TILED)
    rt = fp4.repack_fp4(fp4.repack_fp4(til2, fp4.LAYOUT_CANONICAL), fp4.LAYOUT_TILED)
    for a, b in ((rt.codes, til2.codes), (rt.micro, til2.micro), (rt.macro, til2.macro)):
        assert torch.equal(a, b)


def _outlier_matrix(rng, rows, k):
    x = (0.02 * rng.standard_normal((rows, k))).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 64), replace=False)] *= 100
    return x


@pytest.mark.parametrize("elem", [0, 1])
def test_repack_equals_tiled_quantization_where_requantizing_is_lossy(elem):
    rng = np.random.default_rng(910 + elem)
    rows, k = 512, 2048
    x = torch.from_numpy(_outlier_matrix(rng, rows, k)).cuda()
    print(f"[case] repack vs tiled quantize, outliers, elem={elem}", flush=True)
    can = fp4.quantize_fp4(x, elem=elem, layout=fp4.LAYOUT_CANONICAL)
    til = fp4.quantize_fp4(x, elem=elem, layout=fp4.LAYOUT_TILED)
    rep = fp4.repack_fp4(can, fp4.LAYOUT_TILED)
    for a, b in ((rep.codes, til.codes), (rep.micro, til.micro), (rep.macro, til.macro)):
        assert torch.equal(a, b)
    # re-quantizing dequantized values is not the same tensor: E2M1 after a bf16
    # dequantize (values re-rounded to 8 bits); E4M3 elements even after an exact float32
    # one (a block maximum that rounds down to 416 changes the block's micro-scale)
    dq_dtype = torch.bfloat16 if elem == fp4.ELEM_E2M1 else torch.float32
    req = fp4.quantize_fp4(fp4.dequantize_fp4(can, dq_dtype), elem=elem, layout=fp4.LAYOUT_TILED)
    differ = sum(int((a != b).sum()) for a, b in ((req.codes, til.codes), (req.micro, til.micro),
                                                  (req.macro, til.macro)))
    assert differ > 0, "re-quantization happened to be lossless on this data"
    print(f"  re-quantizing ({dq_dtype}) changes {differ} code bytes and scales; the repack changes none",
          flush=True)


def test_repack_decode_weights_full_size():
    _, w, _ = workloads.decode()
    print("[case] repack decode weights 14336x4096 canonical -> tiled", flush=True)
    wd = torch.from_numpy(w).cuda()
    del w
    can = fp4.quantize_fp4(wd, layout=fp4.LAYOUT_CANONICAL)
    til = fp4.quantize_fp4(wd, layout=fp4.LAYOUT_TILED)
    rep = fp4.repack_fp4(can, fp4.LAYOUT_TILED)
    for a, b in ((rep.codes, til.codes), (rep.micro, til.micro), (rep.macro, til.macro)):
        assert torch.equal(a, b)
    back = fp4.repack_fp4(til, fp4.LAYOUT_CANONICAL)
    for a, b in ((back.codes, can.codes), (back.micro, can.micro), (back.macro, can.macro)):
        assert torch.equal(a, b)


def test_product_on_repacked_weights():
    """Weights quantized by the oracle into the canonical layout (the interchange form a
    checkpoint would hold), copied to the device, repacked, multiplied (W4A4)."""
    rng = np.random.default_rng(920)
    m, n, k = 96, 272, 1024
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = _outlier_matrix(rng, n, k)
    print(f"[case] W4A4 product on repacked oracle weights m={m} n={n} k={k}", flush=True)
    q = oracle.quantize(w.astype(np.float64))
    can = fp4.QTensor(torch.from_numpy(np.ascontiguousarray(q.codes, np.uint8).reshape(-1)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(q.micro, np.uint8).reshape(-1)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(q.macro, np.uint16).reshape(-1).view(np.int16)).cuda(),
                      n, k, fp4.ELEM_E2M1, fp4.LAYOUT_CANONICAL)
    wq = fp4.repack_fp4(can, fp4.LAYOUT_TILED)
    c = fp4.gemm_w4aX(fp4.A4, to_device_bf16(a), wq)
    ref = oracle.gemm(a.astype(np.float64), q, oracle.A4)
    bf16_gate(bf16_values(c), oracle.formats.bf16_round(ref))


def test_repack_rejects_bad_arguments():
    rng = np.random.default_rng(930)
    can = _random_qtensor(rng, 16, 256, 0, fp4.LAYOUT_CANONICAL)
    with pytest.raises(fp4.Fp4Error):  # same layout
        fp4.repack_fp4(can, fp4.LAYOUT_CANONICAL, out=fp4.empty_qtensor(16, 256))
    odd = fp4.QTensor(can.codes, can.micro, can.macro, 8, 512, 0, fp4.LAYOUT_CANONICAL)
    with pytest.raises(fp4.Fp4Error):  # rows % 16
        fp4.repack_fp4(odd, fp4.LAYOUT_TILED)
