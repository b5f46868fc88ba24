"""GPU parity of quantize_fp4 / dequantize_fp4 against the oracle: packed codes, micro-
and macro-scales bit-exact (both layouts), dequantized values exact (float32) or
RNE-bf16-exact, on the workloads' inputs and on edge cases."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
import workloads
from tests._util import qtensor_to_canonical, host, to_device_bf16, bf16_values

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return to_device_bf16(x)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _input_values(t: torch.Tensor) -> np.ndarray:
    return host(t.to(torch.float32)).astype(np.float64)


def _check_quant(x_dev: torch.Tensor, elem: int, layout: int, rows_subset=None):
    rows, k = x_dev.shape
    q = fp4.quantize_fp4(x_dev, elem=elem, layout=layout)
    torch.cuda.synchronize()
    codes, micro, macro = qtensor_to_canonical(q, rows, k)
    xv = _input_values(x_dev)
    sel = np.arange(rows) if rows_subset is None else rows_subset
    ref = oracle.quantize(xv[sel], "e2m1" if elem == 0 else "e4m3")
    assert np.array_equal(macro[sel], ref.macro), "macro-scales differ"
    assert np.array_equal(micro[sel], ref.micro), "micro-scales differ"
    assert np.array_equal(codes[sel], ref.codes), "codes differ"
    return q, ref, sel


@pytest.mark.parametrize("layout", [0, 1])
def test_tiny_workload_weights_and_activations(layout):
    a, w = workloads.tiny()
    print(f"[case] tiny W{w.shape} A{a.shape} layout={layout}", flush=True)
    qw, refw, _ = _check_quant(_dev(w, "f32"), 0, layout)
    # dequantize is exact in float32
    y = host(fp4.dequantize_fp4(qw, torch.float32)).astype(np.float64)
    assert np.array_equal(y, oracle.dequantize(refw))
    yb = bf16_values(fp4.dequantize_fp4(qw, torch.bfloat16))
    assert np.array_equal(yb, F.bf16_round(oracle.dequantize(refw)))
    qa, refa, _ = _check_quant(_dev(a, "f32"), 0, 0)
    ya = host(fp4.dequantize_fp4(qa, torch.float32)).astype(np.float64)
    assert np.array_equal(ya, oracle.dequantize(refa))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("elem,layout", [(0, 0), (0, 1), (1, 0)])
def test_outlier_data_ragged_rows(dtype, elem, layout):
    rng = np.random.default_rng(101)
    rows = 48 if layout == 1 else 37
    k = 768
    x = rng.standard_normal((rows, k)).astype(np.float32) * np.exp(rng.uniform(-6, 6, (rows, 1))).astype(np.float32)
    x[:, rng.choice(k, 4, replace=False)] *= 100.0
    print(f"[case] outliers {rows}x{k} {dtype} elem={elem} layout={layout}", flush=True)
    q, ref, _ = _check_quant(_dev(x, dtype), elem, layout)
    y = host(fp4.dequantize_fp4(q, torch.float32)).astype(np.float64)
    assert np.array_equal(y, oracle.dequantize(ref))


def _edge_matrix():
    rng = np.random.default_rng(102)
    k = 512
    x = np.zeros((32, k), dtype=np.float32)
    x[1, 3] = -0.0                                   # all-zero group with a negative zero
    x[2] = rng.standard_normal(k) * 1e-12            # macro clamps to 2^-24
    x[3] = rng.standard_normal(k) * 3e37             # macro saturates at 65504
    x[4, :16] = 1000.0
    x[4, 16:32] = rng.standard_normal(16) * 1e-7     # micro-scale underflows to 0
    x[5] = np.float32(-0.0)
    x[5, 0] = 6.0                                    # negative zeros inside a live block
    x[6] = rng.standard_normal(k) * 0.02             # subnormal FP16 macro-scales
    # exact tie points t*s with M = 2^-8 and mu = 448 (s = 1.75), see the worked group
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * 1.75
    x[7, :256] = np.resize(np.concatenate([ties, -ties]), 256)
    # block maxima on micro-scale ties (group max 10.5 pins M = 2^-8)
    e4 = F.e4m3_decode(np.arange(0, 0x7F))
    mids = (e4[:-1] + e4[1:]) / 2
    x[8, 0] = 10.5
    for b in range(1, 16):
        x[8, 16 * b] = mids[8 + 7 * b] * 6 * 2.0 ** -8
        x[8, 16 * b + 1:16 * b + 16] = rng.uniform(-1, 1, 15) * x[8, 16 * b]
    x[9:] = rng.standard_normal((23, k)) * np.exp(rng.uniform(-20, 20, (23, 1)))
    return x


@pytest.mark.parametrize("elem,layout", [(0, 0), (0, 1), (1, 0)])
def test_edge_cases(elem, layout):
    x = _edge_matrix()
    print(f"[case] edge elem={elem} layout={layout}", flush=True)
    q, ref, _ = _check_quant(_dev(x, "f32"), elem, layout)
    y = host(fp4.dequantize_fp4(q, torch.float32)).astype(np.float64)
    assert np.array_equal(y, oracle.dequantize(ref))
    assert np.array_equal(np.signbit(y), np.signbit(oracle.dequantize(ref)))


def test_decode_workload_weights_full_size_sampled_rows():
    """The decode weights [14336 x 4096] quantized at full size in the tiled layout the
    product kernels read; the codes, micro-scales and macro-scales of 384 sampled rows
    are checked bit for bit against the oracle."""
    _, w, _ = workloads.decode()
    print("[case] decode weights 14336x4096 tiled", flush=True)
    sel = np.sort(np.random.default_rng(103).choice(w.shape[0], 384, replace=False))
    _check_quant(_dev(w, "f32"), 0, 1, rows_subset=sel)


def test_decode_weights_dequantized_full_size_sampled_rows():
    """Tiled E2M1 weights [14336 x 4096] dequantized at full size, in the one-tile-per-wave
    form the dequantize measurement times: 384 sampled rows are exact in float32 and
    RNE-bf16-exact, against the oracle's dequantization of the oracle's own codes."""
    _, w, _ = workloads.decode()
    print("[case] dequantize decode weights 14336x4096 tiled", flush=True)
    sel = np.sort(np.random.default_rng(105).choice(w.shape[0], 384, replace=False))
    q, ref, _ = _check_quant(_dev(w, "f32"), 0, 1, rows_subset=sel)
    want = oracle.dequantize(ref)
    y32 = host(fp4.dequantize_fp4(q, torch.float32)[torch.from_numpy(sel).cuda()]).astype(np.float64)
    assert np.array_equal(y32, want)
    y16 = bf16_values(fp4.dequantize_fp4(q, torch.bfloat16)[torch.from_numpy(sel).cuda()])
    assert np.array_equal(y16, F.bf16_round(want))


def test_prefill_activations_full_size_sampled_rows():
    a, _, _ = workloads.prefill()
    print("[case] prefill activations 2048x4096 bf16", flush=True)
    sel = np.sort(np.random.default_rng(104).choice(a.shape[0], 256, replace=False))
    for elem in (0, 1):
        _check_quant(_dev(a, "bf16"), elem, 0, rows_subset=sel)


def test_quantize_is_deterministic_and_strided():
    rng = np.random.default_rng(105)
    base = rng.standard_normal((64, 1024)).astype(np.float32)
    big = torch.zeros(64, 1280, device="cuda")
    big[:, :1024] = torch.from_numpy(base).cuda()
    view = big[:, :1024]  # row stride 1280
    q1 = fp4.quantize_fp4(view)
    q2 = fp4.quantize_fp4(torch.from_numpy(base).cuda())
    torch.cuda.synchronize()
    for a, b in ((q1.codes, q2.codes), (q1.micro, q2.micro), (q1.macro, q2.macro)):
        assert torch.equal(a, b)
