"""GPU parity of the sensitive-layer and static-scale paths against the CPU oracle, through
the C ABI: E4M3-element quantization in the tiled layout, static-macro-scale quantization,
activation macro-scale calibration, gemm_w8a8, gemm_w4aX_static and the two policy modes
that route to them.

Gates: codes, micro-scales, macro-scales and calibrated macro-scales bit-exact; float32
dequantization exact; float32 products within 1e-5 relative Frobenius error of the float64
oracle (every operand product is exact, only the float32 accumulation rounds); bf16
products through the bf16 gate. Full-size layers are checked on sampled rows and columns."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._util import host, to_device_bf16, bf16_values, bf16_gate, f32_gate, qtensor_to_canonical

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")

STATIC_CODE = {4: oracle.A4S, 8: oracle.A8S}
ELEM = {0: "e2m1", 1: "e4m3"}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _weights(rng, n, k):
    """N(0, 0.02) weights with blocks scaled far below their group maximum (subnormal E4M3
    micro-scales), a zero row (zero macro-scale) and a zero block."""
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    blocks = rng.choice(n * k // 16, max(1, n * k // 16 // 50), replace=False)
    wb = w.reshape(-1, 16)
    wb[blocks] *= np.float32(1e-5)
    w[1 % n] = 0.0
    w[2 % n, 16:32] = 0.0
    return w


def _acts(rng, m, k, dtype=torch.bfloat16):
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    a[0] = 0.0
    if dtype == torch.bfloat16:
        a = workloads.to_bf16_values(a)
    return a


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    return t.to(dtype) if dtype != torch.float32 else t


def _macro_dev(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).cuda()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,k", [(48, 768), (16, 256)])
def test_quantize_e4m3_tiled_bit_exact(dtype, rows, k):
    rng = np.random.default_rng(400 + rows + k)
    x = _weights(rng, rows, k)
    if dtype == torch.bfloat16:
        x = workloads.to_bf16_values(x)
    print(f"[case] quantize E4M3 tiled {rows}x{k} {dtype}", flush=True)
    q = fp4.quantize_fp4(_dev(x, dtype), elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
    codes, micro, macro = qtensor_to_canonical(q, rows, k)
    ref = oracle.quantize(x.astype(np.float64), "e4m3")
    assert np.array_equal(codes, ref.codes)
    assert np.array_equal(micro, ref.micro)
    assert np.array_equal(macro, ref.macro)
    assert (ref.micro[ref.micro > 0] < 8).any(), "no subnormal micro-scale exercised"
    y = host(fp4.dequantize_fp4(q, torch.float32)).astype(np.float64)
    assert np.array_equal(y, oracle.dequantize(ref))


@pytest.mark.parametrize("elem,layout", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_static_bit_exact(elem, layout, dtype):
    rng = np.random.default_rng(410 + 2 * elem + layout)
    rows, k = 32, 768
    x = _acts(rng, rows, k, dtype)
    # calibrated on a quarter of the range: the largest blocks saturate; group 2 calibrated
    # to zero (all codes 0)
    cal = oracle.calibrate_macro(0.25 * x.astype(np.float64), ELEM[elem])
    cal[2] = 0
    print(f"[case] quantize static {ELEM[elem]} layout={layout} {dtype}", flush=True)
    q = fp4.quantize_fp4_static(_dev(x, dtype), _macro_dev(cal), elem=elem, layout=layout)
    codes, micro, macro = qtensor_to_canonical(q, rows, k)
    ref = oracle.quantize_static(x.astype(np.float64), cal, ELEM[elem])
    assert np.array_equal(codes, ref.codes)
    assert np.array_equal(micro, ref.micro)
    assert np.array_equal(macro, ref.macro)
    assert (ref.micro == 0x7E).any(), "no saturated micro-scale exercised"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("elem", [0, 1])
def test_act_macro_calibrate_two_batches(dtype, elem):
    rng = np.random.default_rng(420 + elem)
    k = 1280
    b1 = _acts(rng, 100, k, dtype)
    b2 = _acts(rng, 37, k, torch.float32) * np.float32(3.0)
    if dtype == torch.bfloat16:
        b2 = workloads.to_bf16_values(b2)  # the device input must hold exactly these values
    b2[:, :256] = 0.0
    b1[:, :256] = 0.0  # an all-zero group: macro-scale 0
    print(f"[case] calibrate {ELEM[elem]} {dtype}", flush=True)
    amax = torch.zeros(k // 256, dtype=torch.float32, device="cuda")
    fp4.act_macro_calibrate(_dev(b1, dtype), amax, elem)
    m1 = host(amax).copy()
    macro = fp4.act_macro_calibrate(_dev(b2, dtype), amax, elem)
    both = np.concatenate([b1, b2]).astype(np.float64)
    assert np.array_equal(m1, np.abs(b1).reshape(100, -1, 256).max(axis=(0, 2)).astype(np.float32))
    assert np.array_equal(host(macro).view(np.uint16), oracle.calibrate_macro(both, ELEM[elem]))
    assert host(macro).view(np.uint16)[0] == 0


@pytest.mark.parametrize("m,n,k", [(200, 400, 768), (17, 128, 256), (130, 272, 1280), (64, 16, 512)])
def test_gemm_w8a8_small_shapes(m, n, k):
    rng = np.random.default_rng(430 + m + n + k)
    a = _acts(rng, m, k)
    w = _weights(rng, n, k)
    print(f"[case] gemm_w8a8 m={m} n={n} k={k}", flush=True)
    wq = fp4.quantize_fp4(_dev(w, torch.float32), elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
    ref = oracle.gemm_w8a8(a.astype(np.float64), oracle.quantize(w.astype(np.float64), "e4m3"))
    ad = to_device_bf16(a)
    f32_gate(host(fp4.gemm_w8a8(ad, wq, out_dtype=torch.float32)), ref)
    bf16_gate(bf16_values(fp4.gemm_w8a8(ad, wq)), oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("m,n,k", [(500, 4800, 512), (500, 4800, 1024), (505, 5008, 1536)])
def test_gemm_w8a8_ten_wave_ring(m, n, k):
    """W8A8 products whose 64 x 128 grid would put two workgroups on some CUs run the E4M3
    10-wave 64 x 160 form with its four-slot stage ring: 2, 4 and 6 groups (the ring's
    copies run past the last stage), a ragged last row tile, a 48-column last tile."""
    name = fp4.fp4_product_kernel(fp4.W8A8, torch.bfloat16, m, n, k, w_e4m3=True)
    assert name.startswith("k_gemm_w10e"), f"shape no longer selects the 10-wave form ({name})"
    rng = np.random.default_rng(440 + m + n + k)
    a = _acts(rng, m, k)
    w = _weights(rng, n, k)
    print(f"[case] gemm_w8a8 10-wave ring m={m} n={n} k={k}", flush=True)
    wq = fp4.quantize_fp4(_dev(w, torch.float32), elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
    ref = oracle.gemm_w8a8(a.astype(np.float64), oracle.quantize(w.astype(np.float64), "e4m3"))
    ad = to_device_bf16(a)
    f32_gate(host(fp4.gemm_w8a8(ad, wq, out_dtype=torch.float32)), ref)
    bf16_gate(bf16_values(fp4.gemm_w8a8(ad, wq)), oracle.formats.bf16_round(ref))


def test_gemm_w8a8_float32_activations():
    rng = np.random.default_rng(435)
    a = _acts(rng, 40, 512, torch.float32)
    w = _weights(rng, 96, 512)
    print("[case] gemm_w8a8 float32 activations", flush=True)
    wq = fp4.quantize_fp4(_dev(w, torch.float32), elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
    c = fp4.gemm_w8a8(_dev(a, torch.float32), wq, out_dtype=torch.float32)
    f32_gate(host(c), oracle.gemm_w8a8(a.astype(np.float64), oracle.quantize(w.astype(np.float64), "e4m3")))


@pytest.mark.parametrize("act", [4, 8])
@pytest.mark.parametrize("m,n,k", [(200, 400, 768), (17, 128, 256), (130, 272, 1280)])
def test_gemm_static_small_shapes(act, m, n, k):
    rng = np.random.default_rng(440 + act + m + n + k)
    a = _acts(rng, m, k)
    w = _weights(rng, n, k)
    cal = oracle.calibrate_macro(0.5 * _acts(rng, 64, k).astype(np.float64), "e2m1" if act == 4 else "e4m3")
    print(f"[case] gemm_w4aX_static A{act} m={m} n={n} k={k}", flush=True)
    wq = fp4.quantize_fp4(_dev(w, torch.float32), layout=fp4.LAYOUT_TILED)
    ref = oracle.gemm_static(a.astype(np.float64), oracle.quantize(w.astype(np.float64)), STATIC_CODE[act], cal)
    ad, md = to_device_bf16(a), _macro_dev(cal)
    f32_gate(host(fp4.gemm_w4aX_static(act, ad, md, wq, out_dtype=torch.float32)), ref)
    bf16_gate(bf16_values(fp4.gemm_w4aX_static(act, ad, md, wq)), oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("mode", [fp4.POLICY_SENSITIVE_W8, fp4.POLICY_STATIC])
def test_policy_modes_full_size_sampled(mode):
    """The 8-layer policy stack (512 x 5120 x 5120 per layer) under the two added modes:
    flagged layers W8A8 / static A8, the others W4A4 / static A4; static macro-scales are
    calibrated on the device from a separate calibration batch per layer."""
    cfg = workloads.WORKLOADS["policy_stack"]
    flags = workloads.policy_flags()
    rng = np.random.default_rng(450 + mode)
    for layer in range(cfg["layers"]):
        w, x = workloads.policy_layer(layer)
        code = fp4.fp4_policy_select(mode, bool(flags[layer]))
        assert code == oracle.policy_select_ext(mode, bool(flags[layer]))
        print(f"[case] policy mode={mode} layer={layer} code={code}", flush=True)
        rows = np.sort(rng.choice(x.shape[0], 32, replace=False))
        cols = np.sort(rng.choice(w.shape[0], 128, replace=False))
        xd = to_device_bf16(x)
        if code == fp4.W8A8:
            wq = fp4.quantize_fp4(_dev(w, torch.float32), elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
            c = fp4.gemm_w8a8(xd, wq)
            ref = oracle.gemm_w8a8(x[rows].astype(np.float64), oracle.quantize(w[cols].astype(np.float64), "e4m3"))
        elif code == fp4.A4:
            c = fp4.gemm_w4aX(fp4.A4, xd, fp4.quantize_fp4(_dev(w, torch.float32), layout=fp4.LAYOUT_TILED))
            ref = oracle.gemm(x[rows].astype(np.float64), oracle.quantize(w[cols].astype(np.float64)), oracle.A4)
        else:
            act = 8 if code == fp4.A8S else 4
            calib = workloads.policy_calibration(layer, rows=cfg["calib_rows"])
            amax = torch.zeros(w.shape[1] // 256, dtype=torch.float32, device="cuda")
            macro = fp4.act_macro_calibrate(to_device_bf16(calib), amax, 1 if act == 8 else 0)
            cal = oracle.calibrate_macro(calib.astype(np.float64), "e4m3" if act == 8 else "e2m1")
            assert np.array_equal(host(macro).view(np.uint16), cal)
            c = fp4.gemm_w4aX_static(act, xd, macro, fp4.quantize_fp4(_dev(w, torch.float32), layout=fp4.LAYOUT_TILED))
            ref = oracle.gemm_static(x[rows].astype(np.float64), oracle.quantize(w[cols].astype(np.float64)), code, cal)
        bf16_gate(bf16_values(c)[np.ix_(rows, cols)], oracle.formats.bf16_round(ref))


def test_w8a8_deterministic():
    rng = np.random.default_rng(460)
    a = _acts(rng, 130, 1280)
    w = _weights(rng, 272, 1280)
    wq = fp4.quantize_fp4(_dev(w, torch.float32), elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
    ad = to_device_bf16(a)
    print("[case] gemm_w8a8 determinism", flush=True)
    c1 = fp4.gemm_w8a8(ad, wq, out_dtype=torch.float32)
    c2 = fp4.gemm_w8a8(ad, wq, out_dtype=torch.float32)
    assert torch.equal(c1, c2)
