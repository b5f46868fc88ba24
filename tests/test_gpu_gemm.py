"""GPU parity of gemm_w4aX (W4A16 decode / W4A16 / W4A8 / W4A4) and grouped_gemm_w4aX
against the float64 oracle, through the C ABI.

Gates (float32 accumulation on exact operands):
  float32 output: ||C - C64||_F / ||C64||_F <= 1e-5
  bf16 output:    ||C - RNE_bf16(C64)||_F / ||RNE_bf16(C64)||_F <= 1e-3 and >= 99.9% of
                  elements equal to RNE_bf16(C64) or one bf16 step away.
Full-size workloads are checked on sampled rows/columns that the oracle computes one by
one; small shapes (several tiles plus ragged tails) are checked in full. Each kernel form
is reached by a shape chosen for it (fp4_product_kernel names the form a shape runs, and
the tests assert it): small dense products run the narrow 64 x 128 tile, 500-row products
the 10-wave 64 x 160 form, large ones (the prefill among them) the 128-row-wave 128 x 256
form, large ones above k = 8192 the 16-wave 64 x 512 form, k > 13056 the 64 x 256 form;
grouped products run the grouped 64 x 256 form. All forms agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._util import host, to_device_bf16, bf16_values, bf16_gate, f32_gate

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")

ACTS = {16: "A16", 8: "A8", 4: "A4"}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _wq(w: np.ndarray) -> "fp4.QTensor":
    return fp4.quantize_fp4(torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(),
                            layout=fp4.LAYOUT_TILED)


def _oracle_c(a_vals: np.ndarray, w: np.ndarray, act: int) -> np.ndarray:
    return oracle.gemm(a_vals, oracle.quantize(w.astype(np.float64)), act)


def test_tiny_w4a16_fp32():
    a, w = workloads.tiny()
    print("[case] tiny W4A16 fp32 16x512x256", flush=True)
    c = fp4.gemm_w4aX(fp4.A16, torch.from_numpy(a).cuda(), _wq(w), out_dtype=torch.float32)
    f32_gate(host(c), _oracle_c(a.astype(np.float64), w, oracle.A16))


@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("k,n", [(256, 16), (1024, 48), (4096, 1024), (8192, 64)])
def test_decode_gemv_shapes(m, k, n):
    rng = np.random.default_rng(200 + m + k + n)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[:, rng.choice(k, 2, replace=False)] *= 100
    a = workloads.to_bf16_values(rng.standard_normal((m, k)).astype(np.float32))
    print(f"[case] gemv m={m} k={k} n={n}", flush=True)
    wq = _wq(w)
    ad = to_device_bf16(a)
    ref = _oracle_c(a.astype(np.float64), w, oracle.A16)
    f32_gate(host(fp4.gemm_w4aX(fp4.A16, ad, wq, out_dtype=torch.float32)), ref)
    bf16_gate(bf16_values(fp4.gemm_w4aX(fp4.A16, ad, wq)), oracle.formats.bf16_round(ref))


def test_decode_workload_full_size_sampled():
    a, w, _ = workloads.decode()
    print("[case] decode W4A16 8x4096x14336 (sampled columns)", flush=True)
    wq = _wq(w)
    c = fp4.gemm_w4aX(fp4.A16, to_device_bf16(a), wq)
    cols = np.sort(np.random.default_rng(201).choice(w.shape[0], 512, replace=False))
    ref = _oracle_c(a.astype(np.float64), w[cols], oracle.A16)
    bf16_gate(bf16_values(c)[:, cols], oracle.formats.bf16_round(ref))


# row-block counts that leave the last workgroup partly empty, at shapes large enough
# for workgroups of two and four row blocks (k-runs of 1 to 8 waves)
@pytest.mark.parametrize("m,k,n", [(5, 4096, 12304), (8, 2048, 8208), (3, 8192, 8208), (8, 1024, 12304)])
def test_decode_gemv_wide_workgroups_ragged(m, k, n):
    rng = np.random.default_rng(210 + m + k + n)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[:, rng.choice(k, 4, replace=False)] *= 100
    a = workloads.to_bf16_values(rng.standard_normal((m, k)).astype(np.float32))
    print(f"[case] gemv wide workgroups m={m} k={k} n={n}", flush=True)
    wq = _wq(w)
    ad = to_device_bf16(a)
    cols = np.union1d(rng.choice(n - 16, 368, replace=False), np.arange(n - 16, n))
    ref = _oracle_c(a.astype(np.float64), w[cols], oracle.A16)
    f32_gate(host(fp4.gemm_w4aX(fp4.A16, ad, wq, out_dtype=torch.float32))[:, cols], ref)
    bf16_gate(bf16_values(fp4.gemm_w4aX(fp4.A16, ad, wq))[:, cols], oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("act", [16, 8, 4])
@pytest.mark.parametrize("m,n,k", [(200, 400, 768), (17, 128, 256), (130, 272, 1280)])
def test_gemm_small_shapes(act, m, n, k):
    rng = np.random.default_rng(300 + act + m + n + k)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm {ACTS[act]} m={m} n={n} k={k}", flush=True)
    wq = _wq(w)
    ad = to_device_bf16(a)
    ref = _oracle_c(a.astype(np.float64), w, act)
    f32_gate(host(fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32)), ref)
    bf16_gate(bf16_values(fp4.gemm_w4aX(act, ad, wq)), oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("act", [16, 8, 4])
@pytest.mark.parametrize("k", [256, 1024, 2816])
def test_gemm_r8_tiles_ragged(act, k):
    """Small products take the narrow 64 x 128 tile; this shape (2043 x 4080: 16 x 16 tiles
    of 128 x 256, the last row and column tiles ragged) is large enough for the 128-row-
    wave form. k = 1024 and 2816 cross 3 and 10 group boundaries (an odd group count ends
    the form's six-stage pass early), so the per-group rescale of both the bf16 (A16) and
    the FP16 (A4 / A8) operand paths runs in it."""
    m, n = 2043, 4080
    name = fp4.fp4_product_kernel(act, torch.bfloat16, m, n, k)
    assert name.startswith("k_gemm_r8"), f"shape no longer selects the 128-row-wave form ({name})"
    rng = np.random.default_rng(310 + act + k)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm 128x256 tiles {ACTS[act]} m={m} n={n} k={k} ({name})", flush=True)
    wq = _wq(w)
    ad = to_device_bf16(a)
    ref = _oracle_c(a.astype(np.float64), w, act)
    f32_gate(host(fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32)), ref)
    bf16_gate(bf16_values(fp4.gemm_w4aX(act, ad, wq)), oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("act", [16, 4])
def test_gemm_wide_512_tiles_large_k_sampled(act):
    """Above k = 8192 the 128-row-wave form's LDS no longer holds its row-factor table, so a
    large dense product (2043 x 4080, ragged) runs the 16-wave 64 x 512 form up to
    k = 13056; k = 8448 (33 groups) checked on sampled rows and columns, the last row and
    column tiles among them."""
    m, n, k = 2043, 4080, 8448
    name = fp4.fp4_product_kernel(act, torch.bfloat16, m, n, k)
    assert name.startswith("k_gemm_w16"), f"shape no longer selects the 16-wave form ({name})"
    rng = np.random.default_rng(315 + act)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 5, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm 64x512 tiles large k {ACTS[act]} m={m} n={n} k={k} (sampled)", flush=True)
    c = fp4.gemm_w4aX(act, to_device_bf16(a), _wq(w), out_dtype=torch.float32)
    rows = np.union1d(rng.choice(m - 64, 24, replace=False), np.arange(m - 11, m))
    cols = np.union1d(rng.choice(n - 512, 48, replace=False), np.arange(n - 496, n, 31))
    ref = _oracle_c(a[rows].astype(np.float64), w[cols], act)
    f32_gate(host(c)[np.ix_(rows, cols)], ref)


@pytest.mark.parametrize("act", [16, 4])
def test_gemm_forms_agree_bit_for_bit(act):
    """Every kernel form gives each output element the same operations in the same order
    (the 16x16x32 MFMA steps in k order, the same per-group rescale), so the same product
    computed through different forms is identical bit for bit: the full 2043 x 4080 x 1024
    product (128-row-wave form), a 64-row slice of it (narrow 64 x 128 form) and two
    576-row slices (10-wave 64 x 160 form) with the same weights, compared on the rows they
    share."""
    m, n, k = 2043, 4080, 1024
    rng = np.random.default_rng(340 + act)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    ad = to_device_bf16(workloads.to_bf16_values(a))
    wq = _wq((0.02 * rng.standard_normal((n, k))).astype(np.float32))
    full = fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32)
    seen = {fp4.fp4_product_kernel(act, torch.bfloat16, m, n, k)}
    for r0, r1 in ((1979, 2043), (0, 576), (1024, 1600)):
        name = fp4.fp4_product_kernel(act, torch.bfloat16, r1 - r0, n, k)
        seen.add(name)
        print(f"[case] forms agree {ACTS[act]} rows {r0}:{r1} ({name})", flush=True)
        part = fp4.gemm_w4aX(act, ad[r0:r1].contiguous(), wq, out_dtype=torch.float32)
        assert torch.equal(part, full[r0:r1]), f"rows {r0}:{r1} ({name}) differ from the full product"
    assert len(seen) == 3, f"the slices no longer exercise three different forms: {seen}"


@pytest.mark.parametrize("act", [4, 8, 16])
@pytest.mark.parametrize("m,n,k", [(500, 4800, 512), (500, 4800, 1024), (505, 5008, 1536)])
def test_gemm_ten_wave_ring_ragged(m, n, k, act):
    """Products whose 64 x 128 grid would put two workgroups on some CUs while the 64 x 160
    grid fits one per CU run the 10-wave form with its four-slot stage ring. Here 2, 4 and
    6 groups (the ring's copies run past the last stage; at 2 groups all but one copy
    after the prologue does), a ragged last row tile, and in 5008 a last column tile of
    48 columns."""
    name = fp4.fp4_product_kernel(act, torch.bfloat16, m, n, k)
    assert name.startswith("k_gemm_w10 "), f"shape no longer selects the 10-wave form ({name})"
    rng = np.random.default_rng(330 + act + k)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm 10-wave ring {ACTS[act]} m={m} n={n} k={k}", flush=True)
    wq = _wq(w)
    ad = to_device_bf16(a)
    ref = _oracle_c(a.astype(np.float64), w, act)
    f32_gate(host(fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32)), ref)
    bf16_gate(bf16_values(fp4.gemm_w4aX(act, ad, wq)), oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("act", [4, 8, 16])
def test_gemm_ten_wave_zero_groups(act):
    """The 10-wave form's group-boundary factors where macro-scales are zero (a zero factor
    counts as 1): a weight row with every group zero, weight rows and activation rows with
    one zero group in the middle (ratios into and out of it), a zero activation row."""
    m, n, k = 500, 4800, 1536
    name = fp4.fp4_product_kernel(act, torch.bfloat16, m, n, k)
    assert name.startswith("k_gemm_w10 "), f"shape no longer selects the 10-wave form ({name})"
    rng = np.random.default_rng(660 + act)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    a[7] = 0.0
    a[11, 512:768] = 0.0
    a[300, 0:256] = 0.0
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[3] = 0.0
    w[17, 256:512] = 0.0
    w[4799, 1280:1536] = 0.0
    w[160:176, 768:1024] = 0.0  # one whole 16-row block's group (another workgroup's tile)
    print(f"[case] gemm 10-wave zero groups {ACTS[act]} m={m} n={n} k={k}", flush=True)
    wq = _wq(w)
    ad = to_device_bf16(a)
    ref = _oracle_c(a.astype(np.float64), w, act)
    got = host(fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32))
    assert np.all(got[7] == 0.0) and np.all(got[:, 3] == 0.0)
    f32_gate(got, ref)
    bf16_gate(bf16_values(fp4.gemm_w4aX(act, ad, wq)), oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("act", [16, 4])
def test_gemm_wide_tiles_large_k_sampled(act):
    """At k = 13312 (52 groups) the 64 x 512 form's macro-scale table no longer fits its LDS,
    so a large dense product (1040 x 8192: 17 x 32 tiles of 64 x 256, the last row tile
    ragged) runs the 8-wave 64 x 256 form; checked on sampled outputs, the last row and
    column tiles among them."""
    m, n, k = 1040, 8192, 13312
    name = fp4.fp4_product_kernel(act, torch.bfloat16, m, n, k)
    assert name == "k_gemm (64 x 256, 8 waves)", f"shape no longer selects the 64 x 256 form ({name})"
    rng = np.random.default_rng(320 + act)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 5, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm wide tiles large k {ACTS[act]} m={m} n={n} k={k} (sampled)", flush=True)
    c = fp4.gemm_w4aX(act, to_device_bf16(a), _wq(w), out_dtype=torch.float32)
    rows = np.union1d(rng.choice(m - 16, 24, replace=False), np.arange(m - 16, m))
    cols = np.union1d(rng.choice(n - 256, 56, replace=False), np.arange(n - 256, n, 32))
    ref = _oracle_c(a[rows].astype(np.float64), w[cols], act)
    f32_gate(host(c)[np.ix_(rows, cols)], ref)


def test_gemm_float32_activations_a4():
    rng = np.random.default_rng(302)
    a = rng.standard_normal((40, 512)).astype(np.float32)
    w = (0.02 * rng.standard_normal((64, 512))).astype(np.float32)
    print("[case] gemm A4 float32 activations", flush=True)
    c = fp4.gemm_w4aX(fp4.A4, torch.from_numpy(a).cuda(), _wq(w), out_dtype=torch.float32)
    f32_gate(host(c), _oracle_c(a.astype(np.float64), w, oracle.A4))


def test_gemm_float32_activations_a4_packed_form():
    """float32 activations on the W4A4 large-product form (the activation pass quantizes
    float32 input to packed E2M1, the product kernel decodes it): oracle gate, and equal
    bit for bit to the same activations given as bf16 when they are bf16 values."""
    rng = np.random.default_rng(303)
    m, n, k = 2043, 4080, 1024
    name = fp4.fp4_product_kernel(fp4.A4, torch.float32, m, n, k)
    assert "decoded in the kernel" in name, name
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm A4 float32 activations, packed form m={m} n={n} k={k}", flush=True)
    wq = _wq(w)
    c = host(fp4.gemm_w4aX(fp4.A4, torch.from_numpy(a).cuda(), wq, out_dtype=torch.float32))
    rows = np.r_[0:40, m - 40:m]
    f32_gate(c[rows], _oracle_c(a[rows].astype(np.float64), w, oracle.A4))
    ab = workloads.to_bf16_values(a)
    c32 = fp4.gemm_w4aX(fp4.A4, torch.from_numpy(ab).cuda(), wq, out_dtype=torch.float32)
    cbf = fp4.gemm_w4aX(fp4.A4, to_device_bf16(ab), wq, out_dtype=torch.float32)
    assert torch.equal(c32, cbf)


def test_prefill_w4a4_full_size_sampled():
    a, w, _ = workloads.prefill()
    print("[case] prefill W4A4 2048x4096x4096 (sampled)", flush=True)
    c = fp4.gemm_w4aX(fp4.A4, to_device_bf16(a), _wq(w))
    rng = np.random.default_rng(203)
    rows = np.sort(rng.choice(a.shape[0], 96, replace=False))
    cols = np.sort(rng.choice(w.shape[0], 384, replace=False))
    ref = _oracle_c(a[rows].astype(np.float64), w[cols], oracle.A4)
    bf16_gate(bf16_values(c)[np.ix_(rows, cols)], oracle.formats.bf16_round(ref))


@pytest.mark.parametrize("mode", [fp4.POLICY_AUTO, fp4.POLICY_Q4, fp4.POLICY_Q8])
def test_policy_stack_full_size_sampled(mode):
    flags = workloads.policy_flags()
    rng = np.random.default_rng(204 + mode)
    for layer in range(8):
        w, x = workloads.policy_layer(layer)
        act = fp4.fp4_policy_select(mode, bool(flags[layer]))
        assert act == oracle.policy_select(mode, bool(flags[layer]))
        print(f"[case] policy mode={mode} layer={layer} act={ACTS[act]}", flush=True)
        c = fp4.gemm_w4aX(act, to_device_bf16(x), _wq(w))
        rows = np.sort(rng.choice(x.shape[0], 32, replace=False))
        cols = np.sort(rng.choice(w.shape[0], 128, replace=False))
        ref = _oracle_c(x[rows].astype(np.float64), w[cols], act)
        bf16_gate(bf16_values(c)[np.ix_(rows, cols)], oracle.formats.bf16_round(ref))
        if mode != fp4.POLICY_AUTO:
            break  # forced modes: one layer is enough


def _grouped_case(act, tokens, experts, top_k, k, n, seed, with_token_map=True):
    logits = workloads.moe_router_logits(tokens=tokens, experts=experts, seed=seed)
    _, _, offsets, row_token, _ = oracle.route(logits, top_k)
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((tokens, k)).astype(np.float32)
    a[:, rng.choice(k, 2, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((experts * n, k))).astype(np.float32)
    R = int(offsets[-1])
    if not with_token_map:
        a = a[row_token]
    wq = _wq(w)
    c = fp4.grouped_gemm_w4aX(act, to_device_bf16(a),
                              torch.from_numpy(row_token).cuda() if with_token_map else None,
                              torch.from_numpy(offsets).cuda(), experts, R, wq,
                              out_dtype=torch.float32)
    got = host(c)
    ref = oracle.grouped_gemm(a.astype(np.float64), row_token if with_token_map else None,
                              offsets, oracle.quantize(w.astype(np.float64)), experts, act)
    full = np.concatenate([ref[e] for e in range(experts)], axis=0)
    f32_gate(got, full)
    return offsets


@pytest.mark.parametrize("act", [4, 8, 16])
@pytest.mark.parametrize("with_token_map", [True, False])
def test_grouped_small(act, with_token_map):
    print(f"[case] grouped {ACTS[act]} token_map={with_token_map}", flush=True)
    offsets = _grouped_case(act, tokens=420, experts=5, top_k=2, k=512, n=144, seed=7,
                            with_token_map=with_token_map)
    assert np.any(np.diff(offsets) > 128)  # some expert spans several row tiles


def test_grouped_empty_expert_and_many_experts():
    print("[case] grouped with empty experts, 100 experts", flush=True)
    offsets = _grouped_case(4, tokens=40, experts=100, top_k=2, k=256, n=32, seed=11)
    assert np.any(np.diff(offsets) == 0)


@pytest.mark.parametrize("act", [4, 8, 16])
@pytest.mark.parametrize("with_token_map", [True, False])
def test_grouped_agrees_with_dense_bit_for_bit(act, with_token_map):
    """A grouped product of 8192 routed rows over 40 uneven experts (one empty, every
    expert's rows ragged at its end; n = 1024, k = 768: 3 groups, an odd count): each
    expert's rows equal, bit for bit, the dense product of those rows alone, and two experts
    pass the float32 gate against the oracle."""
    tokens, experts, top_k, k, n, seed = 2048, 40, 4, 768, 1024, 23
    logits = workloads.moe_router_logits(tokens=tokens, experts=experts, seed=seed)
    logits[:, 7] = -np.inf  # expert 7 receives no rows
    _, _, offsets, row_token, _ = oracle.route(logits, top_k)
    R = int(offsets[-1])
    name = fp4.fp4_product_kernel(act, torch.bfloat16, R, n, k, grouped=True, n_experts=experts)
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((tokens, k)).astype(np.float32)
    a[:, rng.choice(k, 2, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((experts * n, k))).astype(np.float32)
    print(f"[case] grouped vs dense {ACTS[act]} token_map={with_token_map} R={R} ({name})", flush=True)
    a_rows = a if with_token_map else a[row_token]
    wq = _wq(w)
    off = torch.from_numpy(offsets).cuda()
    c = host(fp4.grouped_gemm_w4aX(act, to_device_bf16(a_rows),
                                   torch.from_numpy(row_token).cuda() if with_token_map else None,
                                   off, experts, R, wq, out_dtype=torch.float32))
    counts = np.diff(offsets)
    assert counts[7] == 0 and np.any(counts % 64 != 0)
    for e in range(experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        sub = fp4.QTensor(wq.codes[e * n * k // 2:(e + 1) * n * k // 2], wq.micro[e * n * k // 16:(e + 1) * n * k // 16],
                          wq.macro[e * n * k // 256:(e + 1) * n * k // 256], n, k, 0, fp4.LAYOUT_TILED)
        dense = host(fp4.gemm_w4aX(act, to_device_bf16(a[row_token[lo:hi]]), sub, out_dtype=torch.float32))
        assert np.array_equal(c[lo:hi].view(np.uint32), dense.view(np.uint32)), f"expert {e} differs"
    for e in (int(np.argmax(counts)), 11):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        ref = oracle.gemm(a[row_token[lo:hi]].astype(np.float64),
                          oracle.quantize(w[e * n:(e + 1) * n].astype(np.float64)), act)
        f32_gate(c[lo:hi], ref)


def test_moe_workload_full_size_subset_of_experts():
    cfg = workloads.WORKLOADS["moe_w4a4"]
    E, H, I, T = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["tokens"]
    _, _, offsets, row_token, _ = oracle.route(workloads.moe_router_logits(), cfg["top_k"])
    R = int(offsets[-1])
    x = workloads.moe_tokens()
    counts = np.diff(offsets)
    picks = sorted({int(np.argmin(counts)), int(np.argmax(counts)), 5, 77})
    print(f"[case] MoE W4A4 full size, experts checked {picks}", flush=True)
    w1q = fp4.empty_qtensor(E * 2 * I, H, layout=fp4.LAYOUT_TILED)
    w2q = fp4.empty_qtensor(E * H, I, layout=fp4.LAYOUT_TILED)
    w1_keep, w2_keep = {}, {}
    for e in range(E):
        w1, w2 = workloads.moe_expert_weights(e)
        for wt, q, keep in ((w1, w1q, w1_keep), (w2, w2q, w2_keep)):
            rows, k = wt.shape
            sub = fp4.QTensor(q.codes[e * rows * k // 2:(e + 1) * rows * k // 2],
                              q.micro[e * rows * k // 16:(e + 1) * rows * k // 16],
                              q.macro[e * rows * k // 256:(e + 1) * rows * k // 256],
                              rows, k, 0, fp4.LAYOUT_TILED)
            fp4.quantize_fp4(torch.from_numpy(wt).cuda(), layout=fp4.LAYOUT_TILED, out=sub)
            if e in picks:
                keep[e] = wt
    xd = to_device_bf16(x)
    rt = torch.from_numpy(row_token).cuda()
    off = torch.from_numpy(offsets).cuda()
    y1 = fp4.grouped_gemm_w4aX(fp4.A4, xd, rt, off, E, R, w1q)
    x2 = workloads.moe_down_inputs(R)
    y2 = fp4.grouped_gemm_w4aX(fp4.A4, to_device_bf16(x2), None, off, E, R, w2q)
    y1h, y2h = bf16_values(y1), bf16_values(y2)
    for e in picks:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        r1 = oracle.gemm(x[row_token[lo:hi]].astype(np.float64),
                         oracle.quantize(w1_keep[e].astype(np.float64)), oracle.A4)
        r2 = oracle.gemm(x2[lo:hi].astype(np.float64),
                         oracle.quantize(w2_keep[e].astype(np.float64)), oracle.A4)
        if hi > lo:
            bf16_gate(y1h[lo:hi], oracle.formats.bf16_round(r1))
            bf16_gate(y2h[lo:hi], oracle.formats.bf16_round(r2))


@pytest.mark.parametrize("act", [8, 4])
def test_gemm_small_m_odd_groups(act):
    """A small-m dense product with an odd group count (7) and ragged m and n: full
    parity and bit-identical repeats."""
    m, n, k = 150, 784, 1792
    rng = np.random.default_rng(500 + act)
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 5, replace=False)] *= 50
    a = workloads.to_bf16_values(a)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    print(f"[case] gemm small-m {ACTS[act]} m={m} n={n} k={k}", flush=True)
    wq, ad = _wq(w), to_device_bf16(a)
    ref = _oracle_c(a.astype(np.float64), w, act)
    c1 = fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32)
    f32_gate(host(c1), ref)
    for _ in range(3):
        assert torch.equal(c1, fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32))
    bf16_gate(bf16_values(fp4.gemm_w4aX(act, ad, wq)), oracle.formats.bf16_round(ref))


def test_gemm_deterministic():
    rng = np.random.default_rng(400)
    a = workloads.to_bf16_values(rng.standard_normal((300, 1024)).astype(np.float32))
    w = (0.02 * rng.standard_normal((512, 1024))).astype(np.float32)
    wq, ad = _wq(w), to_device_bf16(a)
    for act in (16, 8, 4):
        c1 = fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32)
        c2 = fp4.gemm_w4aX(act, ad, wq, out_dtype=torch.float32)
        assert torch.equal(c1, c2)
    g1 = fp4.gemm_w4aX(16, ad[:8], wq, out_dtype=torch.float32)
    g2 = fp4.gemm_w4aX(16, ad[:8], wq, out_dtype=torch.float32)
    assert torch.equal(g1, g2)
