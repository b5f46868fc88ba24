"""The C-ABI library loads, exports every function include/fp4_e2m1.h declares, and its
host-side logic (validation before any launch, policy table, workspace sizes, status
strings) behaves as documented. No compute is run here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4_e2m1.h")

lib_mod = pytest.importorskip("block_scaled_fp4_e2m1_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lib_mod.LIB_PATH):
        pytest.fail("libfp4_e2m1.so is not built (python -m block_scaled_fp4_e2m1_amd.build)")
    return lib_mod.library()


def test_header_declares_the_four_operations():
    names = _declared_functions()
    for n in ("quantize_fp4", "dequantize_fp4", "gemm_w4aX", "grouped_gemm_w4aX"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(lib_mod.EXPORTED) == names


def test_probe_library_exports_its_header_and_validates():
    """The measurement probes' library (libfp4_probes.so) exports every function
    include/fp4_probes.h declares, and refuses invalid arguments before any launch."""
    path = os.path.join(ROOT, "block_scaled_fp4_e2m1_amd", "libfp4_probes.so")
    if not os.path.exists(path):
        pytest.fail("libfp4_probes.so is not built (python -m block_scaled_fp4_e2m1_amd.build)")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "fp4_probes.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*int32_t\s+([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)))
    assert names == ["probe_lds_read", "probe_mfma", "probe_mix", "probe_read", "probe_valu"]
    plib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    for n in names:
        assert hasattr(plib, n)
    plib.probe_read.argtypes = [vp, i64, vp, i32, i32, vp]
    plib.probe_mfma.argtypes = [i32, i32, i32, i32, vp, vp]
    plib.probe_lds_read.argtypes = [i32, i32, vp, vp]
    plib.probe_valu.argtypes = [i32, i32, i32, vp, vp]
    plib.probe_mix.argtypes = [i32, i32, i32, vp, vp]
    fake, null = vp(1 << 20), vp(0)
    assert plib.probe_read(fake, 100, fake, 4, 256, null) == 2      # bytes % 16
    assert plib.probe_read(fake, 1024, fake, 4, 96, null) == 2      # threads % 64
    assert plib.probe_read(null, 1024, fake, 4, 256, null) == 2
    assert plib.probe_mfma(3, 8, 4, 4, fake, null) == 2            # unknown kind
    assert plib.probe_mfma(0, 5, 4, 4, fake, null) == 2            # chains
    assert plib.probe_lds_read(4, 0, fake, null) == 2
    assert plib.probe_valu(7, 4, 4, fake, null) == 2
    assert plib.probe_mix(12, 4, 4, fake, null) == 2


def test_status_strings(lib):
    assert lib_mod.status_string(0) == "ok"
    for s in range(1, 11):
        assert lib_mod.status_string(s) not in ("ok", "unknown status")
    assert lib_mod.status_string(99) == "unknown status"


def test_policy_select(lib):
    P = lib_mod
    assert P.fp4_policy_select(P.POLICY_Q4, True) == P.A4
    assert P.fp4_policy_select(P.POLICY_Q4, False) == P.A4
    assert P.fp4_policy_select(P.POLICY_Q8, False) == P.A8
    assert P.fp4_policy_select(P.POLICY_AUTO, True) == P.A8
    assert P.fp4_policy_select(P.POLICY_AUTO, False) == P.A4
    assert P.fp4_policy_select(P.POLICY_SENSITIVE_W8, True) == P.W8A8
    assert P.fp4_policy_select(P.POLICY_SENSITIVE_W8, False) == P.A4
    assert P.fp4_policy_select(P.POLICY_STATIC, True) == P.A8S
    assert P.fp4_policy_select(P.POLICY_STATIC, False) == P.A4S
    with pytest.raises(P.Fp4Error):
        P.fp4_policy_select(3, False)


def test_workspace_bytes(lib):
    P = lib_mod
    assert P.fp4_workspace_bytes(P.A16, 2048, 4096, 4096) == 0
    m, k = 2048, 4096
    need = P.fp4_workspace_bytes(P.A4, m, 4096, k)
    assert need >= m * k * 2 + m * (k // 256) * 4
    assert P.fp4_workspace_bytes(P.A8, m, 4096, k) == need
    assert P.fp4_workspace_bytes(7, m, 4096, k) == 0
    assert P.fp4_workspace_bytes(P.A4S, m, 4096, k) == need
    assert P.fp4_workspace_bytes(P.A8S, m, 4096, k) == need
    assert P.fp4_workspace_bytes(P.W8A8, m, 4096, k) == need


def test_validation_happens_before_any_device_use(lib):
    vp = ctypes.c_void_p
    fake = vp(1 << 20)  # never dereferenced: every call below fails validation first
    null = vp(0)
    # null input
    assert lib.quantize_fp4(null, 1, 16, 256, 256, 0, 0, fake, fake, fake, null) == 1
    # bad dtype / elem / layout / shapes / alignment
    assert lib.quantize_fp4(fake, 7, 16, 256, 256, 0, 0, fake, fake, fake, null) == 4
    assert lib.quantize_fp4(fake, 1, 16, 256, 256, 5, 0, fake, fake, fake, null) == 5
    assert lib.quantize_fp4(fake, 1, 24, 256, 256, 1, 1, fake, fake, fake, null) == 2  # E4M3 tiled, rows % 16
    assert lib.quantize_fp4(fake, 1, 16, 300, 300, 0, 0, fake, fake, fake, null) == 2
    assert lib.quantize_fp4(fake, 1, 15, 256, 256, 0, 1, fake, fake, fake, null) == 2
    assert lib.quantize_fp4(fake, 1, 16, 256, 100, 0, 0, fake, fake, fake, null) == 2
    assert lib.quantize_fp4(vp((1 << 20) + 2), 1, 16, 256, 256, 0, 0, fake, fake, fake, null) == 3
    assert lib.quantize_fp4(fake, 1, 16, 256, 260, 0, 0, fake, fake, fake, null) == 3
    T = lib_mod._Tensor
    w = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 0, 1)
    assert lib.gemm_w4aX(5, fake, 1, 8, 512, ctypes.byref(w), fake, 1, 256, null, 0, null) == 5
    wc = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 0, 0)  # canonical weights
    assert lib.gemm_w4aX(16, fake, 1, 8, 512, ctypes.byref(wc), fake, 1, 256, null, 0, null) == 10
    w8 = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 1, 1)  # E4M3 weights
    assert lib.gemm_w4aX(16, fake, 1, 8, 512, ctypes.byref(w8), fake, 1, 256, null, 0, null) == 4
    wr = T(1 << 20, 1 << 21, 1 << 22, 250, 512, 0, 1)  # rows not a multiple of 16
    assert lib.gemm_w4aX(16, fake, 1, 8, 512, ctypes.byref(wr), fake, 1, 256, null, 0, null) == 2
    # A4 needs a workspace
    assert lib.gemm_w4aX(4, fake, 1, 8, 512, ctypes.byref(w), fake, 1, 256, null, 0, null) == 9
    # grouped: expert count must divide the stacked rows; offsets are required
    assert lib.grouped_gemm_w4aX(4, fake, 1, 64, 512, null, fake, 3, 64, ctypes.byref(w), fake, 1,
                                 256, fake, 1 << 30, null) == 2
    assert lib.grouped_gemm_w4aX(4, fake, 1, 64, 512, null, null, 2, 64, ctypes.byref(w), fake, 1,
                                 256, fake, 1 << 30, null) == 1


def test_product_k_limit_is_checked_before_anything_is_enqueued(lib):
    """The product kernel's per-group tables fit LDS up to k = 21760 (85 groups). Past
    that, every product entry point returns FP4_E_SHAPE before the device is even looked
    at (on this GPU-less host a later check would return FP4_E_NO_DEVICE, and a launch
    FP4_E_HIP): no activation pass is enqueued ahead of a refused product."""
    vp = ctypes.c_void_p
    fake, null = vp(1 << 20), vp(0)
    ws, big = vp(1 << 24), 1 << 40
    T = lib_mod._Tensor
    k_bad, k_ok = 22016, 21760
    w = T(1 << 20, 1 << 21, 1 << 22, 256, k_bad, 0, 1)
    wk = T(1 << 20, 1 << 21, 1 << 22, 256, k_ok, 0, 1)
    for act in (4, 8):
        assert lib.gemm_w4aX(act, fake, 1, 64, k_bad, ctypes.byref(w), fake, 1, 256, ws, big, null) == 2
        assert lib.gemm_w4aX(act, fake, 1, 64, k_ok, ctypes.byref(wk), fake, 1, 256, ws, big, null) == 6
        assert lib.grouped_gemm_w4aX(act, fake, 1, 64, k_bad, null, fake, 2, 64, ctypes.byref(w), fake, 1,
                                     128, ws, big, null) == 2
        assert lib.grouped_gemm_w4aX_gated(act, fake, 64, 2 * k_bad, fake, 2, ctypes.byref(w), fake, 1, 128,
                                           ws, big, null) == 2
        assert lib.gemm_w4aX_static(act, fake, 1, 64, k_bad, fake, ctypes.byref(w), fake, 1, 256, ws, big,
                                    null) == 2
    # bf16 A16: m <= 8 with k <= 8192 runs the decode GEMV; larger k or m runs the product
    assert lib.gemm_w4aX(16, fake, 1, 64, k_bad, ctypes.byref(w), fake, 1, 256, null, 0, null) == 2
    assert lib.gemm_w4aX(16, fake, 1, 8, k_bad, ctypes.byref(w), fake, 1, 256, null, 0, null) == 2
    # float32 A16 runs one thread per output and has no k limit
    assert lib.gemm_w4aX(16, fake, 0, 8, k_bad, ctypes.byref(w), fake, 0, 256, null, 0, null) == 6
    # grouped: an expert row count that is not a multiple of 16
    w24 = T(1 << 20, 1 << 21, 1 << 22, 48, 512, 0, 1)
    assert lib.grouped_gemm_w4aX(4, fake, 1, 64, 512, null, fake, 2, 64, ctypes.byref(w24), fake, 1,
                                 24, ws, big, null) == 2


def test_product_ldc_bound_is_checked_before_anything_is_enqueued(lib):
    """Every product entry point takes n <= ldc <= FP4_MAX_LDC (2^21) and returns
    FP4_E_SHAPE outside it before the device is looked at; at the bound the call reaches
    the device check (FP4_E_NO_DEVICE on this GPU-less host)."""
    vp = ctypes.c_void_p
    fake, null = vp(1 << 20), vp(0)
    ws, big = vp(1 << 24), 1 << 40
    T = lib_mod._Tensor
    w = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 0, 1)
    w8 = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 1, 1)
    top = 1 << 21
    for ldc, want in ((top + 1, 2), (top, 6), (255, 2)):
        assert lib.gemm_w4aX(4, fake, 1, 64, 512, ctypes.byref(w), fake, 1, ldc, ws, big, null) == want
        assert lib.gemm_w4aX_noalloc(4, fake, 1, 64, 512, ctypes.byref(w), fake, 1, ldc, null) == want
        assert lib.gemm_w4aX_static(4, fake, 1, 64, 512, fake, ctypes.byref(w), fake, 1, ldc, ws, big,
                                    null) == want
        assert lib.gemm_w8a8(fake, 1, 64, 512, ctypes.byref(w8), fake, 1, ldc, ws, big, null) == want
    for ldc, want in ((top + 1, 2), (top, 6), (127, 2)):
        assert lib.grouped_gemm_w4aX(4, fake, 1, 64, 512, null, fake, 2, 64, ctypes.byref(w), fake, 1,
                                     ldc, ws, big, null) == want
        assert lib.grouped_gemm_w4aX_gated(4, fake, 64, 1024, fake, 2, ctypes.byref(w), fake, 1, ldc,
                                           ws, big, null) == want
    for ldc, want in ((top + 1, 2), (top, 6), (255, 2)):
        assert lib.gemm_mxfp4(fake, fake, 64, fake, fake, 256, 512, fake, 1, ldc, null) == want


def test_noalloc_validates_before_device_use(lib):
    vp = ctypes.c_void_p
    fake, null = vp(1 << 20), vp(0)
    T = lib_mod._Tensor
    w = T(1 << 20, 1 << 21, 1 << 22, 256, 4096, 0, 1)
    # 4096 x 4096 activations need 33.8 MB of workspace: more than the 32 MiB scratch
    assert lib.gemm_w4aX_noalloc(4, fake, 1, 4096, 4096, ctypes.byref(w), fake, 1, 256, null) == 9
    assert lib.gemm_w4aX_noalloc(4, fake, 1, 4064, 4096, ctypes.byref(w), fake, 1, 256, null) == 6
    assert lib.gemm_w4aX_noalloc(16, fake, 1, 4096, 4096, ctypes.byref(w), fake, 1, 256, null) == 6
    assert lib.gemm_w4aX_noalloc(5, fake, 1, 64, 4096, ctypes.byref(w), fake, 1, 256, null) == 5
    assert lib.gemm_w4aX_noalloc(4, null, 1, 64, 4096, ctypes.byref(w), fake, 1, 256, null) == 1


def test_repack_validates_before_device_use(lib):
    vp = ctypes.c_void_p
    fake, null = vp(1 << 20), vp(0)
    T = lib_mod._Tensor
    can = T(1 << 20, 1 << 21, 1 << 22, 64, 512, 0, 0)
    assert lib.repack_fp4(ctypes.byref(can), 1, null, fake, fake, null) == 1
    assert lib.repack_fp4(None, 1, fake, fake, fake, null) == 1
    assert lib.repack_fp4(ctypes.byref(can), 0, fake, fake, fake, null) == 10  # same layout
    assert lib.repack_fp4(ctypes.byref(can), 3, fake, fake, fake, null) == 5
    assert lib.repack_fp4(ctypes.byref(T(1 << 20, 1 << 21, 1 << 22, 64, 512, 2, 0)), 1, fake, fake, fake,
                          null) == 5
    assert lib.repack_fp4(ctypes.byref(T(1 << 20, 1 << 21, 1 << 22, 40, 512, 0, 0)), 1, fake, fake, fake,
                          null) == 2  # rows % 16
    assert lib.repack_fp4(ctypes.byref(T(1 << 20, 1 << 21, 1 << 22, 64, 500, 0, 0)), 1, fake, fake, fake,
                          null) == 2
    assert lib.repack_fp4(ctypes.byref(can), 1, vp((1 << 20) + 8), fake, fake, null) == 3
    assert lib.repack_fp4(ctypes.byref(T(1 << 20, (1 << 21) + 4, 1 << 22, 64, 512, 0, 0)), 1, fake, fake, fake,
                          null) == 3
    # valid: reaches the device check (no GPU here)
    assert lib.repack_fp4(ctypes.byref(can), 1, fake, fake, fake, null) == 6


def test_moe_entry_points_validate_before_device_use(lib):
    vp = ctypes.c_void_p
    fake = vp(1 << 20)
    null = vp(0)
    T = lib_mod._Tensor
    w = T(1 << 20, 1 << 21, 1 << 22, 512, 256, 0, 1)  # 2 experts x 256 rows, k = 256
    # gated product: A16 has no gated form; gate_up row stride must hold gate and up
    assert lib.grouped_gemm_w4aX_gated(16, fake, 64, 512, fake, 2, ctypes.byref(w), fake, 1, 256,
                                       fake, 1 << 30, null) == 4
    assert lib.grouped_gemm_w4aX_gated(4, fake, 64, 511, fake, 2, ctypes.byref(w), fake, 1, 256,
                                       fake, 1 << 30, null) == 2
    assert lib.grouped_gemm_w4aX_gated(4, fake, 64, 512, null, 2, ctypes.byref(w), fake, 1, 256,
                                       fake, 1 << 30, null) == 1
    assert lib.grouped_gemm_w4aX_gated(4, fake, 64, 512, fake, 3, ctypes.byref(w), fake, 1, 256,
                                       fake, 1 << 30, null) == 2
    assert lib.grouped_gemm_w4aX_gated(8, fake, 64, 512, fake, 2, ctypes.byref(w), fake, 1, 256,
                                       null, 0, null) == 9
    # routing: top_k within [1, min(16, E)], E <= 1024; workspace = E counters (256-byte
    # aligned) + five 64-bit plane words per token and 64 experts
    assert lib.moe_route_workspace_bytes(4096, 128) == 512 + 4096 * 2 * 8 * 5
    assert lib.moe_route_workspace_bytes(10, 65) == 512 + 10 * 2 * 8 * 5
    assert lib.moe_route_workspace_bytes(10, 0) == 0
    ws, big = vp(1 << 24), 1 << 20
    assert lib.moe_route(null, 8, 4, 2, fake, fake, fake, fake, fake, ws, big, null) == 1
    assert lib.moe_route(fake, 8, 4, 5, fake, fake, fake, fake, fake, ws, big, null) == 2
    assert lib.moe_route(fake, 8, 64, 17, fake, fake, fake, fake, fake, ws, big, null) == 2
    assert lib.moe_route(fake, 8, 1025, 2, fake, fake, fake, fake, fake, ws, big, null) == 2
    assert lib.moe_route(fake, 0, 4, 2, fake, fake, fake, fake, fake, ws, big, null) == 2
    assert lib.moe_route(fake, 1 << 28, 128, 8, fake, fake, fake, fake, fake, ws, big, null) == 2
    assert lib.moe_route(fake, 8, 128, 8, fake, fake, fake, fake, fake, ws, 512 + 8 * 80 - 1, null) == 9
    assert lib.moe_route(fake, 8, 128, 8, fake, fake, fake, fake, fake, vp((1 << 24) + 16), big, null) == 9
    assert lib.moe_route(vp((1 << 20) + 2), 8, 4, 2, fake, fake, fake, fake, fake, ws, big, null) == 3
    # combine: hidden a multiple of 8, 16-byte rows, known dtypes
    assert lib.moe_combine(fake, 1, 512, fake, fake, 8, 2, 500, fake, 0, 512, null) == 2
    assert lib.moe_combine(fake, 1, 516, fake, fake, 8, 2, 512, fake, 0, 512, null) == 3  # 1032-byte rows
    assert lib.moe_combine(fake, 7, 512, fake, fake, 8, 2, 512, fake, 0, 512, null) == 4
    assert lib.moe_combine(fake, 1, 512, null, fake, 8, 2, 512, fake, 0, 512, null) == 1
    assert lib.moe_combine(fake, 1, 512, fake, fake, 8, 0, 512, fake, 0, 512, null) == 2


def test_kv_entry_points_validate_before_device_use(lib):
    vp = ctypes.c_void_p
    fake, null = vp(1 << 20), vp(0)
    KV = lib_mod._KvCache
    # sizes: codes n_seq * kv_heads * T * 64, micro * 8, macro n_seq * kv_heads/2 * T * 2
    assert lib.fp4_kv_cache_bytes(32, 16384, 8, 128, 0) == 32 * 8 * 16384 * 64
    assert lib.fp4_kv_cache_bytes(32, 16384, 8, 128, 1) == 32 * 8 * 16384 * 8
    assert lib.fp4_kv_cache_bytes(32, 16384, 8, 128, 2) == 32 * 4 * 16384 * 2
    assert lib.fp4_kv_cache_bytes(1, 96, 2, 128, 0) == 96 * 2 * 64
    for bad in ((1, 40, 2, 128), (1, 64, 3, 128), (1, 64, 2, 64), (1, 64, 34, 128), (0, 64, 2, 128),
                (1, 16, 2, 128)):
        assert lib.fp4_kv_cache_bytes(*bad, 0) == 0
    # 2048-token chunks: 8 per sequence at 16384 tokens; O[128], m, l per (sequence, head, chunk)
    assert lib.attention_workspace_bytes(32, 32, 16384) == 32 * 32 * 8 * 130 * 4
    good = KV(1 << 20, 1 << 21, 1 << 22, 1 << 23, 1 << 24, 1 << 25, 4, 64, 2, 128)
    assert lib.kv_cache_append(None, fake, fake, 1, 256, fake, 1, null) == 1
    assert lib.kv_cache_append(ctypes.byref(good), fake, fake, 1, 255, fake, 1, null) == 2
    assert lib.kv_cache_append(ctypes.byref(good), fake, fake, 1, 256, fake, 0, null) == 2
    assert lib.kv_cache_append(ctypes.byref(good), fake, fake, 7, 256, fake, 1, null) == 4
    assert lib.kv_cache_append(ctypes.byref(good), vp((1 << 20) + 8), fake, 1, 256, fake, 1, null) == 3
    assert lib.kv_cache_append(ctypes.byref(good), fake, null, 1, 256, fake, 1, null) == 1
    odd = KV(1 << 20, 1 << 21, 1 << 22, 1 << 23, 1 << 24, 1 << 25, 4, 64, 3, 128)
    assert lib.kv_cache_append(ctypes.byref(odd), fake, fake, 1, 384, fake, 1, null) == 2
    mis = KV((1 << 20) + 4, 1 << 21, 1 << 22, 1 << 23, 1 << 24, 1 << 25, 4, 64, 2, 128)
    assert lib.kv_cache_append(ctypes.byref(mis), fake, fake, 1, 256, fake, 1, null) == 3
    ws = vp(1 << 26)
    assert lib.attention_decode_fp4kv(fake, 3, ctypes.byref(good), fake, 1.0, fake, 0, ws, 1 << 30, null) == 2
    assert lib.attention_decode_fp4kv(fake, 34, ctypes.byref(good), fake, 1.0, fake, 0, ws, 1 << 30, null) == 2
    assert lib.attention_decode_fp4kv(fake, 8, ctypes.byref(good), fake, 1.0, fake, 0, null, 0, null) == 9
    assert lib.attention_decode_fp4kv(fake, 8, ctypes.byref(good), fake, 1.0, fake, 0, ws, 100, null) == 9
    assert lib.attention_decode_fp4kv(null, 8, ctypes.byref(good), fake, 1.0, fake, 0, ws, 1 << 30, null) == 1
    assert lib.attention_decode_fp4kv(fake, 8, ctypes.byref(good), fake, 1.0, fake, 5, ws, 1 << 30, null) == 4


def test_mx_entry_points_validate_before_device_use(lib):
    vp = ctypes.c_void_p
    fake, null = vp(1 << 20), vp(0)
    # sizes: rows padded to 16; codes rows * k / 2, scales rows * k / 32
    assert lib.mxfp4_bytes(37, 384, 0) == 48 * 384 // 2
    assert lib.mxfp4_bytes(37, 384, 1) == 48 * 384 // 32
    assert lib.mxfp4_bytes(16, 96, 0) == 0 and lib.mxfp4_bytes(0, 128, 0) == 0
    assert lib.quantize_mxfp4(null, 1, 16, 128, 128, fake, fake, null) == 1
    assert lib.quantize_mxfp4(fake, 7, 16, 128, 128, fake, fake, null) == 4
    assert lib.quantize_mxfp4(fake, 1, 16, 96, 96, fake, fake, null) == 2
    assert lib.quantize_mxfp4(fake, 1, 16, 128, 100, fake, fake, null) == 2
    assert lib.quantize_mxfp4(fake, 1, 16, 128, 132, fake, fake, null) == 3
    assert lib.gemm_mxfp4(fake, fake, 16, fake, fake, 16, 192, fake, 1, 16, null) == 2
    assert lib.gemm_mxfp4(fake, fake, 16, fake, fake, 16, 128, fake, 1, 8, null) == 2
    assert lib.gemm_mxfp4(fake, null, 16, fake, fake, 16, 128, fake, 1, 16, null) == 1
    assert lib.gemm_mxfp4(vp((1 << 20) + 4), fake, 16, fake, fake, 16, 128, fake, 1, 16, null) == 3


def test_sensitive_and_static_entry_points_validate_before_device_use(lib):
    vp = ctypes.c_void_p
    fake, null = vp(1 << 20), vp(0)
    ws, big = vp(1 << 24), 1 << 30
    T = lib_mod._Tensor
    w4 = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 0, 1)
    w8 = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 1, 1)
    w8c = T(1 << 20, 1 << 21, 1 << 22, 256, 512, 1, 0)  # canonical E4M3
    w8k = T(1 << 20, 1 << 21, 1 << 22, 256, 32768, 1, 1)  # k past the kernel's tables
    # static quantization: the macro-scales are required and 2-byte aligned
    assert lib.quantize_fp4_static(fake, 1, 16, 256, 256, 0, 0, null, fake, fake, fake, null) == 1
    assert lib.quantize_fp4_static(fake, 1, 16, 256, 256, 0, 0, vp((1 << 20) + 1), fake, fake, fake, null) == 3
    assert lib.quantize_fp4_static(fake, 1, 16, 300, 300, 0, 0, fake, fake, fake, fake, null) == 2
    # calibration
    assert lib.act_macro_calibrate(fake, 1, 64, 512, 512, 0, null, fake, null) == 1
    assert lib.act_macro_calibrate(fake, 7, 64, 512, 512, 0, fake, fake, null) == 4
    assert lib.act_macro_calibrate(fake, 1, 64, 512, 512, 3, fake, fake, null) == 5
    assert lib.act_macro_calibrate(fake, 1, 64, 500, 512, 0, fake, fake, null) == 2
    assert lib.act_macro_calibrate(fake, 1, 0, 512, 512, 0, fake, fake, null) == 2
    assert lib.act_macro_calibrate(fake, 1, 64, 512, 512, 0, vp((1 << 20) + 2), fake, null) == 3
    # static product: A4 / A8 only, macro-scales required, E2M1 tiled weights, workspace
    assert lib.gemm_w4aX_static(16, fake, 1, 8, 512, fake, ctypes.byref(w4), fake, 1, 256, ws, big, null) == 5
    assert lib.gemm_w4aX_static(4, fake, 1, 8, 512, null, ctypes.byref(w4), fake, 1, 256, ws, big, null) == 1
    assert lib.gemm_w4aX_static(4, fake, 1, 8, 512, fake, ctypes.byref(w8), fake, 1, 256, ws, big, null) == 4
    assert lib.gemm_w4aX_static(8, fake, 1, 8, 512, fake, ctypes.byref(w4), fake, 1, 256, null, 0, null) == 9
    # W8A8: E4M3 tiled weights only; k limit; workspace
    assert lib.gemm_w8a8(fake, 1, 8, 512, ctypes.byref(w4), fake, 1, 256, ws, big, null) == 4
    assert lib.gemm_w8a8(fake, 1, 8, 512, ctypes.byref(w8c), fake, 1, 256, ws, big, null) == 10
    assert lib.gemm_w8a8(fake, 1, 8, 32768, ctypes.byref(w8k), fake, 1, 256, ws, big, null) == 2
    assert lib.gemm_w8a8(fake, 1, 8, 512, ctypes.byref(w8), fake, 1, 256, null, 0, null) == 9
    assert lib.gemm_w8a8(fake, 1, 8, 512, ctypes.byref(w8), fake, 1, 200, ws, big, null) == 2
    assert lib.gemm_w8a8(null, 1, 8, 512, ctypes.byref(w8), fake, 1, 256, ws, big, null) == 1


def test_device_check_reports_missing_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.fp4_device_check() == 6
