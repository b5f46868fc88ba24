"""gemm_w4aX_noalloc (the entry point for callers that cannot allocate: its activation
operand lives in the library's per-GPU scratch array) through the C ABI, against
gemm_w4aX with a caller workspace: the same kernels, so the outputs must be identical
bit for bit. Two calls in a row, the second smaller than the first (the scratch keeps
the first call's contents; nothing may leak into the second), for W4A4, W4A8 and W4A16;
an oversized call is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _operands(rng, m, n, k):
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, rng.choice(k, 3, replace=False)] *= 50
    a = torch.from_numpy(workloads.to_bf16_values(a)).cuda().to(torch.bfloat16)
    w = torch.from_numpy((0.02 * rng.standard_normal((n, k))).astype(np.float32)).cuda()
    return a, fp4.quantize_fp4(w, layout=fp4.LAYOUT_TILED)


def _noalloc(act, a, wq, out):
    """Direct C-ABI call (no binding logic in between)."""
    lib = fp4.library()
    ts = wq.c_struct()
    return lib.gemm_w4aX_noalloc(act, ctypes.c_void_p(a.data_ptr()), fp4.BF16, a.shape[0], a.stride(0),
                                 ctypes.byref(ts), ctypes.c_void_p(out.data_ptr()),
                                 fp4.F32 if out.dtype == torch.float32 else fp4.BF16, out.stride(0),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("act", [4, 8, 16])
def test_noalloc_matches_workspace_entry_point_twice(act):
    rng = np.random.default_rng(950 + act)
    # first call: 1983 x 4096 activations (16.3 MB of the 32 MiB scratch), ragged rows;
    # second: smaller, other k, so stale first-call data sits beyond what it writes
    for m, n, k, odt in ((1983, 1040, 4096, torch.float32), (130, 272, 1280, torch.bfloat16)):
        print(f"[case] noalloc act={act} m={m} n={n} k={k} {odt}", flush=True)
        a, wq = _operands(rng, m, n, k)
        want = fp4.gemm_w4aX(act, a, wq, out_dtype=odt)
        got = torch.full((m, n), float("nan"), dtype=odt, device="cuda")
        assert _noalloc(act, a, wq, got) == 0
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"act={act} m={m}: differs from gemm_w4aX"


def test_noalloc_packed_activations_twice():
    """A W4A4 shape on the large-product form (packed E2M1 activations in the scratch,
    decoded by the product kernel), then a smaller one on the same form: identical to
    gemm_w4aX with a workspace both times."""
    rng = np.random.default_rng(970)
    for m, n, k in ((2043, 4080, 1024), (1950, 4096, 512)):
        name = fp4.fp4_product_kernel(fp4.A4, torch.bfloat16, m, n, k)
        assert "decoded in the kernel" in name, name
        print(f"[case] noalloc packed A4 m={m} n={n} k={k} ({name})", flush=True)
        a, wq = _operands(rng, m, n, k)
        want = fp4.gemm_w4aX(fp4.A4, a, wq, out_dtype=torch.bfloat16)
        got = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert _noalloc(fp4.A4, a, wq, got) == 0
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"m={m}: differs from gemm_w4aX"


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    rng = np.random.default_rng(960)
    m, n, k = 4096, 256, 4096  # 4096 x 4096 activations: 33.8 MB > 32 MiB
    assert fp4.fp4_workspace_bytes(fp4.A4, m, n, k) > fp4.NOALLOC_SCRATCH_BYTES
    a, wq = _operands(rng, m, n, k)
    out = torch.zeros(m, n, dtype=torch.float32, device="cuda")
    print("[case] noalloc oversized", flush=True)
    assert _noalloc(fp4.A4, a, wq, out) == 9  # FP4_E_WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()  # nothing was enqueued
    # the same shape in W4A16 needs no scratch
    assert _noalloc(fp4.A16, a, wq, out) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, fp4.gemm_w4aX(fp4.A16, a, wq, out_dtype=torch.float32))
