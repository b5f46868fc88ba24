"""GPU parity of the mixture-of-experts steps around the grouped product (moe_route,
grouped_gemm_w4aX_gated, moe_combine) against the CPU oracle, through the C ABI.

Gates:
  routing: expert ids, offsets, row_token and token_rows bit-exact (integer work);
           weights within 2e-6 relative (float32 softmax of at most 16 terms vs float64).
  gated down product: the bf16 output gate of the products (||C - RNE_bf16(C64)||_F /
           ||RNE_bf16(C64)||_F <= 1e-3 and >= 99.9% of elements within one bf16 step).
           The oracle evaluates silu in float32 with correctly rounded operations; the
           kernel uses the hardware exp and reciprocal approximations (a few float32 ulp).
           That moves h = bf16(silu(g) * u) by one bf16 step in rare elements (a few ulp
           out of the 2^16 ulp of a bf16 step), so the float32 gate is not applied here.
  combine: float32 output within 1e-5 relative Frobenius (float32 sums of <= 8 terms).
  whole layer (route, gate/up, gated down, combine on a small configuration): relative
           Frobenius <= 1e-3 against the float64 oracle pipeline. Intermediate bf16
           outputs computed in float32 (GPU) and float64 (oracle) can differ by one bf16
           step; where that moves an element of h across an E2M1 rounding threshold, its
           quantized value changes by one code step (a relative change of up to 1/3 of
           that element's contribution). The bound leaves room for a few such elements per
           output row; the measured error is about 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._util import host, to_device_bf16, bf16_values, bf16_gate, f32_gate

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _route_both(logits, top_k):
    got = [host(t) for t in fp4.moe_route(torch.from_numpy(logits).cuda(), top_k)]
    ref = oracle.route(logits, top_k)
    return got, ref


def _check_route(logits, top_k):
    (ids, w, off, rt, tr), (rids, rw, roff, rrt, rtr) = _route_both(logits, top_k)
    assert np.array_equal(ids, rids)
    assert np.array_equal(off, roff)
    assert np.array_equal(rt, rrt)
    assert np.array_equal(tr, rtr)
    assert np.all(np.abs(w - rw) <= 2e-6 * rw)  # a zero weight (a -inf logit) must be exact


def test_route_moe_workload():
    logits = workloads.moe_router_logits()
    print("[case] moe_route 4096 tokens x 128 experts top-8", flush=True)
    _check_route(logits, 8)


@pytest.mark.parametrize("t_count,e_count,top_k", [(1, 5, 1), (37, 5, 5), (200, 64, 3), (300, 65, 16),
                                                    (50, 1000, 16), (129, 128, 1)])
def test_route_shapes(t_count, e_count, top_k):
    rng = np.random.default_rng(t_count * 7 + e_count + top_k)
    logits = rng.standard_normal((t_count, e_count)).astype(np.float32)
    print(f"[case] moe_route T={t_count} E={e_count} k={top_k}", flush=True)
    _check_route(logits, top_k)


def test_route_ties_go_to_lower_ids():
    rng = np.random.default_rng(21)
    logits = np.round(rng.standard_normal((96, 70)) * 2).astype(np.float32) / 2  # many ties
    logits[0, :] = 1.0  # all equal: experts 0 .. k-1
    print("[case] moe_route with ties", flush=True)
    _check_route(logits, 6)
    ids = host(fp4.moe_route(torch.from_numpy(logits).cuda(), 6)[0])
    assert list(ids[0]) == [0, 1, 2, 3, 4, 5]


def test_route_masked_experts():
    """-inf logits (experts masked out) rank last; a token with fewer finite logits than
    top_k picks masked experts by id with weight exactly 0."""
    rng = np.random.default_rng(22)
    logits = rng.standard_normal((64, 40)).astype(np.float32)
    logits[rng.random(logits.shape) < 0.5] = -np.inf
    logits[3, 2:] = -np.inf  # two finite logits only
    print("[case] moe_route with -inf logits", flush=True)
    _check_route(logits, 4)


def test_route_nan_logits_still_give_a_permutation():
    """NaN ranks with -inf: the routing stays a valid permutation of the routed rows, and
    tokens without NaN route exactly as the oracle does."""
    rng = np.random.default_rng(23)
    t_count, e_count, top_k = 50, 12, 3
    logits = rng.standard_normal((t_count, e_count)).astype(np.float32)
    bad = [4, 17]
    logits[4, 5] = np.nan
    logits[17, :] = np.nan
    print("[case] moe_route with NaN logits", flush=True)
    ids, w, off, rt, tr = [host(t) for t in fp4.moe_route(torch.from_numpy(logits).cuda(), top_k)]
    for t in range(t_count):
        assert len(set(ids[t].tolist())) == top_k and ids[t].min() >= 0 and ids[t].max() < e_count
    assert off[0] == 0 and off[-1] == t_count * top_k and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(tr.ravel()), np.arange(t_count * top_k))
    for t in range(t_count):
        for j in range(top_k):
            assert rt[tr[t, j]] == t and off[ids[t, j]] <= tr[t, j] < off[ids[t, j] + 1]
    assert list(ids[17]) == [0, 1, 2]  # all NaN: lowest ids
    assert 5 not in ids[4]  # the NaN logit ranks below the finite ones
    good = [t for t in range(t_count) if t not in bad]
    rids, rw, *_ = oracle.route(logits[good], top_k)
    assert np.array_equal(ids[good], rids)
    assert np.all(np.abs(w[good] - rw) <= 2e-6 * rw)


def _routed(t_count, e_count, top_k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((t_count, e_count)).astype(np.float32)
    return oracle.route(logits, top_k)


@pytest.mark.parametrize("act", [4, 8])
def test_gated_down_product(act):
    t_count, e_count, top_k, inter, hidden = 300, 6, 2, 512, 768
    ids, w_tok, offsets, row_token, token_rows = _routed(t_count, e_count, top_k, 31)
    rows = int(offsets[-1])
    rng = np.random.default_rng(32)
    y1 = workloads.to_bf16_values((2.0 * rng.standard_normal((rows, 2 * inter))).astype(np.float32))
    w2 = (0.02 * rng.standard_normal((e_count * hidden, inter))).astype(np.float32)
    print(f"[case] gated down product A{act} rows={rows} inter={inter} hidden={hidden}", flush=True)
    w2q = fp4.quantize_fp4(torch.from_numpy(w2).cuda(), layout=fp4.LAYOUT_TILED)
    got = bf16_values(fp4.grouped_gemm_w4aX_gated(act, to_device_bf16(y1), torch.from_numpy(offsets).cuda(),
                                                  e_count, w2q))
    h = oracle.silu_gate(y1, inter, precision=np.float32)
    ref = oracle.grouped_gemm(h, None, offsets, oracle.quantize(w2.astype(np.float64)), e_count, act)
    full = np.concatenate([ref[e] for e in range(e_count)], axis=0)
    bf16_gate(got, oracle.formats.bf16_round(full))


def test_combine():
    t_count, e_count, top_k, hidden = 257, 9, 4, 1032
    ids, w_tok, offsets, row_token, token_rows = _routed(t_count, e_count, top_k, 41)
    rows = int(offsets[-1])
    rng = np.random.default_rng(42)
    y2 = workloads.to_bf16_values(rng.standard_normal((rows, hidden)).astype(np.float32))
    print(f"[case] moe_combine T={t_count} k={top_k} hidden={hidden}", flush=True)
    w32 = w_tok.astype(np.float32)
    ref = oracle.combine(y2, token_rows, w32.astype(np.float64))
    got = fp4.moe_combine(to_device_bf16(y2), torch.from_numpy(token_rows).cuda(),
                          torch.from_numpy(w32).cuda(), out_dtype=torch.float32)
    f32_gate(host(got), ref)
    got16 = fp4.moe_combine(to_device_bf16(y2), torch.from_numpy(token_rows).cuda(),
                            torch.from_numpy(w32).cuda())
    bf16_gate(bf16_values(got16), oracle.formats.bf16_round(ref))


def test_moe_layer_end_to_end():
    t_count, e_count, top_k, hidden, inter = 256, 8, 2, 512, 256
    rng = np.random.default_rng(51)
    logits = rng.standard_normal((t_count, e_count)).astype(np.float32)
    x = rng.standard_normal((t_count, hidden)).astype(np.float32)
    x[:, rng.choice(hidden, 3, replace=False)] *= 50
    x = workloads.to_bf16_values(x)
    w1 = (0.02 * rng.standard_normal((e_count * 2 * inter, hidden))).astype(np.float32)
    w2 = (0.02 * rng.standard_normal((e_count * hidden, inter))).astype(np.float32)
    print("[case] moe layer end to end", flush=True)
    # GPU: every step through the C ABI
    ids, wts, off, rt, tr = fp4.moe_route(torch.from_numpy(logits).cuda(), top_k)
    w1q = fp4.quantize_fp4(torch.from_numpy(w1).cuda(), layout=fp4.LAYOUT_TILED)
    w2q = fp4.quantize_fp4(torch.from_numpy(w2).cuda(), layout=fp4.LAYOUT_TILED)
    rows = t_count * top_k
    y1 = fp4.grouped_gemm_w4aX(fp4.A4, to_device_bf16(x), rt, off, e_count, rows, w1q)
    y2 = fp4.grouped_gemm_w4aX_gated(fp4.A4, y1, off, e_count, w2q)
    out = host(fp4.moe_combine(y2, tr, wts, out_dtype=torch.float32))
    # oracle pipeline from the same inputs
    _, rw, roff, rrt, rtr = oracle.route(logits, top_k)
    r1 = oracle.grouped_gemm(x, rrt, roff, oracle.quantize(w1.astype(np.float64)), e_count, oracle.A4)
    y1r = oracle.formats.bf16_round(np.concatenate([r1[e] for e in range(e_count)], axis=0))
    h = oracle.silu_gate(y1r, inter)
    r2 = oracle.grouped_gemm(h, None, roff, oracle.quantize(w2.astype(np.float64)), e_count, oracle.A4)
    y2r = oracle.formats.bf16_round(np.concatenate([r2[e] for e in range(e_count)], axis=0))
    ref = oracle.combine(y2r, rtr, rw)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    print(f"  relative Frobenius error {rel:.3e}", flush=True)
    assert rel <= 1e-3


def test_gated_rejects_a16_and_bad_shapes():
    w2q = fp4.quantize_fp4(torch.zeros(32, 256, device="cuda"), layout=fp4.LAYOUT_TILED)
    y1 = torch.zeros(16, 512, dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 16], dtype=torch.int32, device="cuda")
    with pytest.raises(fp4.Fp4Error):
        fp4.grouped_gemm_w4aX_gated(fp4.A16, y1, off, 1, w2q)
    with pytest.raises(fp4.Fp4Error):  # gate_up rows narrower than 2k
        fp4.grouped_gemm_w4aX_gated(fp4.A4, torch.zeros(16, 256, dtype=torch.bfloat16, device="cuda"),
                                    off, 1, w2q)
    with pytest.raises(fp4.Fp4Error):  # top_k > experts
        fp4.moe_route(torch.zeros(4, 3, device="cuda"), 4)
