"""GPU parity of the FP4 KV cache (kv_cache_append) and of decode attention over it
(attention_decode_fp4kv) against the CPU oracle, through the C ABI.

Gates:
  cache contents: codes, micro- and macro-scales bit-exact against the oracle's codec on
      the same token rows (read back through the documented device layout);
  attention, float32 output: ||out - ref||_F <= 2e-6 * ||ref_abs||_F and
      ||out - ref||_F <= 5e-5 * ||ref||_F, where ref is the float64 oracle on the
      oracle's own quantization of the same inputs and ref_abs the same attention applied
      to |V|. An output is a weighted sum; its rounding error scales with the weighted sum
      of magnitudes (the sum's condition), not with the output itself, which for
      near-uniform attention over 10^4 tokens is a mean of signed values ~100x smaller
      than its terms. The first bound comes from the kernel's error model. Scores are
      exact products of cache values and q summed in float32 by 4 MFMAs of 32 terms
      (relative 2^-24 * sqrt(4/3) of |score| <= ~5 in base 2: ~3.5e-7 on a weight);
      exp2 is the hardware approximation (about 1 ulp, 2^-23); the weights enter the
      value product as an FP16 pair hi + lo (2^-22); the value and normalizer sums
      each take a chain of about 60 float32 roundings per output (16 tiles of 32 tokens
      per wave, each two MFMAs and the online rescale, then the 4-wave and the 8-chunk
      combines). With independent roundings, uniform within half an ulp, the error
      against ||ref_abs|| is about sqrt((2^-24)^2 * 2 * 60 / 3 + (2^-22)^2 / 3 +
      (2^-23)^2 / 3 + (3.5e-7)^2) ~ 5.4e-7; the gate is 3.7x that (the largest
      measured is 2.5e-7). The second bound caps the plain relative error so that a
      large condition number cannot hide a real error: ||ref_abs|| / ||ref|| reaches
      ~60 for near-uniform attention over 16384 tokens, where the cap (25x the first
      bound) is the tighter of the two; the largest plain error measured there is 1.4e-5.
      (A single FP16 weight, 2^-12 relative each, measured ~1e-4 and flipped the bf16
      rounding of too many outputs.);
  attention, bf16 output: the bf16 gate (relative Frobenius <= 1e-3 against the rounded
      float64 result, >= 99.9% of elements within one bf16 step).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._util import host, bf16_values, bf16_gate, kv_cache_to_canonical

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_e2m1_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert fp4.fp4_device_check() == 0, "device is not gfx950"


def _rows(rng, n, width, outliers=True):
    x = rng.standard_normal((n, width)).astype(np.float32)
    if outliers:
        x[:, rng.choice(width, max(1, width // 200), replace=False)] *= 20
    return x


def _check_cache(cache, which, b, tokens, rows):
    codes4, micro, macro = kv_cache_to_canonical(cache, which, b, tokens)
    ref = oracle.kv_quantize_rows(rows.astype(np.float64))
    assert np.array_equal(codes4, oracle.unpack_e2m1(ref.codes)), f"{which} codes, sequence {b}"
    assert np.array_equal(micro, ref.micro), f"{which} micro, sequence {b}"
    assert np.array_equal(macro, ref.macro.astype(np.uint16)), f"{which} macro, sequence {b}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_prefill_then_decode_bit_exact(dtype):
    n_seq, kv_heads, T = 3, 4, 160
    width = kv_heads * 128
    rng = np.random.default_rng(71)
    cache = fp4.KvCache(n_seq, T, kv_heads)
    pos0 = np.array([0, 5, 33], dtype=np.int32)
    n_new = 70
    print(f"[case] kv append prefill n_new={n_new} positions={pos0.tolist()} {dtype}", flush=True)
    k = _rows(rng, n_seq * n_new, width)
    v = _rows(rng, n_seq * n_new, width, outliers=False)
    if dtype == torch.bfloat16:
        k, v = workloads.to_bf16_values(k), workloads.to_bf16_values(v)
    fp4.kv_cache_append(cache, torch.from_numpy(k).cuda().to(dtype), torch.from_numpy(v).cuda().to(dtype),
                        torch.from_numpy(pos0).cuda())
    # one decode token per sequence right after the prompt (shares a tile with it)
    k1 = _rows(rng, n_seq, width)
    v1 = _rows(rng, n_seq, width, outliers=False)
    if dtype == torch.bfloat16:
        k1, v1 = workloads.to_bf16_values(k1), workloads.to_bf16_values(v1)
    pos1 = pos0 + n_new
    fp4.kv_cache_append(cache, torch.from_numpy(k1).cuda().to(dtype), torch.from_numpy(v1).cuda().to(dtype),
                        torch.from_numpy(pos1).cuda())
    torch.cuda.synchronize()
    for b in range(n_seq):
        toks = np.arange(pos0[b], pos1[b] + 1)
        krows = np.concatenate([k[b * n_new:(b + 1) * n_new], k1[b:b + 1]])
        vrows = np.concatenate([v[b * n_new:(b + 1) * n_new], v1[b:b + 1]])
        _check_cache(cache, "k", b, toks, krows)
        _check_cache(cache, "v", b, toks, vrows)
        # tokens never written keep the zeroed cache (shared V tiles included)
        untouched = np.setdiff1d(np.arange(T), toks)
        codes4, micro, macro = kv_cache_to_canonical(cache, "v", b, untouched)
        assert not codes4.any() and not micro.any() and not macro.any()


def test_append_skips_positions_past_the_cache_and_negative():
    n_seq, kv_heads, T = 2, 2, 64
    rng = np.random.default_rng(72)
    cache = fp4.KvCache(n_seq, T, kv_heads)
    k = workloads.to_bf16_values(_rows(rng, n_seq * 8, 256))
    v = workloads.to_bf16_values(_rows(rng, n_seq * 8, 256))
    pos = torch.tensor([T - 3, -1], dtype=torch.int32, device="cuda")
    print("[case] kv append past the end / negative position", flush=True)
    fp4.kv_cache_append(cache, torch.from_numpy(k).cuda().to(torch.bfloat16),
                        torch.from_numpy(v).cuda().to(torch.bfloat16), pos)
    torch.cuda.synchronize()
    _check_cache(cache, "k", 0, np.arange(T - 3, T), k[:3])
    _check_cache(cache, "v", 0, np.arange(T - 3, T), v[:3])
    codes4, micro, macro = kv_cache_to_canonical(cache, "k", 1, np.arange(T))
    assert not codes4.any() and not micro.any() and not macro.any()


def attention_gate(got, ref, ref_abs, tol=2e-6, tol_plain=5e-5):
    """||got - ref||_F / ||ref_abs||_F <= tol and ||got - ref||_F / ||ref||_F <= tol_plain;
    returns (the first ratio, the plain relative error)."""
    err = np.linalg.norm(np.asarray(got, np.float64) - ref)
    cond = err / max(np.linalg.norm(ref_abs), 1e-300)
    plain = err / max(np.linalg.norm(ref), 1e-300)
    assert cond <= tol, f"error {cond:.3e} of the weighted magnitudes > {tol} (plain relative {plain:.3e})"
    assert plain <= tol_plain, f"plain relative error {plain:.3e} > {tol_plain} (weighted {cond:.3e})"
    return cond, plain


def _attention_case(n_seq, kv_heads, q_heads, T, lengths, seed, out_dtype):
    rng = np.random.default_rng(seed)
    width = kv_heads * 128
    cache = fp4.KvCache(n_seq, T, kv_heads)
    k = workloads.to_bf16_values(_rows(rng, n_seq * T, width))
    v = workloads.to_bf16_values(_rows(rng, n_seq * T, width, outliers=False))
    q = workloads.to_bf16_values(rng.standard_normal((n_seq, q_heads, 128)).astype(np.float32))
    fp4.kv_cache_append(cache, torch.from_numpy(k).cuda().to(torch.bfloat16),
                        torch.from_numpy(v).cuda().to(torch.bfloat16),
                        torch.zeros(n_seq, dtype=torch.int32, device="cuda"))
    lens = np.asarray(lengths, dtype=np.int32)
    got = fp4.attention_decode_fp4kv(torch.from_numpy(q).cuda().to(torch.bfloat16), cache,
                                     torch.from_numpy(lens).cuda(), out_dtype=out_dtype)
    k_hat = oracle.kv_dequantize_rows(k).reshape(n_seq, T, kv_heads, 128)
    v_hat = oracle.kv_dequantize_rows(v).reshape(n_seq, T, kv_heads, 128)
    eff = np.clip(lens, 0, T)
    ref = np.zeros((n_seq, q_heads, 128))
    ref_abs = np.zeros((n_seq, q_heads, 128))
    live = eff > 0
    if live.any():
        sc = 1.0 / np.sqrt(128)
        ref[live] = oracle.attention_decode(q[live], k_hat[live], v_hat[live], eff[live], sc)
        ref_abs[live] = oracle.attention_decode(q[live], k_hat[live], np.abs(v_hat[live]), eff[live], sc)
    return got, ref, ref_abs


@pytest.mark.parametrize("kv_heads,q_heads", [(2, 8), (2, 2), (2, 32), (8, 64)])
def test_attention_small_f32(kv_heads, q_heads):
    T = 2112  # not a multiple of the 256-token wave span
    lengths = [1, 31, 1057, 2112]
    print(f"[case] attention kv_heads={kv_heads} q_heads={q_heads} T={T} lengths={lengths}", flush=True)
    got, ref, ref_abs = _attention_case(4, kv_heads, q_heads, T, lengths, 73 + q_heads, torch.float32)
    cond, plain = attention_gate(host(got), ref, ref_abs)
    print(f"  error {cond:.2e} of the weighted magnitudes, plain relative {plain:.2e}", flush=True)


def test_attention_bf16_out_and_edge_lengths():
    T = 1088
    lengths = [0, 32, 33, 1024, 1025, 5000]  # 0: zeros; past the cache: clamped to T
    print(f"[case] attention bf16 out lengths={lengths}", flush=True)
    got, ref, _ = _attention_case(6, 2, 8, T, lengths, 79, torch.bfloat16)
    g = bf16_values(got)
    assert not g[0].any()
    bf16_gate(g[1:], oracle.formats.bf16_round(ref[1:]))


def _tile_slot(t: int) -> int:
    """Slot of token t (0..31) in its 32-token V tile (include/fp4_e2m1.h): slots 8g + i
    hold tokens 4g + i for i < 4 and 16 + 4g + i - 4 for i >= 4."""
    return 8 * (t // 4) + t % 4 if t < 16 else 8 * ((t - 16) // 4) + 4 + (t - 16) % 4


def test_attention_ragged_tails_ignore_garbage_past_length():
    """Lengths whose last 32-token tile holds 2-31 tokens (both halves of the slot order,
    16 and 17 included), with the cache past every length poisoned: E4M3 NaN (0x7F) K and
    V micro-scales for the rest of the last tile, FP16 NaN K and V macro-scales for every
    token past the length. The output must match the oracle over the live tokens only."""
    T, kv_heads, q_heads = 1024, 2, 8
    lengths = [2, 5, 15, 16, 17, 20, 27, 30, 100, 529, 1000, 1023]
    n_seq = len(lengths)
    print(f"[case] attention ragged tails with NaN past the length: {lengths}", flush=True)
    rng = np.random.default_rng(97)
    width = kv_heads * 128
    cache = fp4.KvCache(n_seq, T, kv_heads)
    k = workloads.to_bf16_values(_rows(rng, n_seq * T, width))
    v = workloads.to_bf16_values(_rows(rng, n_seq * T, width, outliers=False))
    q = workloads.to_bf16_values(rng.standard_normal((n_seq, q_heads, 128)).astype(np.float32))
    fp4.kv_cache_append(cache, torch.from_numpy(k).cuda().to(torch.bfloat16),
                        torch.from_numpy(v).cuda().to(torch.bfloat16),
                        torch.zeros(n_seq, dtype=torch.int32, device="cuda"))
    km = host(cache.k_micro).reshape(n_seq, kv_heads, T, 8)
    vm = host(cache.v_micro).reshape(n_seq, kv_heads, T // 32, 8, 32)
    kM = host(cache.k_macro).reshape(n_seq, kv_heads // 2, T)
    vM = host(cache.v_macro).reshape(n_seq, kv_heads // 2, T)
    for b, L in enumerate(lengths):
        tile, r = divmod(L, 32)
        for t in range(r, 32 if r else 0):
            km[b, :, 32 * tile + t, :] = 0x7F
            vm[b, :, tile, :, _tile_slot(t)] = 0x7F
        kM[b, :, L:] = 0x7E00
        vM[b, :, L:] = 0x7E00
    for dst, src in ((cache.k_micro, km), (cache.v_micro, vm), (cache.k_macro, kM), (cache.v_macro, vM)):
        dst.copy_(torch.from_numpy(np.ascontiguousarray(src).reshape(-1)))
    lens = np.asarray(lengths, dtype=np.int32)
    got = host(fp4.attention_decode_fp4kv(torch.from_numpy(q).cuda().to(torch.bfloat16), cache,
                                          torch.from_numpy(lens).cuda(), out_dtype=torch.float32))
    assert np.all(np.isfinite(got))
    k_hat = oracle.kv_dequantize_rows(k).reshape(n_seq, T, kv_heads, 128)
    v_hat = oracle.kv_dequantize_rows(v).reshape(n_seq, T, kv_heads, 128)
    sc = 1.0 / np.sqrt(128)
    ref = oracle.attention_decode(q, k_hat, v_hat, lens, sc)
    ref_abs = oracle.attention_decode(q, k_hat, np.abs(v_hat), lens, sc)
    attention_gate(got, ref, ref_abs)


def test_attention_deterministic():
    print("[case] attention repeat", flush=True)
    n_seq, kv_heads, q_heads, T = 2, 2, 8, 1024
    rng = np.random.default_rng(80)
    cache = fp4.KvCache(n_seq, T, kv_heads)
    k = torch.from_numpy(workloads.to_bf16_values(_rows(rng, n_seq * T, 256))).cuda().to(torch.bfloat16)
    v = torch.from_numpy(workloads.to_bf16_values(_rows(rng, n_seq * T, 256))).cuda().to(torch.bfloat16)
    fp4.kv_cache_append(cache, k, v, torch.zeros(n_seq, dtype=torch.int32, device="cuda"))
    q = torch.randn(n_seq, q_heads, 128, device="cuda").to(torch.bfloat16)
    lens = torch.tensor([1000, 777], dtype=torch.int32, device="cuda")
    a = fp4.attention_decode_fp4kv(q, cache, lens, out_dtype=torch.float32)
    for _ in range(3):
        assert torch.equal(a, fp4.attention_decode_fp4kv(q, cache, lens, out_dtype=torch.float32))


def test_attention_rejects_bad_shapes():
    cache = fp4.KvCache(1, 64, 2)
    q = torch.zeros(1, 6, 128, dtype=torch.bfloat16, device="cuda")  # 6 % 2 == 0 but group 3 fine
    lens = torch.ones(1, dtype=torch.int32, device="cuda")
    fp4.attention_decode_fp4kv(q, cache, lens)
    with pytest.raises(fp4.Fp4Error):
        fp4.attention_decode_fp4kv(torch.zeros(1, 3, 128, dtype=torch.bfloat16, device="cuda"), cache, lens)
    with pytest.raises(fp4.Fp4Error):  # 17 query heads per KV head
        fp4.attention_decode_fp4kv(torch.zeros(1, 34, 128, dtype=torch.bfloat16, device="cuda"), cache, lens)
    with pytest.raises(fp4.Fp4Error):
        fp4.KvCache(1, 48 + 8, 2)  # max_tokens % 32 != 0
    with pytest.raises(fp4.Fp4Error):
        fp4.KvCache(1, 64, 3)  # odd kv_heads


def test_decode_workload_full_size_sampled():
    """The bench's workload at full size (32 sequences, 8192-16384 cached tokens, 32 query
    heads, 8 KV heads) in the bench's launch configuration; three (sequence, KV head) pairs
    checked against the oracle, the longest context among them."""
    cfg = workloads.WORKLOADS["decode_attention_fp4kv"]
    B, Hq, Hkv, D, T = cfg["n_seq"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"], cfg["max_tokens"]
    group = Hq // Hkv
    lens = workloads.kv_lengths(B, cfg["min_len"], cfg["max_len"], cfg["seed"])
    samples = [(0, 0), (int(np.argmax(lens)), 5), (31, 7)]
    print(f"[case] decode attention full size, samples {samples}", flush=True)
    ch = workloads.kv_key_outliers(Hkv * D, 0.005, cfg["seed"])
    cache = fp4.KvCache(B, T, Hkv)
    chunk = 4096
    keep = {s: ([], []) for s in samples}
    for i, c0 in enumerate(range(0, T, chunk)):
        k = workloads.kv_rows_device(torch, B * chunk, Hkv * D, cfg["seed"], 2 * i, outliers=ch)
        v = workloads.kv_rows_device(torch, B * chunk, Hkv * D, cfg["seed"], 2 * i + 1)
        fp4.kv_cache_append(cache, k, v, torch.full((B,), c0, dtype=torch.int32, device="cuda"))
        for (b, kvh) in samples:
            cols = slice((kvh // 2) * 256, (kvh // 2) * 256 + 256)  # the head pair's group
            keep[(b, kvh)][0].append(host(k[b * chunk:(b + 1) * chunk, cols].float()))
            keep[(b, kvh)][1].append(host(v[b * chunk:(b + 1) * chunk, cols].float()))
        del k, v
    q = workloads.kv_queries(B, Hq, D, cfg["seed"])
    rng = np.random.default_rng((cfg["seed"], 3))
    k1 = rng.standard_normal((B, Hkv * D), dtype=np.float32)
    v1 = rng.standard_normal((B, Hkv * D), dtype=np.float32)
    k1d, v1d = torch.from_numpy(k1).cuda().to(torch.bfloat16), torch.from_numpy(v1).cuda().to(torch.bfloat16)
    fp4.kv_cache_append(cache, k1d, v1d, torch.from_numpy(lens).cuda())
    out = fp4.attention_decode_fp4kv(torch.from_numpy(q).cuda().to(torch.bfloat16), cache,
                                     torch.from_numpy(lens + 1).cuda(), out_dtype=torch.float32)
    got = host(out).astype(np.float64)
    k1b, v1b = bf16_values(k1d), bf16_values(v1d)
    for (b, kvh) in samples:
        L = int(lens[b])
        cols = slice((kvh // 2) * 256, (kvh // 2) * 256 + 256)
        krows = np.concatenate(keep[(b, kvh)][0])[:L]
        vrows = np.concatenate(keep[(b, kvh)][1])[:L]
        krows = np.concatenate([krows, k1b[b:b + 1, cols]])
        vrows = np.concatenate([vrows, v1b[b:b + 1, cols]])
        half = slice((kvh % 2) * 128, (kvh % 2) * 128 + 128)
        k_hat = oracle.kv_dequantize_rows(krows)[:, half].reshape(1, L + 1, 1, D)
        v_hat = oracle.kv_dequantize_rows(vrows)[:, half].reshape(1, L + 1, 1, D)
        heads = slice(kvh * group, (kvh + 1) * group)
        ref = oracle.attention_decode(q[b:b + 1, heads], k_hat, v_hat, [L + 1], 1.0 / np.sqrt(D))
        ref_abs = oracle.attention_decode(q[b:b + 1, heads], k_hat, np.abs(v_hat), [L + 1], 1.0 / np.sqrt(D))
        cond, plain = attention_gate(got[b:b + 1, heads], ref, ref_abs)
        print(f"  sequence {b} KV head {kvh}: {L + 1} tokens, error {cond:.2e} of the weighted "
              f"magnitudes, plain relative {plain:.2e}", flush=True)
