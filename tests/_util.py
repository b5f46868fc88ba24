"""Test-side helpers: the documented tiled layout as a numpy permutation, the output gates,
and device/host conversions. Nothing here computes the method's arithmetic."""
from __future__ import annotations

import numpy as np
import torch


def tiled_index_maps(rows: int, k: int):
    """Index arrays I such that canonical = tiled[I] for codes, micro and macro, written
    from the tiled-layout definition in include/fp4_e2m1.h."""
    G = k // 256
    r = np.arange(rows)[:, None]
    n = r % 16
    # codes: canonical byte (r, cb) holds columns 2cb, 2cb+1
    col = 2 * np.arange(k // 2)[None, :]
    T = (r // 16) * G + col // 256
    c = col % 256
    t, j = c // 32, (c % 32) // 8
    code_idx = T * 2048 + (t // 4) * 1024 + (16 * j + n) * 16 + (t % 4) * 4 + (c % 8) // 2
    # micro: canonical (r, b)
    b = np.arange(k // 16)[None, :]
    T = (r // 16) * G + b // 16
    bb = b % 16
    micro_idx = T * 256 + (bb % 2) * 128 + n * 8 + bb // 2
    # macro: canonical (r, g)
    g = np.arange(G)[None, :]
    macro_idx = ((r // 16) * G + g) * 16 + n
    return code_idx, micro_idx, macro_idx


def tiled8_code_index(rows: int, k: int):
    """Index array I such that canonical E4M3 codes = tiled[I], from the E4M3 tiled-layout
    definition in include/fp4_e2m1.h (micro and macro share the E2M1 maps)."""
    G = k // 256
    r = np.arange(rows)[:, None]
    n = r % 16
    col = np.arange(k)[None, :]
    T = (r // 16) * G + col // 256
    c = col % 256
    t, j = c // 32, (c % 32) // 8
    return T * 4096 + (t // 4) * 2048 + ((t % 4) // 2) * 1024 + (16 * j + n) * 16 + (t % 2) * 8 + c % 8


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def qtensor_to_canonical(q, rows: int, k: int):
    """(codes [rows, k/2 or k], micro [rows, k/16], macro uint16 [rows, k/256]) on host."""
    codes = host(q.codes).astype(np.uint8)
    micro = host(q.micro).astype(np.uint8)
    macro = host(q.macro).view(np.uint16)
    if q.layout == 1:
        ci, mi, gi = tiled_index_maps(rows, k)
        if q.elem == 1:
            ci = tiled8_code_index(rows, k)
        return codes[ci], micro[mi], macro[gi]
    width = k // 2 if q.elem == 0 else k
    return codes.reshape(rows, width), micro.reshape(rows, k // 16), macro.reshape(rows, k // 256)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    return host(t.to(torch.float32)).astype(np.float64)


def to_device_bf16(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(torch.bfloat16)


def bf16_gate(got: np.ndarray, want_bf16: np.ndarray, rel_frob: float = 1e-3,
              frac_within_1ulp: float = 0.999):
    """bf16 output gate: relative Frobenius error against RNE_bf16(exact) <= rel_frob, and
    at least frac_within_1ulp of elements equal or one bf16 step apart."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want_bf16, np.float64)
    denom = np.linalg.norm(want)
    rel = np.linalg.norm(got - want) / (denom if denom > 0 else 1.0)
    gb = torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int32)
    wb = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int32)
    # ordered integer view of bf16 so neighbours differ by 1 across the sign change too
    def ordered(b):
        b = b & 0xFFFF
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    ulps = np.abs(ordered(gb) - ordered(wb))
    frac = float(np.mean(ulps <= 1)) if ulps.size else 1.0
    assert rel <= rel_frob, f"relative Frobenius error {rel:.3e} > {rel_frob}"
    assert frac >= frac_within_1ulp, f"only {frac:.5f} of elements within 1 bf16 ulp"
    return rel, frac


def f32_gate(got: np.ndarray, want: np.ndarray, rel_frob: float = 1e-5):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    assert rel <= rel_frob, f"relative Frobenius error {rel:.3e} > {rel_frob}"
    return rel


def kv_slot_of_token():
    """Slot of each token (0..31) inside a 32-token V tile (include/fp4_e2m1.h: slot 8g + i
    is token 4g + i for i < 4 and 16 + 4g + i - 4 for i >= 4)."""
    slot = np.zeros(32, dtype=np.int64)
    for g in range(4):
        for i in range(8):
            tok = 4 * g + i if i < 4 else 16 + 4 * g + i - 4
            slot[tok] = 8 * g + i
    return slot


def kv_cache_to_canonical(cache, which: str, b: int, tokens):
    """Canonical codec rows (codes4 uint8 [n, H*128], micro [n, H*8], macro uint16 [n, H/2])
    of the given tokens of sequence b, read back from the documented device layout."""
    H, T = cache.kv_heads, cache.max_tokens
    tokens = np.asarray(tokens, dtype=np.int64)
    codes_dev = host(getattr(cache, which + "_codes")).astype(np.uint8)
    micro_dev = host(getattr(cache, which + "_micro")).astype(np.uint8)
    macro_dev = host(getattr(cache, which + "_macro")).view(np.uint16)
    n = len(tokens)
    codes4 = np.zeros((n, H * 128), dtype=np.uint8)
    micro = np.zeros((n, H * 8), dtype=np.uint8)
    macro = np.zeros((n, H // 2), dtype=np.uint16)
    slot = kv_slot_of_token()
    d = np.arange(128)
    for h in range(H):
        th = b * H + h
        for r, t in enumerate(tokens):
            if which == "k":
                rec = codes_dev[(th * T + t) * 64:(th * T + t + 1) * 64]
                words = rec.view(np.uint32)
                # dword 4g + s holds d = 32s + 8g + i
                for gg in range(4):
                    for s in range(4):
                        w = int(words[4 * gg + s])
                        for i in range(8):
                            codes4[r, h * 128 + 32 * s + 8 * gg + i] = (w >> (4 * i)) & 15
                micro[r, h * 8:(h + 1) * 8] = micro_dev[(th * T + t) * 8:(th * T + t + 1) * 8]
            else:
                tile, sl = t // 32, slot[t % 32]
                base = (th * (T // 32) + tile) * 2048
                byte = codes_dev[base + d * 16 + sl // 2]
                codes4[r, h * 128:(h + 1) * 128] = (byte >> (4 * (sl % 2))) & 15
                mbase = (th * (T // 32) + tile) * 256
                micro[r, h * 8:(h + 1) * 8] = micro_dev[mbase + np.arange(8) * 32 + sl]
    for pr in range(H // 2):
        macro[:, pr] = macro_dev[(b * (H // 2) + pr) * T + tokens]
    return codes4, micro, macro


def mx_tiled_to_canonical(q):
    """(codes4 uint8 [rows, k], scales uint8 [rows, k/32], padding codes, padding scales)
    of an MX tensor, read back through the tiled layout of include/fp4_e2m1.h."""
    rows, k = q.rows, q.k
    pr = (rows + 15) // 16 * 16
    codes = host(q.codes).astype(np.uint8)[: pr * k // 2].reshape(pr // 16, k // 128, 4, 16, 16)
    scales = host(q.scales).astype(np.uint8)[: pr * k // 32].reshape(pr // 16, k // 128, 4, 16)
    # codes [rb][kt][kb][n][byte] -> row rb*16+n, column kt*128 + kb*32 + 2*byte (+1)
    c = codes.transpose(0, 3, 1, 2, 4).reshape(pr, k // 2)
    codes4 = np.empty((pr, k), dtype=np.uint8)
    codes4[:, 0::2] = c & 15
    codes4[:, 1::2] = c >> 4
    s = scales.transpose(0, 3, 1, 2).reshape(pr, k // 32)
    return codes4[:rows], s[:rows], codes4[rows:], s[rows:]
