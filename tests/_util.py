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


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def qtensor_to_canonical(q, rows: int, k: int):
    """(codes [rows, k/2 or k], micro [rows, k/16], macro uint16 [rows, k/256]) on host."""
    codes = host(q.codes).astype(np.uint8)
    micro = host(q.micro).astype(np.uint8)
    macro = host(q.macro).view(np.uint16)
    if q.layout == 1:
        ci, mi, gi = tiled_index_maps(rows, k)
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
