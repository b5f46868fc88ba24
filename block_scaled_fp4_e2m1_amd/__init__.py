"""Python binding of the gfx950 two-level block-scaled FP4 library (libfp4_e2m1.so).

Argument marshalling only: every step of quantization and of the products runs in the
HIP kernels behind the C ABI declared in ``include/fp4_e2m1.h``. torch provides device
memory and the current stream. There is no CPU path: if the library is missing or the
device is not gfx950 the calls raise.

Names follow the C ABI: ``quantize_fp4``, ``dequantize_fp4``, ``gemm_w4aX``,
``grouped_gemm_w4aX``, ``grouped_gemm_w4aX_gated``, ``moe_route``, ``moe_combine``,
``kv_cache_append``, ``attention_decode_fp4kv``, ``quantize_mxfp4``, ``gemm_mxfp4``,
``quantize_fp4_static``, ``act_macro_calibrate``, ``gemm_w4aX_static``, ``gemm_w8a8``,
``repack_fp4``, ``fp4_workspace_bytes``, ``fp4_policy_select``, ``fp4_product_kernel``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4_e2m1.so")

FP4_OK = 0
F32, BF16 = 0, 1
A16, A8, A4 = 16, 8, 4
A4S, A8S, W8A8 = 40, 80, 88
ELEM_E2M1, ELEM_E4M3 = 0, 1
LAYOUT_CANONICAL, LAYOUT_TILED = 0, 1
POLICY_AUTO, POLICY_SENSITIVE_W8, POLICY_STATIC, POLICY_Q4, POLICY_Q8 = 0, 1, 2, 4, 8

EXPORTED = ["quantize_fp4", "dequantize_fp4", "gemm_w4aX", "grouped_gemm_w4aX",
            "grouped_gemm_w4aX_gated", "moe_route", "moe_route_workspace_bytes", "moe_combine",
            "fp4_workspace_bytes", "fp4_policy_select", "fp4_status_string",
            "fp4_device_check", "fp4_kv_cache_bytes", "kv_cache_append",
            "attention_workspace_bytes", "attention_decode_fp4kv", "mxfp4_bytes",
            "quantize_mxfp4", "gemm_mxfp4", "quantize_fp4_static", "act_macro_calibrate",
            "gemm_w4aX_static", "gemm_w8a8", "fp4_product_kernel", "repack_fp4",
            "gemm_w4aX_noalloc"]
NOALLOC_SCRATCH_BYTES = 32 << 20
KV_CODES, KV_MICRO, KV_MACRO = 0, 1, 2


class Fp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class _Tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("micro", ctypes.c_void_p),
                ("macro", ctypes.c_void_p), ("rows", ctypes.c_int64), ("k", ctypes.c_int64),
                ("elem", ctypes.c_int32), ("layout", ctypes.c_int32)]


class _KvCache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_micro", ctypes.c_void_p),
                ("k_macro", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_micro", ctypes.c_void_p), ("v_macro", ctypes.c_void_p),
                ("n_seq", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


_lib = None


def library() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_scaled_fp4_e2m1_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    T = ctypes.POINTER(_Tensor)
    lib.quantize_fp4.argtypes = [vp, i32, i64, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.dequantize_fp4.argtypes = [T, vp, i32, i64, vp]
    lib.gemm_w4aX.argtypes = [i32, vp, i32, i64, i64, T, vp, i32, i64, vp, sz, vp]
    lib.grouped_gemm_w4aX.argtypes = [i32, vp, i32, i64, i64, vp, vp, i32, i64, T, vp, i32,
                                      i64, vp, sz, vp]
    lib.grouped_gemm_w4aX_gated.argtypes = [i32, vp, i64, i64, vp, i32, T, vp, i32, i64, vp, sz, vp]
    lib.moe_route_workspace_bytes.argtypes = [i64, i32]
    lib.moe_route_workspace_bytes.restype = sz
    lib.moe_route.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_combine.argtypes = [vp, i32, i64, vp, vp, i64, i32, i64, vp, i32, i64, vp]
    lib.fp4_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.fp4_workspace_bytes.restype = sz
    lib.fp4_policy_select.argtypes = [i32, i32]
    lib.fp4_policy_select.restype = i32
    lib.fp4_status_string.argtypes = [i32]
    lib.fp4_status_string.restype = ctypes.c_char_p
    lib.fp4_device_check.argtypes = []
    KV = ctypes.POINTER(_KvCache)
    lib.fp4_kv_cache_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.fp4_kv_cache_bytes.restype = sz
    lib.kv_cache_append.argtypes = [KV, vp, vp, i32, i64, vp, i32, vp]
    lib.attention_workspace_bytes.argtypes = [i32, i32, i32]
    lib.attention_workspace_bytes.restype = sz
    lib.attention_decode_fp4kv.argtypes = [vp, i32, KV, vp, ctypes.c_float, vp, i32, vp, sz, vp]
    lib.mxfp4_bytes.argtypes = [i64, i64, i32]
    lib.mxfp4_bytes.restype = sz
    lib.quantize_mxfp4.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    lib.gemm_mxfp4.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, i32, i64, vp]
    lib.quantize_fp4_static.argtypes = [vp, i32, i64, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.act_macro_calibrate.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, vp]
    lib.gemm_w4aX_static.argtypes = [i32, vp, i32, i64, i64, vp, T, vp, i32, i64, vp, sz, vp]
    lib.gemm_w8a8.argtypes = [vp, i32, i64, i64, T, vp, i32, i64, vp, sz, vp]
    lib.repack_fp4.argtypes = [T, i32, vp, vp, vp, vp]
    lib.gemm_w4aX_noalloc.argtypes = [i32, vp, i32, i64, i64, T, vp, i32, i64, vp]
    lib.fp4_product_kernel.argtypes = [i32, i32, i64, i64, i64, i32, i32, i32]
    lib.fp4_product_kernel.restype = ctypes.c_char_p
    for name in ("quantize_fp4", "dequantize_fp4", "gemm_w4aX", "grouped_gemm_w4aX",
                 "grouped_gemm_w4aX_gated", "moe_route", "moe_combine", "fp4_device_check",
                 "kv_cache_append", "attention_decode_fp4kv", "quantize_mxfp4", "gemm_mxfp4",
                 "quantize_fp4_static", "act_macro_calibrate", "gemm_w4aX_static", "gemm_w8a8",
                 "repack_fp4", "gemm_w4aX_noalloc"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().fp4_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != FP4_OK:
        raise Fp4Error(status, where)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}")


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


@dataclass
class QTensor:
    """A quantized [rows x k] tensor in device memory (see include/fp4_e2m1.h)."""
    codes: torch.Tensor   # uint8
    micro: torch.Tensor   # uint8, rows*k/16
    macro: torch.Tensor   # int16 holding FP16 bit patterns, rows*k/256
    rows: int
    k: int
    elem: int = ELEM_E2M1
    layout: int = LAYOUT_CANONICAL

    def c_struct(self) -> _Tensor:
        return _Tensor(self.codes.data_ptr(), self.micro.data_ptr(), self.macro.data_ptr(),
                       self.rows, self.k, self.elem, self.layout)


def empty_qtensor(rows: int, k: int, elem: int = ELEM_E2M1, layout: int = LAYOUT_CANONICAL,
                  device="cuda") -> QTensor:
    ncodes = rows * k // 2 if elem == ELEM_E2M1 else rows * k
    return QTensor(torch.empty(ncodes, dtype=torch.uint8, device=device),
                   torch.empty(rows * k // 16, dtype=torch.uint8, device=device),
                   torch.empty(rows * k // 256, dtype=torch.int16, device=device),
                   rows, k, elem, layout)


def quantize_fp4(x: torch.Tensor, elem: int = ELEM_E2M1, layout: int = LAYOUT_CANONICAL,
                 out: QTensor | None = None) -> QTensor:
    """Two-level block-scaled quantization of a 2-D float32/bf16 device tensor."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    rows, k = x.shape
    q = out if out is not None else empty_qtensor(rows, k, elem, layout, x.device)
    st = library().quantize_fp4(_ptr(x), _dtype_code(x.dtype), rows, k, x.stride(0), elem,
                                layout, _ptr(q.codes), _ptr(q.micro), _ptr(q.macro), _stream())
    _check(st, "quantize_fp4")
    return q


def quantize_fp4_static(x: torch.Tensor, macro_in: torch.Tensor, elem: int = ELEM_E2M1,
                        layout: int = LAYOUT_CANONICAL, out: QTensor | None = None) -> QTensor:
    """quantize_fp4 with the given macro-scales (int16 FP16 bits [k/256], shared by all rows)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    rows, k = x.shape
    if macro_in.numel() != k // 256 or macro_in.element_size() != 2 or not macro_in.is_contiguous():
        raise ValueError("macro_in must hold k/256 contiguous 16-bit values")
    q = out if out is not None else empty_qtensor(rows, k, elem, layout, x.device)
    st = library().quantize_fp4_static(_ptr(x), _dtype_code(x.dtype), rows, k, x.stride(0), elem,
                                       layout, _ptr(macro_in), _ptr(q.codes), _ptr(q.micro),
                                       _ptr(q.macro), _stream())
    _check(st, "quantize_fp4_static")
    return q


def act_macro_calibrate(x: torch.Tensor, amax: torch.Tensor, elem: int = ELEM_E2M1,
                        macro: torch.Tensor | None = None) -> torch.Tensor:
    """Updates the running per-group maximum amax (float32 [k/256], zeroed before the first
    batch) with x [rows, k] and returns the static macro-scales (int16 FP16 bits [k/256])."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    rows, k = x.shape
    if amax.numel() != k // 256 or amax.dtype != torch.float32 or not amax.is_contiguous():
        raise ValueError("amax must be a contiguous float32 tensor of k/256 values")
    if macro is None:
        macro = torch.empty(k // 256, dtype=torch.int16, device=x.device)
    st = library().act_macro_calibrate(_ptr(x), _dtype_code(x.dtype), rows, k, x.stride(0), elem,
                                       _ptr(amax), _ptr(macro), _stream())
    _check(st, "act_macro_calibrate")
    return macro


def repack_fp4(q: QTensor, layout: int, out: QTensor | None = None) -> QTensor:
    """The same quantized tensor in the other packed layout (a byte permutation)."""
    r = out if out is not None else empty_qtensor(q.rows, q.k, q.elem, layout, q.codes.device)
    if r.rows != q.rows or r.k != q.k or r.elem != q.elem or r.layout != layout:
        raise ValueError("out does not match q in the requested layout")
    ts = q.c_struct()
    st = library().repack_fp4(ctypes.byref(ts), layout, _ptr(r.codes), _ptr(r.micro), _ptr(r.macro), _stream())
    _check(st, "repack_fp4")
    return r


def dequantize_fp4(q: QTensor, dtype: torch.dtype = torch.float32,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    y = out if out is not None else torch.empty(q.rows, q.k, dtype=dtype, device=q.codes.device)
    ts = q.c_struct()
    st = library().dequantize_fp4(ctypes.byref(ts), _ptr(y), _dtype_code(y.dtype), y.stride(0),
                                  _stream())
    _check(st, "dequantize_fp4")
    return y


def fp4_workspace_bytes(act: int, m_or_rows: int, n: int, k: int) -> int:
    return int(library().fp4_workspace_bytes(act, m_or_rows, n, k))


def fp4_policy_select(mode: int, layer_flag: bool) -> int:
    r = int(library().fp4_policy_select(mode, int(bool(layer_flag))))
    if r < 0:
        raise Fp4Error(-r, "fp4_policy_select")
    return r


def fp4_device_check() -> int:
    return int(library().fp4_device_check())


def fp4_product_kernel(act: int, a_dtype: torch.dtype, m: int, n: int, k: int, grouped: bool = False,
                       n_experts: int = 0, w_e4m3: bool = False) -> str | None:
    """Name of the kernel form a product of this shape runs (None when it is refused)."""
    r = library().fp4_product_kernel(act, _dtype_code(a_dtype), m, n, k, int(grouped), n_experts,
                                     int(w_e4m3))
    return None if r is None else r.decode()


def _out(out, rows: int, cols: int, dtype: torch.dtype, device) -> torch.Tensor:
    """The product's output: the caller's ``out`` ([rows x cols], contiguous rows, any row
    stride >= cols), checked, or a new tensor."""
    if out is None:
        return torch.empty(rows, cols, dtype=dtype, device=device)
    if out.dim() != 2 or tuple(out.shape) != (rows, cols) or (rows > 0 and out.stride(1) != 1):
        raise ValueError(f"out must be [{rows} x {cols}] with contiguous rows")
    return out


def _workspace(act: int, rows: int, n: int, k: int, device, workspace):
    need = fp4_workspace_bytes(act, rows, n, k)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def gemm_w4aX(act: int, a: torch.Tensor, w: QTensor, out_dtype: torch.dtype = torch.bfloat16,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C = A_hat . W_hat^T (W tiled E2M1 [n x k]); act in {A16, A8, A4}."""
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be 2-D with contiguous rows")
    m = a.shape[0]
    c = _out(out, m, w.rows, out_dtype, a.device)
    ws, wsb = _workspace(act, m, w.rows, w.k, a.device, workspace)
    ts = w.c_struct()
    st = library().gemm_w4aX(act, _ptr(a), _dtype_code(a.dtype), m, a.stride(0), ctypes.byref(ts),
                             _ptr(c), _dtype_code(c.dtype), c.stride(0), _ptr(ws), wsb, _stream())
    _check(st, "gemm_w4aX")
    return c


def gemm_w4aX_noalloc(act: int, a: torch.Tensor, w: QTensor, out: torch.Tensor) -> torch.Tensor:
    """gemm_w4aX without a workspace (the library's per-GPU scratch array); ``out`` is the
    caller's [m x n] output (bf16 or float32), so the call allocates nothing."""
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be 2-D with contiguous rows")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != a.shape[0] or out.shape[1] != w.rows:
        raise ValueError("out must be [m x n] with contiguous rows")
    ts = w.c_struct()
    st = library().gemm_w4aX_noalloc(act, _ptr(a), _dtype_code(a.dtype), a.shape[0], a.stride(0),
                                     ctypes.byref(ts), _ptr(out), _dtype_code(out.dtype), out.stride(0),
                                     _stream())
    _check(st, "gemm_w4aX_noalloc")
    return out


def gemm_w4aX_static(act: int, a: torch.Tensor, act_macro: torch.Tensor, w: QTensor,
                     out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_w4aX (act A4 or A8) with static activation macro-scales act_macro (int16 FP16
    bits [k/256])."""
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be 2-D with contiguous rows")
    if act_macro.numel() != w.k // 256 or act_macro.element_size() != 2 or not act_macro.is_contiguous():
        raise ValueError("act_macro must hold k/256 contiguous 16-bit values")
    m = a.shape[0]
    c = _out(out, m, w.rows, out_dtype, a.device)
    ws, wsb = _workspace(act, m, w.rows, w.k, a.device, workspace)
    ts = w.c_struct()
    st = library().gemm_w4aX_static(act, _ptr(a), _dtype_code(a.dtype), m, a.stride(0), _ptr(act_macro),
                                    ctypes.byref(ts), _ptr(c), _dtype_code(c.dtype), c.stride(0), _ptr(ws),
                                    wsb, _stream())
    _check(st, "gemm_w4aX_static")
    return c


def gemm_w8a8(a: torch.Tensor, w: QTensor, out_dtype: torch.dtype = torch.bfloat16,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C = A8(a) . W_hat^T with W quantized with E4M3 elements in the tiled layout."""
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be 2-D with contiguous rows")
    m = a.shape[0]
    c = _out(out, m, w.rows, out_dtype, a.device)
    ws, wsb = _workspace(W8A8, m, w.rows, w.k, a.device, workspace)
    ts = w.c_struct()
    st = library().gemm_w8a8(_ptr(a), _dtype_code(a.dtype), m, a.stride(0), ctypes.byref(ts), _ptr(c),
                             _dtype_code(c.dtype), c.stride(0), _ptr(ws), wsb, _stream())
    _check(st, "gemm_w8a8")
    return c


def grouped_gemm_w4aX(act: int, a: torch.Tensor, row_token: torch.Tensor | None,
                      expert_offsets: torch.Tensor, n_experts: int, total_rows: int, w: QTensor,
                      out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Mixture-of-experts product over routed rows (experts stacked in w along rows)."""
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be 2-D with contiguous rows")
    n = w.rows // n_experts
    c = _out(out, total_rows, n, out_dtype, a.device)
    ws, wsb = _workspace(act, a.shape[0], n, w.k, a.device, workspace)
    ts = w.c_struct()
    st = library().grouped_gemm_w4aX(act, _ptr(a), _dtype_code(a.dtype), a.shape[0], a.stride(0),
                                     _ptr(row_token), _ptr(expert_offsets), n_experts, total_rows,
                                     ctypes.byref(ts), _ptr(c), _dtype_code(c.dtype), c.stride(0),
                                     _ptr(ws), wsb, _stream())
    _check(st, "grouped_gemm_w4aX")
    return c


def grouped_gemm_w4aX_gated(act: int, gate_up: torch.Tensor, expert_offsets: torch.Tensor,
                            n_experts: int, w: QTensor, out_dtype: torch.dtype = torch.bfloat16,
                            out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Down product of a mixture-of-experts layer: rows of gate_up (bf16 [R x 2k], gate then
    up) become h = bf16(silu(gate) * up), quantized (act A4 / A8) and multiplied by expert
    e's weights (w stacked [n_experts * n x k]) for the rows of expert e."""
    if gate_up.dim() != 2 or gate_up.stride(1) != 1:
        raise ValueError("gate_up must be 2-D with contiguous rows")
    rows, n = gate_up.shape[0], w.rows // n_experts
    c = _out(out, rows, n, out_dtype, gate_up.device)
    ws, wsb = _workspace(act, rows, n, w.k, gate_up.device, workspace)
    ts = w.c_struct()
    st = library().grouped_gemm_w4aX_gated(act, _ptr(gate_up), rows, gate_up.stride(0),
                                           _ptr(expert_offsets), n_experts, ctypes.byref(ts),
                                           _ptr(c), _dtype_code(c.dtype), c.stride(0), _ptr(ws),
                                           wsb, _stream())
    _check(st, "grouped_gemm_w4aX_gated")
    return c


def moe_route(logits: torch.Tensor, top_k: int, workspace: torch.Tensor | None = None,
              out: tuple | None = None):
    """Float32 top-k routing. Returns (topk_ids int32 [T x k], topk_weights float32 [T x k],
    expert_offsets int32 [E + 1], row_token int32 [T * k], token_rows int32 [T x k]); with
    ``out`` (a tuple of those five tensors) the results are written there."""
    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous float32 [tokens x experts] tensor")
    t_count, e_count = logits.shape
    dev = logits.device
    shapes = [((t_count, top_k), torch.int32), ((t_count, top_k), torch.float32),
              ((e_count + 1,), torch.int32), ((t_count * top_k,), torch.int32),
              ((t_count, top_k), torch.int32)]
    if out is None:
        out = tuple(torch.empty(shp, dtype=dt, device=dev) for shp, dt in shapes)
    elif len(out) != 5 or any(tuple(o.shape) != shp or o.dtype != dt or not o.is_contiguous()
                              for o, (shp, dt) in zip(out, shapes)):
        raise ValueError("out must hold five contiguous tensors of the documented shapes and dtypes")
    ids, wts, offsets, row_token, token_rows = out
    lib = library()
    need = int(lib.moe_route_workspace_bytes(t_count, e_count))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.moe_route(_ptr(logits), t_count, e_count, top_k, _ptr(ids), _ptr(wts), _ptr(offsets),
                       _ptr(row_token), _ptr(token_rows), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "moe_route")
    return ids, wts, offsets, row_token, token_rows


def moe_combine(y: torch.Tensor, token_rows: torch.Tensor, topk_weights: torch.Tensor,
                out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """out[t] = sum_j topk_weights[t, j] * y[token_rows[t, j]] (float32 sums, j in order)."""
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be 2-D with contiguous rows")
    if (token_rows.dim() != 2 or token_rows.dtype != torch.int32 or not token_rows.is_contiguous()
            or topk_weights.shape != token_rows.shape or topk_weights.dtype != torch.float32
            or not topk_weights.is_contiguous()):
        raise ValueError("token_rows (int32) and topk_weights (float32) must be contiguous [T x k]")
    t_count, top_k = token_rows.shape
    hidden = y.shape[1]
    o = out if out is not None else torch.empty(t_count, hidden, dtype=out_dtype, device=y.device)
    st = library().moe_combine(_ptr(y), _dtype_code(y.dtype), y.stride(0), _ptr(token_rows),
                               _ptr(topk_weights), t_count, top_k, hidden, _ptr(o),
                               _dtype_code(o.dtype), o.stride(0), _stream())
    _check(st, "moe_combine")
    return o


class KvCache:
    """Device arrays of a KV cache in the two-level FP4 format (layout: include/fp4_e2m1.h).
    Only allocation happens here (torch); the arrays are filled by ``kv_cache_append``."""

    def __init__(self, n_seq: int, max_tokens: int, kv_heads: int, head_dim: int = 128,
                 device="cuda"):
        lib = library()
        sizes = [int(lib.fp4_kv_cache_bytes(n_seq, max_tokens, kv_heads, head_dim, part))
                 for part in (KV_CODES, KV_MICRO, KV_MACRO)]
        if sizes[0] == 0:
            raise Fp4Error(2, "KvCache")
        self.n_seq, self.max_tokens, self.kv_heads, self.head_dim = n_seq, max_tokens, kv_heads, head_dim
        self.k_codes = torch.zeros(sizes[0], dtype=torch.uint8, device=device)
        self.k_micro = torch.zeros(sizes[1], dtype=torch.uint8, device=device)
        self.k_macro = torch.zeros(sizes[2] // 2, dtype=torch.int16, device=device)
        self.v_codes = torch.zeros(sizes[0], dtype=torch.uint8, device=device)
        self.v_micro = torch.zeros(sizes[1], dtype=torch.uint8, device=device)
        self.v_macro = torch.zeros(sizes[2] // 2, dtype=torch.int16, device=device)

    def c_struct(self) -> _KvCache:
        return _KvCache(self.k_codes.data_ptr(), self.k_micro.data_ptr(), self.k_macro.data_ptr(),
                        self.v_codes.data_ptr(), self.v_micro.data_ptr(), self.v_macro.data_ptr(),
                        self.n_seq, self.max_tokens, self.kv_heads, self.head_dim)


def kv_cache_append(cache: KvCache, k_new: torch.Tensor, v_new: torch.Tensor,
                    positions: torch.Tensor) -> None:
    """k_new, v_new [n_seq * n_new, kv_heads * head_dim] (bf16 or float32): row
    b * n_new + i becomes token positions[b] + i of sequence b."""
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype or k_new.dim() != 2 or \
            k_new.stride(0) != v_new.stride(0) or k_new.stride(1) != 1 or v_new.stride(1) != 1:
        raise ValueError("k_new and v_new must be 2-D with equal shapes, dtypes and row strides")
    if positions.dtype != torch.int32 or positions.numel() != cache.n_seq:
        raise ValueError("positions must be int32 [n_seq]")
    n_new = k_new.shape[0] // cache.n_seq
    if n_new * cache.n_seq != k_new.shape[0]:
        raise ValueError("k_new rows must be n_seq * n_new")
    cs = cache.c_struct()
    st = library().kv_cache_append(ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _dtype_code(k_new.dtype),
                                   k_new.stride(0), _ptr(positions), n_new, _stream())
    _check(st, "kv_cache_append")


def attention_decode_fp4kv(q: torch.Tensor, cache: KvCache, lengths: torch.Tensor,
                           scale: float | None = None, out_dtype: torch.dtype = torch.bfloat16,
                           out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """q bf16 [n_seq, q_heads, head_dim] -> out [n_seq, q_heads, head_dim]."""
    if q.dim() != 3 or q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [n_seq, q_heads, head_dim] tensor")
    if lengths.dtype != torch.int32 or lengths.numel() != cache.n_seq:
        raise ValueError("lengths must be int32 [n_seq]")
    q_heads = q.shape[1]
    o = out if out is not None else torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if not o.is_contiguous() or o.shape != q.shape:
        raise ValueError("out must be contiguous with the shape of q")
    lib = library()
    need = int(lib.attention_workspace_bytes(cache.n_seq, q_heads, cache.max_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    cs = cache.c_struct()
    sc = (1.0 / cache.head_dim ** 0.5) if scale is None else float(scale)
    st = lib.attention_decode_fp4kv(_ptr(q), q_heads, ctypes.byref(cs), _ptr(lengths), sc, _ptr(o),
                                    _dtype_code(o.dtype), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "attention_decode_fp4kv")
    return o


@dataclass
class MxTensor:
    """MX-native FP4 tensor in the tiled layout (include/fp4_e2m1.h): codes, E8M0 scales."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    k: int


def quantize_mxfp4(x: torch.Tensor, out: MxTensor | None = None) -> MxTensor:
    """x [rows, k] (bf16 or float32, contiguous rows) -> MX-native FP4 (tiled)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    rows, k = x.shape
    lib = library()
    nc, ns = int(lib.mxfp4_bytes(rows, k, 0)), int(lib.mxfp4_bytes(rows, k, 1))
    if nc == 0:
        raise Fp4Error(2, "quantize_mxfp4")
    q = out if out is not None else MxTensor(torch.empty(nc, dtype=torch.uint8, device=x.device),
                                             torch.empty(ns, dtype=torch.uint8, device=x.device), rows, k)
    if q.codes.numel() < nc or q.scales.numel() < ns or q.rows != rows or q.k != k:
        raise ValueError("out does not match x")
    st = lib.quantize_mxfp4(_ptr(x), _dtype_code(x.dtype), rows, k, x.stride(0), _ptr(q.codes), _ptr(q.scales),
                            _stream())
    _check(st, "quantize_mxfp4")
    return q


def gemm_mxfp4(a: MxTensor, w: MxTensor, out_dtype: torch.dtype = torch.bfloat16,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """C [a.rows, w.rows] = A_hat . W_hat^T on the block-scaled FP4 matrix instruction."""
    if a.k != w.k:
        raise ValueError("a and w must have the same k")
    c = _out(out, a.rows, w.rows, out_dtype, a.codes.device)
    st = library().gemm_mxfp4(_ptr(a.codes), _ptr(a.scales), a.rows, _ptr(w.codes), _ptr(w.scales), w.rows, a.k,
                              _ptr(c), _dtype_code(c.dtype), c.stride(0), _stream())
    _check(st, "gemm_mxfp4")
    return c
