// C ABI of the gfx950 two-level block-scaled FP4 library: argument validation, the
// device-architecture check, and dispatch to the kernels. Every error is reported before
// anything is enqueued; no other precision or path is ever substituted.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/fp4_e2m1.h"
#include "fp4_kernels.h"

namespace {

constexpr int kMaxDevices = 64;
int g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

fp4_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP4_E_NO_DEVICE;
  if (dev < kMaxDevices && g_arch_state[dev] != 0) return g_arch_state[dev] == 1 ? FP4_OK : FP4_E_ARCH;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP4_E_NO_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev] = ok ? 1 : 2;
  return ok ? FP4_OK : FP4_E_ARCH;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t dtype_size(int32_t dt) { return dt == FP4_F32 ? 4 : 2; }
bool valid_dtype(int32_t dt) { return dt == FP4_F32 || dt == FP4_BF16; }
bool valid_act(int32_t act) { return act == FP4_A16 || act == FP4_A8 || act == FP4_A4; }

fp4_status launched(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_E_HIP; }

// Checks on a quantized weight tensor shared by the matrix entry points (elem: the
// element type the product takes).
fp4_status check_weights(const fp4_tensor* w, int32_t elem = FP4_ELEM_E2M1) {
  if (!w || !w->codes || !w->micro || !w->macro) return FP4_E_NULL;
  if (w->elem != FP4_ELEM_E2M1 && w->elem != FP4_ELEM_E4M3) return FP4_E_MODE;
  if (w->elem != elem) return FP4_E_DTYPE;
  if (w->layout != FP4_LAYOUT_TILED)
    return w->layout == FP4_LAYOUT_CANONICAL ? FP4_E_LAYOUT : FP4_E_MODE;
  if (w->rows < 16 || w->rows % 16 || w->k < 256 || w->k % 256) return FP4_E_SHAPE;
  if (!aligned16(w->codes) || !aligned16(w->micro) || !aligned(w->macro, 8)) return FP4_E_ALIGN;
  return FP4_OK;
}

// Row stride (elements) of the FP16 activation workspace. Dense rows: padding the rows
// (k + 64) measured slower with the product kernel's LDS-DMA operand copies.
int64_t act_ws_stride(int64_t k) { return k; }

// precision codes of the policy table -> the activation quantization they run
int32_t act_of(int32_t code) {
  switch (code) {
    case FP4_A4S: return FP4_A4;
    case FP4_A8S: case FP4_W8A8: return FP4_A8;
    default: return code;
  }
}

size_t act_workspace(int32_t act, int64_t rows, int64_t k) {
  if (act == FP4_A16) return 0;
  const size_t aq = ((size_t)rows * (size_t)act_ws_stride(k) * 2 + 255) & ~(size_t)255;
  return aq + (size_t)rows * (size_t)(k / 256) * 4;
}

// Scratch of gemm_w4aX_noalloc, for callers that cannot allocate: the activation pass's
// FP16 operand and per-group factors live here instead of a caller workspace. Each GPU
// holds its own copy for the life of the process. In host code `scratch` names a host-side
// stand-in, not device memory: host code only ever uses the device address that
// hipGetSymbolAddress returns for the current device (looked up once per device and kept).
constexpr size_t kScratchBytes = FP4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

fp4_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP4_E_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  void* p = dev < kMaxDevices ? g_scratch_ptr[dev] : nullptr;
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP4_E_HIP;
    if (dev < kMaxDevices) g_scratch_ptr[dev] = p;
  }
  *out = p;
  return FP4_OK;
}

// Launch limits of the matrix path a call takes (the activation pass over act_rows rows
// for FP4_A4 / FP4_A8, then the product kernel), checked before anything is enqueued so
// that a shape the kernels do not cover returns FP4_E_SHAPE with the stream untouched.
fp4_status check_product(int32_t act, int64_t act_rows, int64_t m, int64_t n, int64_t k, bool grouped,
                         int32_t n_experts, bool w_e4m3) {
  if (!fp4lib::gemm_plan_ok(m, n, k, grouped ? 1 : 0, n_experts, w_e4m3 ? 1 : 0)) return FP4_E_SHAPE;
  if (act != FP4_A16 && !fp4lib::quantize_grid_ok(act_rows, k)) return FP4_E_SHAPE;
  return FP4_OK;
}

// Runs the activation pass when needed and fills the activation part of GemmArgs.
// act_macro: static activation macro-scales (FP16 bits per group) or nullptr (dynamic).
fp4_status prepare_activations(int32_t act, const void* a, int32_t a_dtype, int64_t rows,
                               int64_t k, int64_t lda, void* ws, fp4lib::GemmArgs& g,
                               hipStream_t st, const uint16_t* act_macro = nullptr) {
  if (act == FP4_A16) {
    g.a = a;
    g.a_is_bf16 = 1;
    g.lda = lda;
    g.a_scale = nullptr;
    return FP4_OK;
  }
  const int64_t ldq = act_ws_stride(k);
  _Float16* aq = static_cast<_Float16*>(ws);
  float* scale = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                          (((size_t)rows * (size_t)ldq * 2 + 255) & ~(size_t)255));
  const hipError_t e = fp4lib::launch_act_prep(a, a_dtype == FP4_BF16, rows, k, lda,
                                               act == FP4_A8, aq, ldq, scale, act_macro, st);
  if (e != hipSuccess) return FP4_E_HIP;
  g.a = aq;
  g.a_is_bf16 = 0;
  g.lda = ldq;
  g.a_scale = scale;
  return FP4_OK;
}

// W4A4 on the 128-row-wave form: the activations are quantized to E2M1 in the canonical
// layout (quantize_fp4's output: codes, micro-scales, macro-scales, each 256-byte aligned
// in the workspace, together smaller than the FP16 operand of the activation pass) and
// the product kernel decodes them into the same FP16 operand itself.
fp4_status prepare_packed_a4(const void* a, int32_t a_dtype, int64_t rows, int64_t k, int64_t lda, void* ws,
                             fp4lib::GemmArgs& g, hipStream_t st) {
  if (!fp4lib::quantize_grid_ok(rows, k)) return FP4_E_SHAPE;
  const auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t* codes = static_cast<uint8_t*>(ws);
  uint8_t* micro = codes + up((size_t)rows * (size_t)(k / 2));
  uint16_t* macro = reinterpret_cast<uint16_t*>(micro + up((size_t)rows * (size_t)(k / 16)));
  const hipError_t e = fp4lib::launch_quantize(a, a_dtype == FP4_BF16, rows, k, lda, 0, 0, codes, micro, macro,
                                               nullptr, st);
  if (e != hipSuccess) return FP4_E_HIP;
  g.a = codes;
  g.a_is_bf16 = 0;
  g.lda = k / 2;
  g.a_scale = nullptr;
  g.a_packed = 1;
  g.a_micro = micro;
  g.a_macro = macro;
  return FP4_OK;
}

}  // namespace

extern "C" {

const char* fp4_status_string(fp4_status s) {
  switch (s) {
    case FP4_OK: return "ok";
    case FP4_E_NULL: return "null pointer";
    case FP4_E_SHAPE: return "invalid shape";
    case FP4_E_ALIGN: return "misaligned pointer or stride";
    case FP4_E_DTYPE: return "unsupported dtype combination";
    case FP4_E_MODE: return "unknown mode, element type or layout";
    case FP4_E_NO_DEVICE: return "no HIP device";
    case FP4_E_ARCH: return "device is not gfx950";
    case FP4_E_HIP: return "HIP launch failed";
    case FP4_E_WORKSPACE: return "workspace missing or too small";
    case FP4_E_LAYOUT: return "wrong packed layout for this operation";
    default: return "unknown status";
  }
}

fp4_status fp4_device_check(void) { return check_device(); }

const char* fp4_product_kernel(int32_t act, int32_t a_dtype, int64_t m, int64_t n, int64_t k, int32_t grouped,
                               int32_t n_experts, int32_t w_e4m3) {
  if (act == FP4_A4 && !grouped && !w_e4m3 && valid_dtype(a_dtype) && m >= 1 && n >= 16 && n % 16 == 0 &&
      k >= 256 && k % 256 == 0 && fp4lib::gemm_packed_a4(m, n, k))
    return "k_gemm_r8 (128 x 256, 8 waves of 128 x 32; E2M1 activations decoded in the kernel)";
  act = act_of(act);
  if (!valid_act(act) || !valid_dtype(a_dtype) || m < 1 || n < 16 || n % 16 || k < 256 || k % 256) return nullptr;
  if (w_e4m3 && (act != FP4_A8 || grouped)) return nullptr;
  if (!grouped && !w_e4m3 && act == FP4_A16) {
    if (a_dtype == FP4_F32) return m <= (int64_t)0xFFFFFF00 / n ? "k_gemm_f32act (one thread per output)" : nullptr;
    if (fp4lib::gemv_supports(m, n, k)) return "k_gemv_bf16 (decode)";
  }
  if (grouped && act == FP4_A16 && a_dtype != FP4_BF16) return nullptr;
  return fp4lib::gemm_kernel_name(m, n, k, grouped ? 1 : 0, n_experts, w_e4m3 ? 1 : 0);
}

int32_t fp4_policy_select(int32_t mode, int32_t layer_flag) {
  switch (mode) {
    case FP4_POLICY_Q4: return FP4_A4;
    case FP4_POLICY_Q8: return FP4_A8;
    case FP4_POLICY_AUTO: return layer_flag ? FP4_A8 : FP4_A4;
    case FP4_POLICY_SENSITIVE_W8: return layer_flag ? FP4_W8A8 : FP4_A4;
    case FP4_POLICY_STATIC: return layer_flag ? FP4_A8S : FP4_A4S;
    default: return -FP4_E_MODE;
  }
}

size_t fp4_workspace_bytes(int32_t act, int64_t m_or_rows, int64_t n, int64_t k) {
  (void)n;
  act = act_of(act);
  if (!valid_act(act) || m_or_rows < 0 || k < 0) return 0;
  return act_workspace(act, m_or_rows, k);
}

namespace {
fp4_status quantize_impl(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx,
                         int32_t elem, int32_t layout, const uint16_t* macro_in, void* codes,
                         uint8_t* micro, uint16_t* macro, void* stream) {
  if (!x || !codes || !micro || !macro) return FP4_E_NULL;
  if (!valid_dtype(x_dtype)) return FP4_E_DTYPE;
  if (elem != FP4_ELEM_E2M1 && elem != FP4_ELEM_E4M3) return FP4_E_MODE;
  if (layout != FP4_LAYOUT_CANONICAL && layout != FP4_LAYOUT_TILED) return FP4_E_MODE;
  if (rows < 1 || k < 256 || k % 256 || ldx < k) return FP4_E_SHAPE;
  if (layout == FP4_LAYOUT_TILED && rows % 16) return FP4_E_SHAPE;
  if (!fp4lib::quantize_grid_ok(rows, k)) return FP4_E_SHAPE;
  if (!aligned16(x) || (ldx * (int64_t)dtype_size(x_dtype)) % 16 || !aligned16(codes) ||
      !aligned16(micro) || !aligned(macro, 2) || (macro_in && !aligned(macro_in, 2)))
    return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_quantize(x, x_dtype == FP4_BF16, rows, k, ldx,
                                          elem == FP4_ELEM_E4M3, layout == FP4_LAYOUT_TILED,
                                          static_cast<uint8_t*>(codes), micro, macro, macro_in,
                                          static_cast<hipStream_t>(stream)));
}
}  // namespace

fp4_status quantize_fp4(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx,
                        int32_t elem, int32_t layout, void* codes, uint8_t* micro,
                        uint16_t* macro, void* stream) {
  return quantize_impl(x, x_dtype, rows, k, ldx, elem, layout, nullptr, codes, micro, macro, stream);
}

fp4_status quantize_fp4_static(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx,
                               int32_t elem, int32_t layout, const uint16_t* macro_in, void* codes,
                               uint8_t* micro, uint16_t* macro, void* stream) {
  if (!macro_in) return FP4_E_NULL;
  return quantize_impl(x, x_dtype, rows, k, ldx, elem, layout, macro_in, codes, micro, macro, stream);
}

fp4_status repack_fp4(const fp4_tensor* src, int32_t layout, void* codes, uint8_t* micro, uint16_t* macro,
                      void* stream) {
  if (!src || !src->codes || !src->micro || !src->macro || !codes || !micro || !macro) return FP4_E_NULL;
  if (src->elem != FP4_ELEM_E2M1 && src->elem != FP4_ELEM_E4M3) return FP4_E_MODE;
  if ((src->layout != FP4_LAYOUT_CANONICAL && src->layout != FP4_LAYOUT_TILED) ||
      (layout != FP4_LAYOUT_CANONICAL && layout != FP4_LAYOUT_TILED))
    return FP4_E_MODE;
  if (layout == src->layout) return FP4_E_LAYOUT;
  if (!fp4lib::repack_supports(src->rows, src->k, src->elem == FP4_ELEM_E4M3)) return FP4_E_SHAPE;
  if (!aligned16(src->codes) || !aligned16(src->micro) || !aligned(src->macro, 2) || !aligned16(codes) ||
      !aligned16(micro) || !aligned(macro, 2))
    return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_repack(static_cast<const uint8_t*>(src->codes), src->micro, src->macro,
                                        static_cast<uint8_t*>(codes), micro, macro, src->rows, src->k,
                                        src->elem == FP4_ELEM_E4M3, layout == FP4_LAYOUT_TILED,
                                        static_cast<hipStream_t>(stream)));
}

fp4_status act_macro_calibrate(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx,
                               int32_t elem, float* amax, uint16_t* macro, void* stream) {
  if (!x || !amax || !macro) return FP4_E_NULL;
  if (!valid_dtype(x_dtype)) return FP4_E_DTYPE;
  if (elem != FP4_ELEM_E2M1 && elem != FP4_ELEM_E4M3) return FP4_E_MODE;
  if (rows < 1 || k < 256 || k % 256 || ldx < k || k / 256 > 0x7FFFFFFF) return FP4_E_SHAPE;
  if (!aligned16(x) || (ldx * (int64_t)dtype_size(x_dtype)) % 16 || !aligned(amax, 4) || !aligned(macro, 2))
    return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_act_calibrate(x, x_dtype == FP4_BF16, rows, k, ldx, elem == FP4_ELEM_E4M3,
                                               amax, macro, static_cast<hipStream_t>(stream)));
}

fp4_status dequantize_fp4(const fp4_tensor* q, void* y, int32_t y_dtype, int64_t ldy,
                          void* stream) {
  if (!q || !q->codes || !q->micro || !q->macro || !y) return FP4_E_NULL;
  if (!valid_dtype(y_dtype)) return FP4_E_DTYPE;
  if (q->elem != FP4_ELEM_E2M1 && q->elem != FP4_ELEM_E4M3) return FP4_E_MODE;
  if (q->layout != FP4_LAYOUT_CANONICAL && q->layout != FP4_LAYOUT_TILED) return FP4_E_MODE;
  if (q->rows < 1 || q->k < 256 || q->k % 256 || ldy < q->k) return FP4_E_SHAPE;
  if (q->layout == FP4_LAYOUT_TILED && q->rows % 16) return FP4_E_SHAPE;
  if (!fp4lib::dequantize_grid_ok(q->rows, q->k)) return FP4_E_SHAPE;
  if (!aligned16(y) || (ldy * (int64_t)dtype_size(y_dtype)) % 16 || !aligned16(q->codes) ||
      !aligned(q->macro, 2))
    return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_dequantize(
      static_cast<const uint8_t*>(q->codes), q->micro, q->macro, q->rows, q->k,
      q->elem == FP4_ELEM_E4M3, q->layout == FP4_LAYOUT_TILED, y, y_dtype == FP4_BF16, ldy,
      static_cast<hipStream_t>(stream)));
}

namespace {
// gemm_w4aX with either a caller workspace or (noalloc) this device's scratch array.
fp4_status gemm_w4aX_impl(int32_t act, const void* a, int32_t a_dtype, int64_t m, int64_t lda,
                          const fp4_tensor* w, void* c, int32_t c_dtype, int64_t ldc, void* workspace,
                          size_t workspace_bytes, void* stream, bool noalloc) {
  if (!valid_act(act)) return FP4_E_MODE;
  if (!a || !c) return FP4_E_NULL;
  const fp4_status ws_ok = check_weights(w);
  if (ws_ok != FP4_OK) return ws_ok;
  if (!valid_dtype(a_dtype) || !valid_dtype(c_dtype)) return FP4_E_DTYPE;
  const int64_t n = w->rows, k = w->k;
  if (m < 1 || lda < k || ldc < n || ldc > FP4_MAX_LDC) return FP4_E_SHAPE;
  if (!aligned16(a) || (lda * (int64_t)dtype_size(a_dtype)) % 16) return FP4_E_ALIGN;
  if (!aligned(c, dtype_size(c_dtype))) return FP4_E_ALIGN;
  const size_t need = act_workspace(act, m, k);
  if (noalloc) {
    if (need > kScratchBytes) return FP4_E_WORKSPACE;
  } else if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) {
    return FP4_E_WORKSPACE;
  }
  // path: float32 activations (A16) -> one thread per output; A16 bf16 with m <= 8 -> the
  // decode GEMV; everything else -> activation pass (A4 / A8) and the product kernel
  const bool f32_path = act == FP4_A16 && a_dtype == FP4_F32;
  const bool gemv_path = act == FP4_A16 && !f32_path && fp4lib::gemv_supports(m, n, k);
  if (f32_path && m > (int64_t)0xFFFFFF00 / n) return FP4_E_SHAPE;
  if (!f32_path && !gemv_path) {
    const fp4_status lim = check_product(act, m, m, n, k, false, 0, false);
    if (lim != FP4_OK) return lim;
  }
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  if (noalloc && need) {
    const fp4_status sa = scratch_address(&workspace);
    if (sa != FP4_OK) return sa;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* codes = static_cast<const uint8_t*>(w->codes);

  if (f32_path)
    return launched(fp4lib::launch_gemm_f32act(static_cast<const float*>(a), lda, m, k, codes,
                                               w->micro, w->macro, n, c, c_dtype == FP4_BF16,
                                               ldc, st));
  if (gemv_path)
    return launched(fp4lib::launch_gemv_bf16(static_cast<const uint16_t*>(a), lda, m, k, codes,
                                             w->micro, w->macro, n, c, c_dtype == FP4_BF16,
                                             ldc, st));
  fp4lib::GemmArgs g{};
  const fp4_status prep = act == FP4_A4 && fp4lib::gemm_packed_a4(m, n, k)
                              ? prepare_packed_a4(a, a_dtype, m, k, lda, workspace, g, st)
                              : prepare_activations(act, a, a_dtype, m, k, lda, workspace, g, st);
  if (prep != FP4_OK) return prep;
  g.m = m;
  g.n = n;
  g.k = k;
  g.codes = codes;
  g.micro = w->micro;
  g.macro = w->macro;
  g.c = c;
  g.c_is_bf16 = c_dtype == FP4_BF16;
  g.ldc = ldc;
  return launched(fp4lib::launch_gemm(g, st));
}
}  // namespace

fp4_status gemm_w4aX(int32_t act, const void* a, int32_t a_dtype, int64_t m, int64_t lda,
                     const fp4_tensor* w, void* c, int32_t c_dtype, int64_t ldc,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_w4aX_impl(act, a, a_dtype, m, lda, w, c, c_dtype, ldc, workspace, workspace_bytes, stream, false);
}

fp4_status gemm_w4aX_noalloc(int32_t act, const void* a, int32_t a_dtype, int64_t m, int64_t lda,
                             const fp4_tensor* w, void* c, int32_t c_dtype, int64_t ldc, void* stream) {
  return gemm_w4aX_impl(act, a, a_dtype, m, lda, w, c, c_dtype, ldc, nullptr, 0, stream, true);
}

fp4_status gemm_w4aX_static(int32_t act, const void* a, int32_t a_dtype, int64_t m, int64_t lda,
                            const uint16_t* act_macro, const fp4_tensor* w, void* c, int32_t c_dtype,
                            int64_t ldc, void* workspace, size_t workspace_bytes, void* stream) {
  if (act != FP4_A4 && act != FP4_A8) return FP4_E_MODE;
  if (!a || !c || !act_macro) return FP4_E_NULL;
  const fp4_status ws_ok = check_weights(w);
  if (ws_ok != FP4_OK) return ws_ok;
  if (!valid_dtype(a_dtype) || !valid_dtype(c_dtype)) return FP4_E_DTYPE;
  const int64_t n = w->rows, k = w->k;
  if (m < 1 || lda < k || ldc < n || ldc > FP4_MAX_LDC) return FP4_E_SHAPE;
  const fp4_status lim = check_product(act, m, m, n, k, false, 0, false);
  if (lim != FP4_OK) return lim;
  if (!aligned16(a) || (lda * (int64_t)dtype_size(a_dtype)) % 16) return FP4_E_ALIGN;
  if (!aligned(c, dtype_size(c_dtype)) || !aligned(act_macro, 2)) return FP4_E_ALIGN;
  const size_t need = act_workspace(act, m, k);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return FP4_E_WORKSPACE;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  hipStream_t st = static_cast<hipStream_t>(stream);
  fp4lib::GemmArgs g{};
  const fp4_status prep = prepare_activations(act, a, a_dtype, m, k, lda, workspace, g, st, act_macro);
  if (prep != FP4_OK) return prep;
  g.m = m;
  g.n = n;
  g.k = k;
  g.codes = static_cast<const uint8_t*>(w->codes);
  g.micro = w->micro;
  g.macro = w->macro;
  g.c = c;
  g.c_is_bf16 = c_dtype == FP4_BF16;
  g.ldc = ldc;
  return launched(fp4lib::launch_gemm(g, st));
}

fp4_status gemm_w8a8(const void* a, int32_t a_dtype, int64_t m, int64_t lda, const fp4_tensor* w, void* c,
                     int32_t c_dtype, int64_t ldc, void* workspace, size_t workspace_bytes, void* stream) {
  if (!a || !c) return FP4_E_NULL;
  const fp4_status ws_ok = check_weights(w, FP4_ELEM_E4M3);
  if (ws_ok != FP4_OK) return ws_ok;
  if (!valid_dtype(a_dtype) || !valid_dtype(c_dtype)) return FP4_E_DTYPE;
  const int64_t n = w->rows, k = w->k;
  if (m < 1 || lda < k || ldc < n || ldc > FP4_MAX_LDC) return FP4_E_SHAPE;
  const fp4_status lim = check_product(FP4_A8, m, m, n, k, false, 0, true);
  if (lim != FP4_OK) return lim;
  if (!aligned16(a) || (lda * (int64_t)dtype_size(a_dtype)) % 16) return FP4_E_ALIGN;
  if (!aligned(c, dtype_size(c_dtype))) return FP4_E_ALIGN;
  const size_t need = act_workspace(FP4_A8, m, k);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return FP4_E_WORKSPACE;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  hipStream_t st = static_cast<hipStream_t>(stream);
  fp4lib::GemmArgs g{};
  const fp4_status prep = prepare_activations(FP4_A8, a, a_dtype, m, k, lda, workspace, g, st);
  if (prep != FP4_OK) return prep;
  g.m = m;
  g.n = n;
  g.k = k;
  g.codes = static_cast<const uint8_t*>(w->codes);
  g.micro = w->micro;
  g.macro = w->macro;
  g.c = c;
  g.c_is_bf16 = c_dtype == FP4_BF16;
  g.ldc = ldc;
  g.w_e4m3 = 1;
  return launched(fp4lib::launch_gemm(g, st));
}

fp4_status grouped_gemm_w4aX(int32_t act, const void* a, int32_t a_dtype, int64_t a_rows,
                             int64_t lda, const int32_t* row_token,
                             const int32_t* expert_offsets, int32_t n_experts,
                             int64_t total_rows, const fp4_tensor* w, void* c,
                             int32_t c_dtype, int64_t ldc, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!valid_act(act)) return FP4_E_MODE;
  if (!a || !c || !expert_offsets) return FP4_E_NULL;
  const fp4_status ws_ok = check_weights(w);
  if (ws_ok != FP4_OK) return ws_ok;
  if (!valid_dtype(a_dtype) || !valid_dtype(c_dtype)) return FP4_E_DTYPE;
  if (act == FP4_A16 && a_dtype != FP4_BF16) return FP4_E_DTYPE;
  if (n_experts < 1 || w->rows % n_experts) return FP4_E_SHAPE;
  const int64_t n = w->rows / n_experts, k = w->k;
  if (n % 16 || a_rows < 1 || total_rows < 0 || lda < k || ldc < n || ldc > FP4_MAX_LDC) return FP4_E_SHAPE;
  if (!row_token && total_rows > a_rows) return FP4_E_SHAPE;
  // gathered rows are addressed with 32-bit byte offsets from the start of the operand
  // (bf16 A for W4A16, the FP16 activation workspace otherwise: both 2 bytes/element)
  if (row_token && a_rows * (act == FP4_A16 ? lda : k) * 2 > (int64_t)0xFFFFFFFF) return FP4_E_SHAPE;
  if (!aligned16(a) || (lda * (int64_t)dtype_size(a_dtype)) % 16) return FP4_E_ALIGN;
  if (!aligned(c, dtype_size(c_dtype)) || !aligned(expert_offsets, 4) ||
      (row_token && !aligned(row_token, 4)))
    return FP4_E_ALIGN;
  const size_t need = act_workspace(act, a_rows, k);
  if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return FP4_E_WORKSPACE;
  if (total_rows > 0) {
    const fp4_status lim = check_product(act, a_rows, total_rows, n, k, true, n_experts, false);
    if (lim != FP4_OK) return lim;
  }
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  if (total_rows == 0) return FP4_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  fp4lib::GemmArgs g{};
  const fp4_status prep = prepare_activations(act, a, a_dtype, a_rows, k, lda, workspace, g, st);
  if (prep != FP4_OK) return prep;
  g.m = total_rows;
  g.n = n;
  g.k = k;
  g.codes = static_cast<const uint8_t*>(w->codes);
  g.micro = w->micro;
  g.macro = w->macro;
  g.c = c;
  g.c_is_bf16 = c_dtype == FP4_BF16;
  g.ldc = ldc;
  g.row_token = row_token;
  g.expert_offsets = expert_offsets;
  g.n_experts = n_experts;
  return launched(fp4lib::launch_gemm(g, st));
}

fp4_status grouped_gemm_w4aX_gated(int32_t act, const void* gate_up, int64_t rows, int64_t ld,
                                   const int32_t* expert_offsets, int32_t n_experts,
                                   const fp4_tensor* w, void* c, int32_t c_dtype, int64_t ldc,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_act(act)) return FP4_E_MODE;
  if (act == FP4_A16) return FP4_E_DTYPE;  // the gated operand only exists quantized
  if (!gate_up || !c || !expert_offsets) return FP4_E_NULL;
  const fp4_status ws_ok = check_weights(w);
  if (ws_ok != FP4_OK) return ws_ok;
  if (!valid_dtype(c_dtype)) return FP4_E_DTYPE;
  if (n_experts < 1 || w->rows % n_experts) return FP4_E_SHAPE;
  const int64_t n = w->rows / n_experts, k = w->k;
  if (n % 16 || rows < 0 || ld < 2 * k || ldc < n || ldc > FP4_MAX_LDC) return FP4_E_SHAPE;
  if (!aligned16(gate_up) || (ld * 2) % 16) return FP4_E_ALIGN;
  if (!aligned(c, dtype_size(c_dtype)) || !aligned(expert_offsets, 4)) return FP4_E_ALIGN;
  const size_t need = act_workspace(act, rows, k);
  if (rows > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return FP4_E_WORKSPACE;
  if (rows > 0) {
    const fp4_status lim = check_product(act, rows, rows, n, k, true, n_experts, false);
    if (lim != FP4_OK) return lim;
  }
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  if (rows == 0) return FP4_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t ldq = act_ws_stride(k);
  _Float16* aq = static_cast<_Float16*>(workspace);
  float* scale = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                          (((size_t)rows * (size_t)ldq * 2 + 255) & ~(size_t)255));
  if (fp4lib::launch_act_prep_gated(static_cast<const uint16_t*>(gate_up), rows, k, ld, act == FP4_A8,
                                    aq, ldq, scale, st) != hipSuccess)
    return FP4_E_HIP;
  fp4lib::GemmArgs g{};
  g.a = aq;
  g.a_is_bf16 = 0;
  g.lda = ldq;
  g.a_scale = scale;
  g.m = rows;
  g.n = n;
  g.k = k;
  g.codes = static_cast<const uint8_t*>(w->codes);
  g.micro = w->micro;
  g.macro = w->macro;
  g.c = c;
  g.c_is_bf16 = c_dtype == FP4_BF16;
  g.ldc = ldc;
  g.row_token = nullptr;
  g.expert_offsets = expert_offsets;
  g.n_experts = n_experts;
  return launched(fp4lib::launch_gemm(g, st));
}

size_t moe_route_workspace_bytes(int64_t tokens, int32_t n_experts) {
  return n_experts < 1 || tokens < 0 ? 0 : fp4lib::route_workspace_bytes(tokens, n_experts);
}

fp4_status moe_route(const float* logits, int64_t tokens, int32_t n_experts, int32_t top_k,
                     int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                     int32_t* row_token, int32_t* token_rows, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!logits || !topk_ids || !topk_weights || !expert_offsets || !row_token || !token_rows)
    return FP4_E_NULL;
  if (tokens < 1 || tokens * (int64_t)top_k > 0x7FFFFFFF || !fp4lib::route_supports(n_experts, top_k))
    return FP4_E_SHAPE;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(expert_offsets, 4) || !aligned(row_token, 4) || !aligned(token_rows, 4))
    return FP4_E_ALIGN;
  if (!workspace || workspace_bytes < moe_route_workspace_bytes(tokens, n_experts) ||
      !aligned(workspace, 256))
    return FP4_E_WORKSPACE;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_moe_route(logits, tokens, n_experts, top_k, topk_ids, topk_weights,
                                           expert_offsets, row_token, token_rows, workspace,
                                           static_cast<hipStream_t>(stream)));
}

fp4_status moe_combine(const void* y, int32_t y_dtype, int64_t ldy, const int32_t* token_rows,
                       const float* topk_weights, int64_t tokens, int32_t top_k, int64_t hidden,
                       void* out, int32_t out_dtype, int64_t ldo, void* stream) {
  if (!y || !token_rows || !topk_weights || !out) return FP4_E_NULL;
  if (!valid_dtype(y_dtype) || !valid_dtype(out_dtype)) return FP4_E_DTYPE;
  if (tokens < 1 || tokens > 0x7FFFFFFF || top_k < 1 || hidden < 8 || hidden % 8 || ldy < hidden ||
      ldo < hidden)
    return FP4_E_SHAPE;
  if (!aligned16(y) || (ldy * (int64_t)dtype_size(y_dtype)) % 16 || !aligned16(out) ||
      (ldo * (int64_t)dtype_size(out_dtype)) % 16 || !aligned(token_rows, 4) || !aligned(topk_weights, 4))
    return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_moe_combine(y, y_dtype == FP4_BF16, ldy, token_rows, topk_weights,
                                             tokens, top_k, hidden, out, out_dtype == FP4_BF16, ldo,
                                             static_cast<hipStream_t>(stream)));
}

// ---- MX-native FP4 ----

size_t mxfp4_bytes(int64_t rows, int64_t k, int32_t part) {
  if (rows < 1 || k < 128 || k % 128) return 0;
  const size_t padded = (size_t)fp4lib::mx_padded_rows(rows);
  if (part == FP4_MX_CODES) return padded * (size_t)k / 2;
  if (part == FP4_MX_SCALES) return padded * (size_t)k / 32;
  return 0;
}

fp4_status quantize_mxfp4(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx, void* codes,
                          uint8_t* scales, void* stream) {
  if (!x || !codes || !scales) return FP4_E_NULL;
  if (!valid_dtype(x_dtype)) return FP4_E_DTYPE;
  if (rows < 1 || k < 128 || k % 128 || ldx < k) return FP4_E_SHAPE;
  // one thread per 32-element block (rows padded to 16), 256 per workgroup
  if (fp4lib::mx_padded_rows(rows) > (int64_t)0x7FFFFFFF * 256 / (k / 32)) return FP4_E_SHAPE;
  if (!aligned16(x) || (ldx * (int64_t)dtype_size(x_dtype)) % 16 || !aligned16(codes)) return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_mx_quantize(x, x_dtype == FP4_BF16, rows, k, ldx, static_cast<uint8_t*>(codes),
                                             scales, static_cast<hipStream_t>(stream)));
}

fp4_status gemm_mxfp4(const void* a_codes, const uint8_t* a_scales, int64_t m, const void* w_codes,
                      const uint8_t* w_scales, int64_t n, int64_t k, void* c, int32_t c_dtype, int64_t ldc,
                      void* stream) {
  if (!a_codes || !a_scales || !w_codes || !w_scales || !c) return FP4_E_NULL;
  if (!valid_dtype(c_dtype)) return FP4_E_DTYPE;
  if (m < 1 || n < 1 || k < 128 || k % 128 || ldc < n || ldc > FP4_MAX_LDC || (m + 127) / 128 > 65535 ||
      (n + 127) / 128 > 0x7FFFFFFF)
    return FP4_E_SHAPE;
  if (!aligned16(a_codes) || !aligned16(w_codes) || !aligned(c, dtype_size(c_dtype))) return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_gemm_mx(static_cast<const uint8_t*>(a_codes), a_scales, m,
                                         static_cast<const uint8_t*>(w_codes), w_scales, n, k, c,
                                         c_dtype == FP4_BF16, ldc, static_cast<hipStream_t>(stream)));
}

// ---- KV cache and decode attention ----

namespace {
fp4_status check_kv_cache(const fp4_kv_cache* c) {
  if (!c || !c->k_codes || !c->k_micro || !c->k_macro || !c->v_codes || !c->v_micro || !c->v_macro)
    return FP4_E_NULL;
  // per (sequence, head) arrays stay under 2^31 bytes (32-bit buffer offsets)
  if (c->n_seq < 1 || c->n_seq > 65535 || c->max_tokens > (1 << 24) ||
      !fp4lib::kv_cache_supports(c->max_tokens, c->kv_heads, c->head_dim))
    return FP4_E_SHAPE;
  if (!aligned16(c->k_codes) || !aligned16(c->v_codes) || !aligned(c->k_micro, 8) ||
      !aligned(c->v_micro, 8) || !aligned(c->k_macro, 8) || !aligned(c->v_macro, 8))
    return FP4_E_ALIGN;
  return FP4_OK;
}
fp4lib::KvCacheArgs kv_args(const fp4_kv_cache* c) {
  fp4lib::KvCacheArgs a;
  a.k_codes = static_cast<uint8_t*>(c->k_codes);
  a.k_micro = c->k_micro;
  a.k_macro = c->k_macro;
  a.v_codes = static_cast<uint8_t*>(c->v_codes);
  a.v_micro = c->v_micro;
  a.v_macro = c->v_macro;
  a.n_seq = c->n_seq;
  a.max_tokens = c->max_tokens;
  a.kv_heads = c->kv_heads;
  return a;
}
}  // namespace

size_t fp4_kv_cache_bytes(int32_t n_seq, int32_t max_tokens, int32_t kv_heads, int32_t head_dim,
                          int32_t part) {
  if (n_seq < 1 || !fp4lib::kv_cache_supports(max_tokens, kv_heads, head_dim)) return 0;
  const size_t tokens = (size_t)n_seq * (size_t)kv_heads * (size_t)max_tokens;
  switch (part) {
    case FP4_KV_CODES: return tokens * (size_t)head_dim / 2;
    case FP4_KV_MICRO: return tokens * (size_t)head_dim / 16;
    case FP4_KV_MACRO: return tokens / 2 * sizeof(uint16_t);
    default: return 0;
  }
}

fp4_status kv_cache_append(const fp4_kv_cache* cache, const void* k_new, const void* v_new,
                           int32_t dtype, int64_t ld, const int32_t* positions, int32_t n_new,
                           void* stream) {
  const fp4_status cs = check_kv_cache(cache);
  if (cs != FP4_OK) return cs;
  if (!k_new || !v_new || !positions) return FP4_E_NULL;
  if (!valid_dtype(dtype)) return FP4_E_DTYPE;
  if (n_new < 1 || n_new > (1 << 20) || ld < (int64_t)cache->kv_heads * cache->head_dim) return FP4_E_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || (ld * (int64_t)dtype_size(dtype)) % 16 ||
      !aligned(positions, 4))
    return FP4_E_ALIGN;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_kv_append(kv_args(cache), k_new, v_new, dtype == FP4_BF16, ld, positions,
                                           n_new, static_cast<hipStream_t>(stream)));
}

size_t attention_workspace_bytes(int32_t n_seq, int32_t q_heads, int32_t max_tokens) {
  if (n_seq < 1 || q_heads < 1 || max_tokens < 1) return 0;
  return fp4lib::attention_partial_bytes(n_seq, q_heads, max_tokens);
}

fp4_status attention_decode_fp4kv(const void* q, int32_t q_heads, const fp4_kv_cache* cache,
                                  const int32_t* lengths, float scale, void* out, int32_t out_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const fp4_status cs = check_kv_cache(cache);
  if (cs != FP4_OK) return cs;
  if (!q || !lengths || !out) return FP4_E_NULL;
  if (!valid_dtype(out_dtype)) return FP4_E_DTYPE;
  if (q_heads < 1 || q_heads % cache->kv_heads || q_heads / cache->kv_heads > 16) return FP4_E_SHAPE;
  if (!aligned16(q) || !aligned(lengths, 4) || !aligned(out, dtype_size(out_dtype))) return FP4_E_ALIGN;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < attention_workspace_bytes(cache->n_seq, q_heads, cache->max_tokens))
    return FP4_E_WORKSPACE;
  const fp4_status dev = check_device();
  if (dev != FP4_OK) return dev;
  return launched(fp4lib::launch_attention_decode(kv_args(cache), static_cast<const uint16_t*>(q), q_heads,
                                                  lengths, scale, static_cast<float*>(workspace), out,
                                                  out_dtype == FP4_BF16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
