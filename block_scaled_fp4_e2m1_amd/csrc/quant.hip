// Two-level block-scaled quantization kernels for gfx950: quantize (E2M1 or E4M3
// elements; canonical or tiled output), dequantize, and the activation pass that feeds
// the matrix kernels.
//
// Work mapping (quantize and the activation pass): 16 lanes own one 256-element group of
// one row, one 16-element micro-vector per lane (two 16-byte loads for bf16, four for
// float32), so the block max is lane-local and the group max is four cross-lane
// exchanges; the per-lane scale arithmetic (two correctly rounded divisions and two
// round-to-nearest-even conversions) is amortized over 16 elements. The segments cover
// the (row, group) pairs of the input in row-major order.
// Dequantize keeps 32 lanes per group (8 elements per lane, 8 groups per block).
// Source of the method: "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for
// Blackwell B200", section "The Mathematical Breakthrough of Microscopic FP4 Scaling".
#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;

namespace {


// Grid mappings. Quantize and the activation pass: 16 lanes per 256-group; a block of 256
// threads covers 16 consecutive (row, group) pairs of the row-major order
// f = row * groups + group, so blocks stay full whatever the number of groups per row (a
// block per row would leave most lanes idle for k = 768). (A capped grid walking the
// pairs with the next pair's input in flight measured slower at every cap tried.)
// Dequantize: 32 lanes per group, block b is row b / gchunks, groups
// (b % gchunks) * 8 + 0..7, with gchunks = ceil(groups / 8).
__device__ __forceinline__ bool seg_index16(int64_t rows, int64_t groups, int64_t& r, int64_t& g) {
  const uint32_t f = blockIdx.x * 16u + (threadIdx.x >> 4);  // < 2^28: see blocks_for16
  if ((int64_t)f >= rows * groups) return false;
  const uint32_t row = f / (uint32_t)groups;
  r = row;
  g = (int64_t)(f - row * (uint32_t)groups);
  return true;
}
__device__ __forceinline__ bool seg_index(int64_t groups, int64_t& r, int64_t& g) {
  const uint32_t gchunks = (uint32_t)((groups + 7) >> 3);
  const uint32_t b = blockIdx.x;
  const uint32_t row = b / gchunks;
  r = row;
  g = (int64_t)(b - row * gchunks) * 8 + (threadIdx.x >> 5);
  return g < groups;
}

// Encodes one micro-vector (v, 16 elements of row r at column col) and stores its codes,
// micro-scale and (lane 0 of the group) macro-scale.
template <int ELEM_E4M3, int TILED>
__device__ __forceinline__ void quantize_item(const float v[16], int64_t r, int64_t g, int li,
                                              int64_t k, int64_t groups, uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ micro, uint16_t* __restrict__ macro) {
  const int64_t col = g * kGroup + li * 16;
  uint32_t m_bits, mu_byte;
  float m_val;
  const float s = block_scales(v, ELEM_E4M3 ? 448.0f : 6.0f, m_bits, mu_byte, m_val);

  if (!ELEM_E4M3) {
    uint32_t w0, w1;
    e2m1_encode16(v, s, w0, w1);
    if (TILED) {
      *reinterpret_cast<uint32_t*>(codes + tiled_code_offset(r, col, groups)) = w0;
      *reinterpret_cast<uint32_t*>(codes + tiled_code_offset(r, col + 8, groups)) = w1;
    } else {
      *reinterpret_cast<uint2*>(codes + r * (k >> 1) + (col >> 1)) = make_uint2(w0, w1);
    }
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (s > 0.0f) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        w[i >> 2] |= (e4m3_rne_pos(fabsf(v[i]) / s) | (sign_of(v[i]) << 7)) << (8 * (i & 3));
    }
    *reinterpret_cast<uint4*>(codes + r * k + col) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  {
    const int64_t off = TILED ? tiled_micro_offset(r, col, groups) : r * (k >> 4) + (col >> 4);
    micro[off] = (uint8_t)mu_byte;
  }
  if (li == 0) {
    const int64_t off = TILED ? tiled_macro_offset(r, col, groups) : r * groups + g;
    macro[off] = (uint16_t)m_bits;
  }
}

template <int IN_BF16, int ELEM_E4M3, int TILED>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t ldx,
                                                  int64_t rows, int64_t k,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ micro,
                                                  uint16_t* __restrict__ macro) {
  const int64_t groups = k >> 8;
  const int li = threadIdx.x & 15;  // micro-vector of the group
  int64_t r, g;
  if (!seg_index16(rows, groups, r, g)) return;  // whole 16-lane segments leave together
  Raw16<IN_BF16> raw;
  load_raw16<IN_BF16>(x, r * ldx + g * kGroup + li * 16, raw);
  float v[16];
  unpack16<IN_BF16>(raw, v);
  quantize_item<ELEM_E4M3, TILED>(v, r, g, li, k, groups, codes, micro, macro);
}

template <int OUT_BF16, int ELEM_E4M3, int TILED>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ micro,
                                                    const uint16_t* __restrict__ macro,
                                                    int64_t rows, int64_t k, void* __restrict__ y,
                                                    int64_t ldy) {
  const int64_t groups = k >> 8;
  const int li = threadIdx.x & 31;
  int64_t r, g;
  if (!seg_index(groups, r, g)) return;  // whole 32-lane segments leave together
  const int64_t col = g * kGroup + li * 8;

  const int64_t mu_off = TILED ? tiled_micro_offset(r, col, groups) : r * (k >> 4) + (col >> 4);
  const int64_t m_off = TILED ? tiled_macro_offset(r, col, groups) : r * groups + g;
  const float scale = e4m3_value(micro[mu_off]) * fp16_value(macro[m_off]);  // exact
  float v[8];
  if (!ELEM_E4M3) {
    const int64_t off = TILED ? tiled_code_offset(r, col, groups) : r * (k >> 1) + (col >> 1);
    const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (word >> (4 * i)) & 15u;
      const float mag = e2m1_mag_value(c & 7u) * scale;
      v[i] = (c & 8u) ? -mag : mag;
    }
  } else {
    const uint2 p = *reinterpret_cast<const uint2*>(codes + r * k + col);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = ((i < 4 ? p.x : p.y) >> (8 * (i & 3))) & 0xFFu;
      v[i] = e4m3_value(b) * scale;
    }
  }
  if (OUT_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_rne_bits(v[2 * i]) | (bf16_rne_bits(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + r * ldy + col) =
        make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(y) + r * ldy + col);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Activation pass for the matrix kernels. Quantizes each row like k_quantize and writes
// the *decoded* element times its micro-scale as FP16 (exact: E2M1 * mu has at most 6
// significant bits in [2^-10, 2688]; E4M3 * mu * 2^-3 at most 8 bits in [2^-21, 25088]),
// plus one float32 factor per 256-group (M, or 8*M for E4M3 elements; 1 for an all-zero
// group), so that
//   A_hat[r, c] = aq[r, c] * scale[r, c / 256]   exactly.
// GATED: the row of a holds gate in columns [0, k) and up in [k, 2k) (bf16); the operand
// is h = bf16(silu(gate) * up), silu(x) = x / (1 + exp(-x)) in float32 (hardware exp and
// reciprocal approximations), quantized as
// above (the SiLU-gated activation between a mixture-of-experts layer's gate/up and down
// products, fused with the down product's dynamic quantization).
// Encodes one micro-vector of the activation pass (v, 16 elements of row r at column col)
// into the FP16 operand and, from lane 0 of the group, the group factor.
template <int ELEM_E4M3>
__device__ __forceinline__ void act_item(float v[16], int64_t r, int64_t g, int li, int64_t groups,
                                         _Float16* __restrict__ aq, int64_t ldq,
                                         float* __restrict__ scale) {
  const int64_t col = g * kGroup + li * 16;
  uint32_t m_bits, mu_byte;
  float m_val;
  const float s = block_scales(v, ELEM_E4M3 ? 448.0f : 6.0f, m_bits, mu_byte, m_val);
  const float mu = e4m3_value(mu_byte);
  half2_t out[8];
  if (!ELEM_E4M3) {
    // codes as in k_quantize, then decoded two at a time by the hardware conversion
    // (scale 1: exact) and multiplied by mu in FP16 (E2M1 * mu is exact in FP16)
    uint32_t w0, w1;
    e2m1_encode16(v, s, w0, w1);
    const _Float16 muh = (_Float16)mu;
    const half2_t m2 = {muh, muh};
    out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0) * m2;
    out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1) * m2;
    out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) * m2;
    out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) * m2;
    out[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0) * m2;
    out[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1) * m2;
    out[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2) * m2;
    out[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3) * m2;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = s > 0.0f ? e4m3_value(e4m3_rne_pos(fabsf(v[i]) / s)) : 0.0f;
      const float mag = e * mu * 0.125f;
      const _Float16 h = (_Float16)(sign_of(v[i]) ? -mag : mag);
      if (i & 1) out[i >> 1][1] = h; else out[i >> 1][0] = h;
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(aq + r * ldq + col);
  dst[0] = make_uint4(__builtin_bit_cast(uint32_t, out[0]), __builtin_bit_cast(uint32_t, out[1]),
                      __builtin_bit_cast(uint32_t, out[2]), __builtin_bit_cast(uint32_t, out[3]));
  dst[1] = make_uint4(__builtin_bit_cast(uint32_t, out[4]), __builtin_bit_cast(uint32_t, out[5]),
                      __builtin_bit_cast(uint32_t, out[6]), __builtin_bit_cast(uint32_t, out[7]));
  // a group whose macro-scale is 0 has only zero operands: its factor is written as 1, so
  // the product kernel's factor ratios never divide by zero
  if (li == 0) scale[r * groups + g] = m_val > 0.0f ? (ELEM_E4M3 ? m_val * 8.0f : m_val) : 1.0f;
}

template <int IN_BF16, int ELEM_E4M3, int GATED>
__global__ __launch_bounds__(256) void k_act_prep(const void* __restrict__ a, int64_t lda,
                                                  int64_t rows, int64_t k,
                                                  _Float16* __restrict__ aq, int64_t ldq,
                                                  float* __restrict__ scale) {
  const int64_t groups = k >> 8;
  const int li = threadIdx.x & 15;
  int64_t r, g;
  if (!seg_index16(rows, groups, r, g)) return;
  Raw16<IN_BF16> raw;
  load_raw16<IN_BF16>(a, r * lda + g * kGroup + li * 16, raw);
  float v[16];
  unpack16<IN_BF16>(raw, v);
  if (GATED) {
    // h = bf16(silu(gate) * up); exp and reciprocal by the hardware approximations (a few
    // float32 ulp, far below the bf16 step h is rounded to)
    Raw16<IN_BF16> raw_up;
    load_raw16<IN_BF16>(a, r * lda + k + g * kGroup + li * 16, raw_up);
    float up[16];
    unpack16<IN_BF16>(raw_up, up);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float h = v[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-v[i])) * up[i];
      v[i] = __uint_as_float(bf16_rne_bits(h) << 16);
    }
  }
  act_item<ELEM_E4M3>(v, r, g, li, groups, aq, ldq, scale);
}

// one block per 16 (row, group) pairs; 0 when the grid would exceed 2^32 work-items (the
// launchers then refuse the shape).
inline unsigned blocks_for16(int64_t rows, int64_t k) {
  const int64_t blocks = (rows * (k >> 8) + 15) >> 4;
  return blocks <= (int64_t)0xFFFFFFFF / 256 ? (unsigned)blocks : 0u;
}

// one block per (row, run of 8 groups); see seg_index. 0 when the grid would exceed
// 2^32 work-items (the launchers then refuse the shape).
inline unsigned blocks_for(int64_t rows, int64_t k) {
  const int64_t blocks = rows * (((k >> 8) + 7) >> 3);
  return blocks <= (int64_t)0xFFFFFFFF / 256 ? (unsigned)blocks : 0u;
}

}  // namespace

namespace fp4lib {

hipError_t launch_quantize(const void* x, int in_bf16, int64_t rows, int64_t k, int64_t ldx,
                           int elem_e4m3, int tiled, uint8_t* codes, uint8_t* micro,
                           uint16_t* macro, hipStream_t st) {
  const dim3 grid(blocks_for16(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
#define FP4_Q(B, E, T) \
  hipLaunchKernelGGL((k_quantize<B, E, T>), grid, block, 0, st, x, ldx, rows, k, codes, micro, macro)
  if (in_bf16) {
    if (elem_e4m3) FP4_Q(1, 1, 0); else if (tiled) FP4_Q(1, 0, 1); else FP4_Q(1, 0, 0);
  } else {
    if (elem_e4m3) FP4_Q(0, 1, 0); else if (tiled) FP4_Q(0, 0, 1); else FP4_Q(0, 0, 0);
  }
#undef FP4_Q
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                             int64_t rows, int64_t k, int elem_e4m3, int tiled, void* y,
                             int out_bf16, int64_t ldy, hipStream_t st) {
  const dim3 grid(blocks_for(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
#define FP4_D(B, E, T) \
  hipLaunchKernelGGL((k_dequantize<B, E, T>), grid, block, 0, st, codes, micro, macro, rows, k, y, ldy)
  if (out_bf16) {
    if (elem_e4m3) FP4_D(1, 1, 0); else if (tiled) FP4_D(1, 0, 1); else FP4_D(1, 0, 0);
  } else {
    if (elem_e4m3) FP4_D(0, 1, 0); else if (tiled) FP4_D(0, 0, 1); else FP4_D(0, 0, 0);
  }
#undef FP4_D
  return hipGetLastError();
}

hipError_t launch_act_prep(const void* a, int in_bf16, int64_t rows, int64_t k, int64_t lda,
                           int elem_e4m3, _Float16* aq, int64_t ldq, float* scale, hipStream_t st) {
  const dim3 grid(blocks_for16(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
#define FP4_ACT(B, E, G) hipLaunchKernelGGL((k_act_prep<B, E, G>), grid, block, 0, st, a, lda, rows, k, aq, ldq, scale)
  if (in_bf16) { if (elem_e4m3) FP4_ACT(1, 1, 0); else FP4_ACT(1, 0, 0); }
  else { if (elem_e4m3) FP4_ACT(0, 1, 0); else FP4_ACT(0, 0, 0); }
  return hipGetLastError();
}

hipError_t launch_act_prep_gated(const uint16_t* a, int64_t rows, int64_t k, int64_t lda, int elem_e4m3,
                                 _Float16* aq, int64_t ldq, float* scale, hipStream_t st) {
  const dim3 grid(blocks_for16(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
  if (elem_e4m3) FP4_ACT(1, 1, 1); else FP4_ACT(1, 0, 1);
#undef FP4_ACT
  return hipGetLastError();
}

}  // namespace fp4lib
