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
// TILE_ORDER (tiled output, rows % 16 == 0): the 16 segments of a workgroup are the 16 rows
// of one tile (one group of one 16-row block), so the workgroup writes the tile's 2 KB of
// codes, micro- and macro-scales whole; in row order a workgroup wrote one row's piece of
// 16 tiles in scattered 4-byte stores, and partly written lines left the L2 as partial
// writes (2.4x the bytes).
template <int TILE_ORDER = 0>
__device__ __forceinline__ bool seg_index16(int64_t rows, int64_t groups, int64_t& r, int64_t& g) {
  const uint32_t f = blockIdx.x * 16u + (threadIdx.x >> 4);  // < 2^28: see blocks_for16
  if ((int64_t)f >= rows * groups) return false;
  if (TILE_ORDER) {
    const uint32_t tile = f >> 4, rb = tile / (uint32_t)groups;
    r = (int64_t)rb * 16 + (f & 15u);
    g = (int64_t)(tile - rb * (uint32_t)groups);
    return true;
  }
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

// Scales of a lane that owns one micro-vector when the macro-scale is given (static
// activation scales, calibrated beforehand): mu = RNE_e4m3(amax_16 / (emax * M)), which
// saturates at 448 for blocks beyond the calibrated range; M = 0 gives mu = 0.
__device__ __forceinline__ float static_block_scales(const float v[16], float emax, uint32_t m_in,
                                                     uint32_t& m_bits, uint32_t& mu_byte, float& m_val) {
  float amax_b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));
  m_bits = m_in & 0xFFFFu;
  m_val = fp16_value(m_bits);
  mu_byte = m_val > 0.0f ? e4m3_rne_pos(amax_b / (emax * m_val)) : 0u;
  return e4m3_value(mu_byte) * m_val;
}

template <int ELEM_E4M3, int STATIC>
__device__ __forceinline__ float item_scales(const float v[16], int64_t g, const uint16_t* __restrict__ macro_in,
                                             uint32_t& m_bits, uint32_t& mu_byte, float& m_val) {
  const float emax = ELEM_E4M3 ? 448.0f : 6.0f;
  if (STATIC) return static_block_scales(v, emax, macro_in[g], m_bits, mu_byte, m_val);
  return block_scales(v, emax, m_bits, mu_byte, m_val);
}

// Encodes one micro-vector (v, 16 elements of row r at column col) and stores its codes,
// micro-scale and (lane 0 of the group) macro-scale. STATIC: the macro-scale of group g is
// macro_in[g] (shared by every row) instead of the group's own.
template <int ELEM_E4M3, int TILED, int STATIC>
__device__ __forceinline__ void quantize_item(const float v[16], int64_t r, int64_t g, int li,
                                              int64_t k, int64_t groups, uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ micro, uint16_t* __restrict__ macro,
                                              const uint16_t* __restrict__ macro_in) {
  const int64_t col = g * kGroup + li * 16;
  uint32_t m_bits, mu_byte;
  float m_val;
  const float s = item_scales<ELEM_E4M3, STATIC>(v, g, macro_in, m_bits, mu_byte, m_val);

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
    if (TILED) {
      *reinterpret_cast<uint2*>(codes + tiled8_code_offset(r, col, groups)) = make_uint2(w[0], w[1]);
      *reinterpret_cast<uint2*>(codes + tiled8_code_offset(r, col + 8, groups)) = make_uint2(w[2], w[3]);
    } else {
      *reinterpret_cast<uint4*>(codes + r * k + col) = make_uint4(w[0], w[1], w[2], w[3]);
    }
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

template <int IN_BF16, int ELEM_E4M3, int TILED, int STATIC>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t ldx,
                                                  int64_t rows, int64_t k,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ micro,
                                                  uint16_t* __restrict__ macro,
                                                  const uint16_t* __restrict__ macro_in) {
  const int64_t groups = k >> 8;
  const int li = threadIdx.x & 15;  // micro-vector of the group
  int64_t r, g;
  if (!seg_index16<TILED>(rows, groups, r, g)) return;  // whole 16-lane segments leave together
  Raw16<IN_BF16> raw;
  load_raw16<IN_BF16>(x, r * ldx + g * kGroup + li * 16, raw);
  float v[16];
  unpack16<IN_BF16>(raw, v);
  quantize_item<ELEM_E4M3, TILED, STATIC>(v, r, g, li, k, groups, codes, micro, macro, macro_in);
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
    const int64_t off = TILED ? tiled8_code_offset(r, col, groups) : r * k + col;
    const uint2 p = *reinterpret_cast<const uint2*>(codes + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = ((i < 4 ? p.x : p.y) >> (8 * (i & 3))) & 0xFFu;
      v[i] = e4m3_value(b) * scale;
    }
  }
  if (OUT_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16x2_rne(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + r * ldy + col) =
        make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(y) + r * ldy + col);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Tiled E2M1 weights to bf16 / float32, one 16 x 256 tile per wave. The tile's code bytes
// arrive as two coalesced 1 KB loads: lane 16 j + n then holds row n's codes at columns
// 32 t + 8 j .. + 7 (t = 0..7; its four dwords of the first half, then of the second). Its
// micro-scales (blocks 2 t + j / 2 of row n) are one 8-byte word, and the row's
// macro-scale one load. The lane writes eight runs of 8 columns of its row. Same arithmetic
// as k_dequantize (the element times mu * M, both exact in float32, then the output's
// rounding), so the same bits, without the scattered per-lane reads of the tiled layout.
template <int OUT_BF16>
__global__ __launch_bounds__(256) void k_dequantize_tiled(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ micro,
                                                          const uint16_t* __restrict__ macro, int64_t tiles,
                                                          int64_t groups, void* __restrict__ y, int64_t ldy) {
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= tiles) return;  // whole waves
  const int lane = threadIdx.x & 63, n = lane & 15, j = lane >> 4;
  const uint4 c0 = *reinterpret_cast<const uint4*>(codes + tile * kTileCodeBytes + lane * 16);
  const uint4 c1 = *reinterpret_cast<const uint4*>(codes + tile * kTileCodeBytes + 1024 + lane * 16);
  const uint2 mu = *reinterpret_cast<const uint2*>(micro + tile * kTileMicroBytes + (j >> 1) * 128 + n * 8);
  const float M = fp16_value(macro[tile * kTileMacro + n]);
  const int64_t r = (tile / groups) * 16 + n;
  const int64_t col0 = (tile % groups) * kGroup + 8 * j;
  const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float scale = e4m3_value(((t < 4 ? mu.x : mu.y) >> (8 * (t & 3))) & 0xFFu) * M;  // exact
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (cw[t] >> (4 * i)) & 15u;
      const float mag = e2m1_mag_value(c & 7u) * scale;
      v[i] = (c & 8u) ? -mag : mag;
    }
    const int64_t col = col0 + 32 * t;
    if (OUT_BF16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + r * ldy + col) =
          make_uint4(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]), bf16x2_rne(v[4], v[5]), bf16x2_rne(v[6], v[7]));
    } else {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(y) + r * ldy + col);
      p[0] = make_float4(v[0], v[1], v[2], v[3]);
      p[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
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
// STATIC: the macro-scale of group g is macro_in[g] for every row (calibrated activation
// scales); the factor written is then the same for all rows.
template <int ELEM_E4M3, int STATIC>
__device__ __forceinline__ void act_item(float v[16], int64_t r, int64_t g, int li, int64_t groups,
                                         _Float16* __restrict__ aq, int64_t ldq,
                                         float* __restrict__ scale, const uint16_t* __restrict__ macro_in) {
  const int64_t col = g * kGroup + li * 16;
  uint32_t m_bits, mu_byte;
  float m_val;
  const float s = item_scales<ELEM_E4M3, STATIC>(v, g, macro_in, m_bits, mu_byte, m_val);
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

template <int IN_BF16, int ELEM_E4M3, int GATED, int STATIC>
__global__ __launch_bounds__(256) void k_act_prep(const void* __restrict__ a, int64_t lda,
                                                  int64_t rows, int64_t k,
                                                  _Float16* __restrict__ aq, int64_t ldq,
                                                  float* __restrict__ scale,
                                                  const uint16_t* __restrict__ macro_in) {
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
  act_item<ELEM_E4M3, STATIC>(v, r, g, li, groups, aq, ldq, scale, macro_in);
}

// Calibration of static activation macro-scales. k_amax_update keeps a running maximum
// of |x| per 256-column group over every row it has seen: block (group g, runs of 64 rows
// strided by gridDim.y) reads 8 rows per pass, 32 lanes x 16 bytes per row; the block's
// maximum enters amax[g] by an atomic maximum on the float bits (non-negative floats
// order as their bit patterns, so the result does not depend on the order).
// k_macro_from_amax then applies the dynamic macro rule to that maximum.
constexpr int kCalRows = 64;

template <int IN_BF16>
__global__ __launch_bounds__(256) void k_amax_update(const void* __restrict__ x, int64_t ldx, int64_t rows,
                                                     float* __restrict__ amax) {
  const int64_t g = blockIdx.x;
  const int sub = threadIdx.x >> 5, li = threadIdx.x & 31;
  float m = 0.0f;
  for (int64_t r0 = (int64_t)blockIdx.y * kCalRows; r0 < rows; r0 += (int64_t)gridDim.y * kCalRows) {
    const int64_t r_end = min(r0 + kCalRows, rows);
    for (int64_t r = r0 + sub; r < r_end; r += 8) {
      const int64_t off = r * ldx + g * kGroup + li * 8;
      if (IN_BF16) {
        const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[j] << 16)), fabsf(__uint_as_float(w[j] & 0xFFFF0000u))));
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float4 f = p[j];
          m = fmaxf(m, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
        }
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  __shared__ float s_m[4];
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float bm = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax + g), __float_as_uint(bm));
  }
}

__global__ __launch_bounds__(256) void k_macro_from_amax(const float* __restrict__ amax, int64_t groups, float emax,
                                                         uint16_t* __restrict__ macro) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  const float a = amax[g];
  macro[g] = (uint16_t)(a > 0.0f ? fp16_rne_pos_clamped(a / (emax * 448.0f)) : 0u);
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

bool quantize_grid_ok(int64_t rows, int64_t k) { return rows >= 1 && k >= 256 && blocks_for16(rows, k) != 0; }
bool dequantize_grid_ok(int64_t rows, int64_t k) { return rows >= 1 && k >= 256 && blocks_for(rows, k) != 0; }

hipError_t launch_quantize(const void* x, int in_bf16, int64_t rows, int64_t k, int64_t ldx,
                           int elem_e4m3, int tiled, uint8_t* codes, uint8_t* micro,
                           uint16_t* macro, const uint16_t* macro_in, hipStream_t st) {
  const dim3 grid(blocks_for16(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
  const int stat = macro_in != nullptr;
#define FP4_Q(B, E, T, S) \
  hipLaunchKernelGGL((k_quantize<B, E, T, S>), grid, block, 0, st, x, ldx, rows, k, codes, micro, macro, macro_in)
#define FP4_Q_S(B, E, T) \
  if (stat) FP4_Q(B, E, T, 1); else FP4_Q(B, E, T, 0)
#define FP4_Q_T(B, E) \
  if (tiled) { FP4_Q_S(B, E, 1); } else { FP4_Q_S(B, E, 0); }
#define FP4_Q_E(B) \
  if (elem_e4m3) { FP4_Q_T(B, 1) } else { FP4_Q_T(B, 0) }
  if (in_bf16) { FP4_Q_E(1) } else { FP4_Q_E(0) }
#undef FP4_Q_E
#undef FP4_Q_T
#undef FP4_Q_S
#undef FP4_Q
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                             int64_t rows, int64_t k, int elem_e4m3, int tiled, void* y,
                             int out_bf16, int64_t ldy, hipStream_t st) {
  if (tiled && !elem_e4m3 && (reinterpret_cast<uintptr_t>(micro) & 7u) == 0) {
    // tiled E2M1 (rows % 16 == 0, k % 256 == 0): one tile per wave, four per workgroup
    const int64_t tiles = (rows / 16) * (k / kGroup);
    const int64_t blocks = (tiles + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (out_bf16)
      hipLaunchKernelGGL((k_dequantize_tiled<1>), dim3((unsigned)blocks), dim3(256), 0, st, codes, micro, macro,
                         tiles, k / kGroup, y, ldy);
    else
      hipLaunchKernelGGL((k_dequantize_tiled<0>), dim3((unsigned)blocks), dim3(256), 0, st, codes, micro, macro,
                         tiles, k / kGroup, y, ldy);
    return hipGetLastError();
  }
  const dim3 grid(blocks_for(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
#define FP4_D(B, E, T) \
  hipLaunchKernelGGL((k_dequantize<B, E, T>), grid, block, 0, st, codes, micro, macro, rows, k, y, ldy)
#define FP4_D_E(B) \
  if (elem_e4m3) { if (tiled) FP4_D(B, 1, 1); else FP4_D(B, 1, 0); } \
  else { if (tiled) FP4_D(B, 0, 1); else FP4_D(B, 0, 0); }
  if (out_bf16) { FP4_D_E(1) } else { FP4_D_E(0) }
#undef FP4_D_E
#undef FP4_D
  return hipGetLastError();
}

hipError_t launch_act_prep(const void* a, int in_bf16, int64_t rows, int64_t k, int64_t lda,
                           int elem_e4m3, _Float16* aq, int64_t ldq, float* scale,
                           const uint16_t* macro_in, hipStream_t st) {
  const dim3 grid(blocks_for16(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
#define FP4_ACT(B, E, G, S) \
  hipLaunchKernelGGL((k_act_prep<B, E, G, S>), grid, block, 0, st, a, lda, rows, k, aq, ldq, scale, macro_in)
#define FP4_ACT_S(B, E) \
  if (macro_in) FP4_ACT(B, E, 0, 1); else FP4_ACT(B, E, 0, 0)
  if (in_bf16) { if (elem_e4m3) { FP4_ACT_S(1, 1); } else { FP4_ACT_S(1, 0); } }
  else { if (elem_e4m3) { FP4_ACT_S(0, 1); } else { FP4_ACT_S(0, 0); } }
#undef FP4_ACT_S
  return hipGetLastError();
}

hipError_t launch_act_prep_gated(const uint16_t* a, int64_t rows, int64_t k, int64_t lda, int elem_e4m3,
                                 _Float16* aq, int64_t ldq, float* scale, hipStream_t st) {
  const dim3 grid(blocks_for16(rows, k)), block(256);
  if (grid.x == 0) return hipErrorInvalidValue;
  const uint16_t* macro_in = nullptr;
  if (elem_e4m3) FP4_ACT(1, 1, 1, 0); else FP4_ACT(1, 0, 1, 0);
#undef FP4_ACT
  return hipGetLastError();
}

hipError_t launch_act_calibrate(const void* x, int in_bf16, int64_t rows, int64_t k, int64_t ldx,
                                int elem_e4m3, float* amax, uint16_t* macro, hipStream_t st) {
  const int64_t groups = k >> 8;
  if (groups < 1 || groups > 0x7FFFFFFF || rows < 1) return hipErrorInvalidValue;
  const int64_t chunks = (rows + kCalRows - 1) / kCalRows;
  const dim3 grid((unsigned)groups, (unsigned)min(chunks, (int64_t)65535)), block(256);
  if (in_bf16) hipLaunchKernelGGL((k_amax_update<1>), grid, block, 0, st, x, ldx, rows, amax);
  else hipLaunchKernelGGL((k_amax_update<0>), grid, block, 0, st, x, ldx, rows, amax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_macro_from_amax, dim3((unsigned)((groups + 255) / 256)), block, 0, st, amax, groups,
                     elem_e4m3 ? 448.0f : 6.0f, macro);
  return hipGetLastError();
}

}  // namespace fp4lib
