// Device helpers shared by the gfx950 kernels: exact scale conversions, vector types,
// the packed-layout index maps. Format: "NVIDIA Ships TensorRT-LLM 0.16: Native FP4
// Quantization for Blackwell B200", section "The Mathematical Breakthrough of
// Microscopic FP4 Scaling" (E2M1 elements, FP8 E4M3 per 16, FP16 per 256).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed data that is read once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// s_waitcnt immediate that waits until at most N vector-memory operations are pending
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at "no wait").
template <int N>
struct kVmcntWait {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  static constexpr int value = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
};

// Same, also waiting for every pending LDS / scalar-memory operation (lgkmcnt 0).
template <int N>
struct kVmcntLgkmWait {
  static constexpr int value = kVmcntWait<N>::value & ~(15 << 8);
};

constexpr int kBlock = 16;    // elements per micro-scale
constexpr int kGroup = 256;   // elements per macro-scale
constexpr int kTileRows = 16;
constexpr int kTileCodeBytes = 2048;  // 16 rows x 256 E2M1 codes
constexpr int kTile8CodeBytes = 4096;  // 16 rows x 256 E4M3 codes
constexpr int kTileMicroBytes = 256;  // 16 rows x 16 micro-scales
constexpr int kTileMacro = 16;        // 16 rows x 1 macro-scale

// Round a finite t > 0 to OCP E4M3 (nearest, ties to even significand, saturating at
// 448) and return the byte. Integer arithmetic on the float32 bits, so the result is the
// correctly rounded one whatever the hardware rounding mode is.
__device__ __forceinline__ uint32_t e4m3_rne_pos(float t) {
  if (!(t > 0x1p-10f)) return 0u;        // at or below half the smallest subnormal
  if (t >= 464.0f) return 0x7Eu;         // would round past 448
  const uint32_t u = __float_as_uint(t);
  const int e = (int)(u >> 23) - 127;    // t > 2^-10 is a normal float32
  const uint32_t sig = (u & 0x7FFFFFu) | 0x800000u;
  const int eq = e > -6 ? e : -6;        // binade of the result (or the subnormal range)
  const int shift = 20 + (eq - e);       // keep 3 fraction bits: units of 2^(eq-3)
  uint32_t q = sig >> shift;
  const uint32_t rem = sig & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  const uint32_t byte = (uint32_t)((eq + 6) * 8) + q;  // q in [0, 16] carries into e
  return byte < 0x7Eu ? byte : 0x7Eu;
}

// Value of an E4M3 byte (no NaN bytes are ever produced by this library).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))  // 2^(e-7)(1+m/8)
                : (float)m * 0x1p-9f;
  return (b & 0x80u) ? -mag : mag;
}

// Round a finite t > 0 to FP16 and clamp into [2^-24, 65504]; returns the bit pattern.
__device__ __forceinline__ uint32_t fp16_rne_pos_clamped(float t) {
  if (t >= 65504.0f) return 0x7BFFu;
  const uint32_t u = __float_as_uint(t);
  const int e = (int)(u >> 23) - 127;
  if (e < -25) return 0x0001u;           // rounds to zero: clamp to the smallest subnormal
  const uint32_t sig = (u & 0x7FFFFFu) | 0x800000u;
  const int eq = e > -14 ? e : -14;
  const int shift = 13 + (eq - e);       // keep 10 fraction bits
  uint32_t q = sig >> shift;
  const uint32_t rem = sig & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  uint32_t bits = (uint32_t)((eq + 14) * 1024) + q;
  if (bits == 0u) bits = 1u;
  return bits < 0x7BFFu ? bits : 0x7BFFu;
}

// Value of an FP16 bit pattern (exact, subnormals included).
__device__ __forceinline__ float fp16_value(uint32_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  float mag = e ? __uint_as_float(((e + 112u) << 23) | (m << 13)) : (float)m * 0x1p-24f;
  return (h & 0x8000u) ? -mag : mag;
}

// Same value through the hardware conversion (exact; FP16 denormals are kept in the
// default floating-point mode). Branch-free, for the inner loops.
__device__ __forceinline__ float fp16_value_hw(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// bfloat16 bits of a float32, round to nearest even, by the hardware conversion
// (v_cvt_pk_bf16_f32): on every non-NaN value, denormals, ties and overflow to infinity
// included, the same bits as integer rounding of the float pattern; a NaN stays a NaN.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) { return bf16x2_rne(f, 0.0f) & 0xFFFFu; }

__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// E2M1 magnitude (3-bit code) of |x| for effective scale s > 0, by comparing against the
// exact tie points t*s (t = .25 .75 1.25 1.75 2.5 3.5 5); '>' vs '>=' alternates so that a
// tie resolves to the even significand. Each t*s is exact in float32.
struct E2M1Thresholds {
  float s025, s075, s125, s175, s25, s35, s5;
  __device__ __forceinline__ explicit E2M1Thresholds(float s)
      : s025(0.25f * s), s075(0.75f * s), s125(1.25f * s), s175(1.75f * s), s25(2.5f * s),
        s35(3.5f * s), s5(5.0f * s) {}
  // The tie points increase, so the code is the number of them that |x| passes. Counted
  // branch-free: a three-level search written with nested selects was lowered to one
  // divergent branch region per element, which kept every element's partial code live
  // until the final pack (the bf16 quantize kernels sat at 71 VGPRs, 7 waves per SIMD).
  __device__ __forceinline__ uint32_t mag(float ax) const {
    return (uint32_t)(ax > s025) + (uint32_t)(ax >= s075) + (uint32_t)(ax > s125) +
           (uint32_t)(ax >= s175) + (uint32_t)(ax > s25) + (uint32_t)(ax >= s35) + (uint32_t)(ax > s5);
  }
};

__device__ __forceinline__ float e2m1_mag_value(uint32_t mag) {
  // 0, .5, 1, 1.5, 2, 3, 4, 6
  const uint32_t e = mag >> 1, m = mag & 1u;
  return e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
}

// 16 consecutive input elements as raw 16-byte words, so that the next item's input can
// be in flight while the current one is encoded.
template <int IN_BF16>
struct Raw16 {
  uint4 q[IN_BF16 ? 2 : 4];
};

template <int IN_BF16>
__device__ __forceinline__ void load_raw16(const void* __restrict__ x, int64_t off, Raw16<IN_BF16>& d) {
  const uint4* p = IN_BF16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off)
                           : reinterpret_cast<const uint4*>(static_cast<const float*>(x) + off);
#pragma unroll
  for (int i = 0; i < (IN_BF16 ? 2 : 4); ++i) d.q[i] = p[i];
}

template <int IN_BF16>
__device__ __forceinline__ void unpack16(const Raw16<IN_BF16>& d, float v[16]) {
#pragma unroll
  for (int i = 0; i < (IN_BF16 ? 2 : 4); ++i) {
    const uint32_t w[4] = {d.q[i].x, d.q[i].y, d.q[i].z, d.q[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (IN_BF16) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      } else {
        v[4 * i + j] = __uint_as_float(w[j]);
      }
    }
  }
}

// Scales of a lane that owns one whole micro-vector (16 lanes per group).
__device__ __forceinline__ float block_scales(const float v[16], float emax, uint32_t& m_bits,
                                              uint32_t& mu_byte, float& m_val) {
  float amax_b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));
  float amax_g = amax_b;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax_g = fmaxf(amax_g, __shfl_xor(amax_g, o));
  m_bits = 0u;
  m_val = 0.0f;
  mu_byte = 0u;
  if (amax_g > 0.0f) {
    m_bits = fp16_rne_pos_clamped(amax_g / (emax * 448.0f));
    m_val = fp16_value(m_bits);
    mu_byte = e4m3_rne_pos(amax_b / (emax * m_val));
  }
  return e4m3_value(mu_byte) * m_val;
}

__device__ __forceinline__ uint32_t sign_of(float f) { return __float_as_uint(f) >> 31; }

// E2M1 codes of 16 elements for effective scale s (codes 0 when s = 0): element i of
// v[0..7] in nibble i of w0, of v[8..15] in nibble i of w1 (low nibble first).
__device__ __forceinline__ void e2m1_encode16(const float v[16], float s, uint32_t& w0, uint32_t& w1) {
  w0 = 0u;
  w1 = 0u;
  if (s > 0.0f) {
    const E2M1Thresholds th(s);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0 |= (th.mag(fabsf(v[i])) | (sign_of(v[i]) << 3)) << (4 * i);
      w1 |= (th.mag(fabsf(v[8 + i])) | (sign_of(v[8 + i]) << 3)) << (4 * i);
    }
  }
}

// Byte offset of the code dword (8 codes) for row r, columns [c8*8, c8*8+8) inside the
// tiled layout, and the micro/macro offsets (see the header for the layout).
__device__ __forceinline__ int64_t tiled_code_offset(int64_t r, int64_t col, int64_t groups) {
  const int64_t tile = (r >> 4) * groups + (col >> 8);
  const int c = (int)(col & 255), n = (int)(r & 15);
  const int t = c >> 5, j = (c >> 3) & 3;
  return tile * kTileCodeBytes + (t >> 2) * 1024 + (16 * j + n) * 16 + (t & 3) * 4;
}
// E4M3 elements in the tiled layout: 8 codes of row r at columns [col, col + 8) (col % 8
// == 0). Per tile, half h = t / 4 of the 256 columns (t = c / 32) holds two 1024-byte
// pieces p = (t % 4) / 2; lane 16 j + n (j = (c % 32) / 8) owns 16 bytes of each piece,
// the 8 codes of column run t in bytes 8 (t % 2) .. +7.
__device__ __forceinline__ int64_t tiled8_code_offset(int64_t r, int64_t col, int64_t groups) {
  const int64_t tile = (r >> 4) * groups + (col >> 8);
  const int c = (int)(col & 255), n = (int)(r & 15);
  const int t = c >> 5, j = (c >> 3) & 3;
  return tile * kTile8CodeBytes + (t >> 2) * 2048 + ((t >> 1) & 1) * 1024 + (16 * j + n) * 16 + (t & 1) * 8;
}
__device__ __forceinline__ int64_t tiled_micro_offset(int64_t r, int64_t col, int64_t groups) {
  const int64_t tile = (r >> 4) * groups + (col >> 8);
  const int c = (int)(col & 255), n = (int)(r & 15);
  const int b = c >> 4;
  return tile * kTileMicroBytes + (b & 1) * 128 + n * 8 + (b >> 1);
}
__device__ __forceinline__ int64_t tiled_macro_offset(int64_t r, int64_t col, int64_t groups) {
  return ((r >> 4) * groups + (col >> 8)) * kTileMacro + (r & 15);
}

}  // namespace fp4dev
