// Operand traits of the 16-bit MFMA products (shared by the product kernels): the exact
// weight operand e2m1 * mu (or e4m3 * mu) in FP16 or bf16, and the 16x16x32 MFMA.
// Format: "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200",
// section "The Mathematical Breakthrough of Microscopic FP4 Scaling".
#pragma once
#include "fp4_device.h"

namespace fp4gemm {

using namespace fp4dev;

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

template <int A_BF16>
struct OpTraits;

template <>
struct OpTraits<0> {  // FP16 operands
  typedef half8_t frag;
  // micro-scale operand: the E4M3 byte shifted into the FP16 bit positions of both halves
  // is mu * 2^-8 exactly (E4M3 subnormals land on FP16 subnormals); the 2^8 is folded
  // into the column factor
  static constexpr float kMicroUnit = 256.0f;
  __device__ static __forceinline__ uint32_t micro_operand(uint32_t byte) { return (byte << 7) | (byte << 23); }
  __device__ static __forceinline__ frag weight(uint32_t cw, uint32_t mu_op) {
    const half2_t m2 = __builtin_bit_cast(half2_t, mu_op);
    const half2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * m2;
    const half2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * m2;
    const half2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * m2;
    const half2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * m2;
    return frag{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
  }
  // E4M3 weights (8 codes in two dwords): each code pair is converted with scale 2^5
  // (exact: the conversion applies a power of two) and multiplied by mu * 2^-8, so the
  // operand is e4m3 * mu * 2^-3, exact in FP16 (at most 8 significant bits, lowest bit
  // >= 2^-21, at most 25088); the column factor carries the 8
  static constexpr float kMicroUnit8 = 8.0f;
  __device__ static __forceinline__ frag weight8(uint32_t d0, uint32_t d1, uint32_t mu_op) {
    const half2_t m2 = __builtin_bit_cast(half2_t, mu_op);
    const half2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 32.0f, false) * m2;
    const half2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 32.0f, true) * m2;
    const half2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 32.0f, false) * m2;
    const half2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 32.0f, true) * m2;
    return frag{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
  }
  __device__ static __forceinline__ float4_t mfma(frag a, frag b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // Weight fragment of step T (0..3) of a word of four micro-scale bytes: the micro-scale
  // operands of two steps are formed at once, bytes 0 and 2 (even T) or 1 and 3 (odd T)
  // shifted into the FP16 bit positions of the low and high half (mu * 2^-8 exactly, as
  // micro_operand), and the half of step T is broadcast by the packed multiply's operand
  // select.
  template <int T>
  __device__ static __forceinline__ uint32_t micro_pair(uint32_t word) {
    return (T & 1) ? (word >> 1) & 0x7F807F80u : (word << 7) & 0x7F807F80u;
  }
  // The same fragment in five independent pieces, so that a kernel can spread them over
  // its MFMAs: the broadcast micro-scale operand of step T, then the packed pair of part P
  // (codes 2P and 2P + 1 of the word).
  typedef half2_t micro_t;
  template <int T>
  __device__ static __forceinline__ micro_t micro_step(uint32_t word) {
    const half2_t pr = __builtin_bit_cast(half2_t, micro_pair<T>(word));
    const _Float16 m = (T >> 1) ? pr[1] : pr[0];
    return half2_t{m, m};
  }
  template <int P>
  __device__ static __forceinline__ uint32_t weight_part(uint32_t cw, micro_t m2) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, P) * m2);
  }
  template <int T>
  __device__ static __forceinline__ frag weight_step(uint32_t cw, uint32_t word) {
    const micro_t m2 = micro_step<T>(word);
    return __builtin_bit_cast(frag, make_uint4(weight_part<0>(cw, m2), weight_part<1>(cw, m2),
                                               weight_part<2>(cw, m2), weight_part<3>(cw, m2)));
  }
};

template <>
struct OpTraits<1> {  // bf16 operands
  typedef bf16x8_t frag;
  // micro-scale operand: the E4M3 value as float32 bits
  static constexpr float kMicroUnit = 1.0f;
  __device__ static __forceinline__ uint32_t micro_operand(uint32_t byte) {
    return __float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)byte, 0));
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    // both values are exact in bf16: take the high halves
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  __device__ static __forceinline__ frag weight(uint32_t cw, uint32_t mu_op) {
    const float mu = __uint_as_float(mu_op);
    uint32_t w[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float2_t f;
      if (s == 0) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
      else if (s == 1) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
      else if (s == 2) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
      else f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
      w[s] = pack(f[0] * mu, f[1] * mu);
    }
    return __builtin_bit_cast(frag, make_uint4(w[0], w[1], w[2], w[3]));
  }
  __device__ static __forceinline__ float4_t mfma(frag a, frag b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // weight fragment of step T (0..3) of a word of four micro-scale bytes, whole or in the
  // pieces of the FP16 traits (micro-scale of step T as float32, packed pair of part P)
  typedef float micro_t;
  template <int T>
  __device__ static __forceinline__ micro_t micro_step(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8((int)word, T);
  }
  template <int P>
  __device__ static __forceinline__ uint32_t weight_part(uint32_t cw, micro_t mu) {
    const float2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, P);
    return pack(f[0] * mu, f[1] * mu);
  }
  template <int T>
  __device__ static __forceinline__ frag weight_step(uint32_t cw, uint32_t word) {
    return weight(cw, __float_as_uint(micro_step<T>(word)));
  }
};


}  // namespace fp4gemm
