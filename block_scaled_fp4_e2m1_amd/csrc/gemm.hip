// Dense and grouped (mixture-of-experts) products on gfx950 MFMA.
//
//   C[r, n] = sum_g sA[r,g] * M_W[n,g] * sum_{k in g} A'[r,k] * (e2m1(W[n,k]) * mu_W[n,k/16])
//
// A' is the activation operand with everything but its per-256 factor sA applied: for
// W4A4 / W4A8 it is the FP16 output of the activation pass (exact), for W4A16 the raw
// bf16 activations (sA = 1). The weight operand e2m1 * mu is exact in FP16 (at most 6
// significant bits, range [2^-10, 2688]) and in bf16, so every MFMA product is exact and
// only the float32 accumulation rounds. The per-256 factors cannot be folded into the
// 16-bit operands exactly, so each 256-column group is accumulated separately and folded
// into the running sums with one float32 multiply-add per output element per group.
//
// Tiling: 256 threads = 2 x 2 waves, 64 x 64 outputs per wave as 4 x 4 tiles of
// v_mfma_f32_16x16x32_{f16,bf16}; the workgroup covers 128 rows x 128 weight rows.
// Weight fragments come straight from the tiled layout (each lane's 16-byte load is one
// MFMA operand row); activation fragments are 16-byte row loads.
//
// Grouped form: the workgroup grid enumerates (expert, 128-row tile) pairs; each
// workgroup finds its expert by a prefix sum over the per-expert tile counts, so one
// launch covers every expert whatever the routing produced (including empty experts).
// "llama.cpp Put Precision Policy Inside the Model", section "One model can need more
// than one precision": the same W4A4/W4A8 routing serves dense and mixture-of-experts.
#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;
using fp4lib::GemmArgs;

namespace {

constexpr int BM = 128, BN = 128;

template <int A_BF16>
struct OpTraits;

template <>
struct OpTraits<0> {  // FP16 operands
  typedef half8_t frag;
  __device__ static __forceinline__ frag weight(uint32_t cw, float mu) {
    const _Float16 h = (_Float16)mu;  // E4M3 values are exact in FP16
    const half2_t m2 = {h, h};
    const half2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * m2;
    const half2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * m2;
    const half2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * m2;
    const half2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * m2;
    return frag{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
  }
  __device__ static __forceinline__ float4_t mfma(frag a, frag b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct OpTraits<1> {  // bf16 operands
  typedef bf16x8_t frag;
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    // both values are exact in bf16: take the high halves
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  __device__ static __forceinline__ frag weight(uint32_t cw, float mu) {
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
};

// Locate the tile of a grouped launch: tile index t runs over the concatenation of every
// expert's ceil(rows_e / BM) row tiles. One wave computes the prefix sum of the tile
// counts (each lane sums a contiguous range of experts, then a 64-lane scan); the lane
// whose range holds t finds the expert. Returns false past the last tile.
__device__ bool find_expert_tile(const int32_t* __restrict__ offsets, int n_experts, int64_t t,
                                 int& expert, int64_t& row_begin, int64_t& row_end) {
  __shared__ int s_expert;
  __shared__ int s_first;
  if (threadIdx.x == 0) s_expert = -1;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (n_experts + 63) / 64;
    const int e_lo = min(lane * per, n_experts), e_hi = min(e_lo + per, n_experts);
    int cnt = 0;
    for (int e = e_lo; e < e_hi; ++e) cnt += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    const int excl = incl - cnt;
    if (t >= excl && t < incl) {  // exactly one lane
      int base = excl;
      for (int e = e_lo; e < e_hi; ++e) {
        const int te = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
        if (t < base + te) { s_expert = e; s_first = base; break; }
        base += te;
      }
    }
  }
  __syncthreads();
  if (s_expert < 0) return false;
  expert = s_expert;
  row_begin = offsets[expert] + (t - s_first) * BM;
  row_end = offsets[expert + 1];
  return true;
}

template <int A_BF16, int C_BF16, int GROUPED>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs args) {
  typedef OpTraits<A_BF16> Op;
  typedef typename Op::frag frag;
  const int64_t groups = args.k >> 8;
  const int64_t n = args.n;
  const int64_t tiles_n = (n + BN - 1) / BN;
  const int64_t tn = blockIdx.x % tiles_n;
  const int64_t tm = blockIdx.x / tiles_n;

  int64_t row_begin, row_end;
  int64_t w_row_base = 0;  // first weight row of this product (expert offset)
  if (GROUPED) {
    int expert;
    if (!find_expert_tile(args.expert_offsets, args.n_experts, tm, expert, row_begin, row_end))
      return;
    w_row_base = (int64_t)expert * n;
  } else {
    row_begin = tm * BM;
    row_end = args.m;
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t m0 = row_begin + wm * 64;      // first routed row of this wave
  const int64_t n0 = tn * BN + wn * 64;         // first output column of this wave
  const int64_t nblocks = n >> 4;

  // source rows of the A operand for this lane (operand row = l16 of each 16-row tile)
  int64_t a_row[4];
  bool a_ok[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t r = m0 + 16 * mi + l16;
    a_ok[mi] = r < row_end;
    int64_t src = r;
    if (GROUPED && args.row_token && a_ok[mi]) src = args.row_token[r];
    a_row[mi] = a_ok[mi] ? src : 0;
  }
  // source rows of the lane's output elements (for the activation factors)
  int64_t o_src[4][4];
  bool o_ok[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = m0 + 16 * mi + 4 * q + i;
      o_ok[mi][i] = r < row_end;
      int64_t src = r;
      if (GROUPED && args.row_token && o_ok[mi][i]) src = args.row_token[r];
      o_src[mi][i] = o_ok[mi][i] ? src : 0;
    }
  bool w_ok[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) w_ok[ni] = (n0 / 16 + ni) < nblocks;

  float4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const uint16_t* a16 = static_cast<const uint16_t*>(args.a);

  for (int64_t g = 0; g < groups; ++g) {
    // weight fragments of this group: codes, micro-scales, macro-scale per column
    uint4 wc[4][2];
    uint2 wmu[4];
    float wM[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t tile = (w_row_base / 16 + n0 / 16 + ni) * groups + g;
      if (w_ok[ni]) {
        const uint4* cp = reinterpret_cast<const uint4*>(args.codes + tile * kTileCodeBytes) + lane;
        wc[ni][0] = cp[0];
        wc[ni][1] = cp[64];
        wmu[ni] = *reinterpret_cast<const uint2*>(args.micro + tile * kTileMicroBytes + (q >> 1) * 128 + l16 * 8);
        wM[ni] = fp16_value(args.macro[tile * kTileMacro + l16]);
      } else {
        wc[ni][0] = wc[ni][1] = make_uint4(0, 0, 0, 0);
        wmu[ni] = make_uint2(0, 0);
        wM[ni] = 0.0f;
      }
    }
    float4_t part[4][4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      frag af[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (a_ok[mi]) v = *reinterpret_cast<const uint4*>(a16 + a_row[mi] * args.lda + g * kGroup + 32 * t + 8 * q);
        af[mi] = __builtin_bit_cast(frag, v);
      }
      frag wf[4];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const uint4 c4 = wc[ni][t >> 2];
        const uint32_t cw = (t & 3) == 0 ? c4.x : (t & 3) == 1 ? c4.y : (t & 3) == 2 ? c4.z : c4.w;
        const uint32_t mw = (t < 4) ? wmu[ni].x : wmu[ni].y;
        const float2_t mu2 = (t & 2) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)mw, true)
                                     : __builtin_amdgcn_cvt_pk_f32_fp8((int)mw, false);
        wf[ni] = Op::weight(cw, (t & 1) ? mu2[1] : mu2[0]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          part[mi][ni] = Op::mfma(af[mi], wf[ni], t == 0 ? float4_t{0.0f, 0.0f, 0.0f, 0.0f} : part[mi][ni]);
    }
    // fold this group's partial sums with its factors
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      float sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sa[i] = (args.a_scale && o_ok[mi][i]) ? args.a_scale[o_src[mi][i] * groups + g] : 1.0f;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[mi][ni][i] = fmaf(sa[i] * wM[ni], part[mi][ni][i], acc[mi][ni][i]);
    }
  }

  // store
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      if (!w_ok[ni]) continue;
      const int64_t col = n0 + 16 * ni + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!o_ok[mi][i]) continue;
        const int64_t r = m0 + 16 * mi + 4 * q + i;
        if (C_BF16)
          static_cast<uint16_t*>(args.c)[r * args.ldc + col] = (uint16_t)bf16_rne_bits(acc[mi][ni][i]);
        else
          static_cast<float*>(args.c)[r * args.ldc + col] = acc[mi][ni][i];
      }
    }
}

// float32 activations: one thread per output, exact weight values, float32 FMA.
template <int C_BF16>
__global__ __launch_bounds__(256) void k_gemm_f32act(const float* __restrict__ a, int64_t lda,
                                                     int64_t m, int64_t k,
                                                     const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ micro,
                                                     const uint16_t* __restrict__ macro,
                                                     int64_t n, void* __restrict__ c, int64_t ldc) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= m * n) return;
  const int64_t row = idx / n, col = idx - row * n;
  const int64_t groups = k >> 8;
  float acc = 0.0f;
  for (int64_t g = 0; g < groups; ++g) {
    float part = 0.0f;
    for (int b = 0; b < 16; ++b) {
      const int64_t kk = g * kGroup + b * 16;
      const float mu = e4m3_value(micro[tiled_micro_offset(col, kk, groups)]);
      float blk = 0.0f;
      for (int e8 = 0; e8 < 2; ++e8) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + tiled_code_offset(col, kk + 8 * e8, groups));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t cd = (w >> (4 * i)) & 15u;
          const float v = e2m1_mag_value(cd & 7u);
          blk = fmaf(a[row * lda + kk + 8 * e8 + i], (cd & 8u) ? -v : v, blk);
        }
      }
      part = fmaf(mu, blk, part);
    }
    acc = fmaf(fp16_value(macro[tiled_macro_offset(col, g * kGroup, groups)]), part, acc);
  }
  if (C_BF16) static_cast<uint16_t*>(c)[row * ldc + col] = (uint16_t)bf16_rne_bits(acc);
  else static_cast<float*>(c)[row * ldc + col] = acc;
}

}  // namespace

namespace fp4lib {

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  const int64_t tiles_n = (g.n + BN - 1) / BN;
  int64_t tiles_m;
  if (g.expert_offsets) tiles_m = (g.m + BM - 1) / BM + g.n_experts;  // upper bound
  else tiles_m = (g.m + BM - 1) / BM;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks <= 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
#define FP4_GEMM(A, C, G) hipLaunchKernelGGL((k_gemm<A, C, G>), grid, block, 0, st, g)
  const int grouped = g.expert_offsets != nullptr;
  if (g.a_is_bf16) {
    if (g.c_is_bf16) { if (grouped) FP4_GEMM(1, 1, 1); else FP4_GEMM(1, 1, 0); }
    else { if (grouped) FP4_GEMM(1, 0, 1); else FP4_GEMM(1, 0, 0); }
  } else {
    if (g.c_is_bf16) { if (grouped) FP4_GEMM(0, 1, 1); else FP4_GEMM(0, 1, 0); }
    else { if (grouped) FP4_GEMM(0, 0, 1); else FP4_GEMM(0, 0, 0); }
  }
#undef FP4_GEMM
  return hipGetLastError();
}

hipError_t launch_gemm_f32act(const float* a, int64_t lda, int64_t m, int64_t k,
                              const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                              int64_t n, void* c, int out_bf16, int64_t ldc, hipStream_t st) {
  const int64_t total = m * n;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (out_bf16)
    hipLaunchKernelGGL((k_gemm_f32act<1>), grid, block, 0, st, a, lda, m, k, codes, micro, macro, n, c, ldc);
  else
    hipLaunchKernelGGL((k_gemm_f32act<0>), grid, block, 0, st, a, lda, m, k, codes, micro, macro, n, c, ldc);
  return hipGetLastError();
}

}  // namespace fp4lib
