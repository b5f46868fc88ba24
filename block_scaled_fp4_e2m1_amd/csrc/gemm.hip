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

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

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
                                 int& expert, int64_t& row_begin, int64_t& row_end, int BM) {
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

// ---------------------------------------------------------------------------------
// Main product kernel. Workgroup: 4 waves side by side along n; tile 64 rows x 256
// weight rows; each wave owns a 64 x 64 block as 4 x 4 MFMA tiles, so every weight
// fragment is decoded by exactly one wave. The k loop runs in half-groups of 128:
//   - activation tiles (64 x 128, 16 KB) are copied into LDS by LDS-DMA in MFMA-fragment
//     order, double-buffered in two separate LDS objects (so the copy into one buffer
//     never has to wait for reads of the other);
//   - weight codes of the next half-group are prefetched into registers, micro-scales
//     one group ahead;
//   - the per-row activation factors and per-column macro-scales of every group are
//     copied into LDS once, at the start.
// Each 256-column group accumulates into fresh MFMA sums that are folded into the
// running sums with one float32 multiply-add (factor sA * M_W) per output element.
// ---------------------------------------------------------------------------------
constexpr int kBM = 64;              // rows per workgroup
constexpr int kBN = 256;             // weight rows (output columns) per workgroup
constexpr int kHalf = 128;           // k per pipeline stage
constexpr int kMaxGroupsLds = 64;    // k <= 16384 for the LDS factor tables
constexpr int kAStage = kBM * kHalf * 2 / 16;  // 16-byte chunks per activation stage

__shared__ uint4 g_abuf0[kAStage];
__shared__ uint4 g_abuf1[kAStage];
__shared__ float g_sa[kBM * kMaxGroupsLds];         // [row][group] activation factors
__shared__ uint16_t g_mw[(kBN / 16) * kMaxGroupsLds * 16];  // tiled macro-scales of the tile

template <int A_BF16, int C_BF16, int GROUPED>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs args) {
  typedef OpTraits<A_BF16> Op;
  typedef typename Op::frag frag;
  const int groups = (int)(args.k >> 8);
  const int64_t n = args.n;
  const int64_t nblocks = n >> 4;
  const int tiles_n = (int)((n + kBN - 1) / kBN);

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of tiles (n fastest) so its L2 keeps the same activation rows.
  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int tn = bid % tiles_n;
  const int tm = bid / tiles_n;

  int64_t row_begin, row_end, w_row_base = 0;
  if (GROUPED) {
    int expert;
    if (!find_expert_tile(args.expert_offsets, args.n_experts, tm, expert, row_begin, row_end, kBM))
      return;
    w_row_base = (int64_t)expert * n;
  } else {
    row_begin = (int64_t)tm * kBM;
    row_end = args.m;
    if (row_begin >= row_end) return;
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t n0 = (int64_t)tn * kBN + wave * 64;  // first output column of this wave
  const int64_t nb_tile0 = w_row_base / 16 + (int64_t)tn * (kBN / 16);  // first row block of the tile

  // ---- one-time tables: activation factors [row][g] and macro-scales of the tile ----
  {
    // activation factors: lane-wise DMA of 4-byte elements (row r, group g) -> g_sa[r*G+g]
    const int elems = kBM * groups;
    for (int e0 = wave * 64; e0 < elems; e0 += 256) {
      const int e = min(e0 + lane, elems - 1);
      const int r = e / groups, g = e - r * groups;
      int64_t src_row = min(row_begin + r, row_end - 1);
      if (GROUPED && args.row_token) src_row = args.row_token[src_row];
      const float* src = args.a_scale ? args.a_scale + src_row * groups + g : nullptr;
      if (src)
        __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)(g_sa + e0), 4, 0, 0);
    }
    // macro-scales: the tile's 16 row blocks x G groups x 16 rows are contiguous
    const int mw_elems = (kBN / 16) * groups * 16;       // uint16 count
    const int64_t mw_first = nb_tile0 * groups * 16;
    const int64_t mw_last = (w_row_base / 16 + nblocks) * groups * 16;  // exclusive bound
    for (int c0 = wave * 64 * 2; c0 < mw_elems; c0 += 256 * 2) {  // 4-byte lanes = 2 entries
      const int64_t src = min(mw_first + c0 + 2 * lane, mw_last - 2);
      __builtin_amdgcn_global_load_lds((global_void_ptr)(args.macro + src), (lds_void_ptr)(g_mw + c0), 4, 0, 0);
    }
  }

  // ---- activation DMA: wave w copies row tile mi = w (16 rows) for the 4 steps of a stage ----
  const uint16_t* a16 = static_cast<const uint16_t*>(args.a);
  int64_t a_src_row = min(row_begin + wave * 16 + l16, row_end - 1);
  if (GROUPED && args.row_token) a_src_row = args.row_token[a_src_row];
  const uint16_t* a_lane_src = a16 + a_src_row * args.lda + 8 * q;
  auto dma_stage = [&](uint4* buf, int stage) {  // stage = 2 g + h
    const int64_t k0 = (int64_t)stage * kHalf;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      __builtin_amdgcn_global_load_lds((global_void_ptr)(a_lane_src + k0 + 32 * t),
                                       (lds_void_ptr)(buf + (wave * 4 + t) * 64), 16, 0, 0);
  };

  // ---- weights: 4 row blocks (16 columns each) per wave ----
  int64_t wtile0[4];
  bool w_ok[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int64_t nb = n0 / 16 + ni;
    w_ok[ni] = nb < nblocks;
    wtile0[ni] = (w_row_base / 16 + min(nb, nblocks - 1)) * groups;
  }
  auto load_codes = [&](uint4 (&wc)[4], int stage) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      wc[ni] = *(reinterpret_cast<const uint4*>(args.codes + (wtile0[ni] + (stage >> 1)) * kTileCodeBytes +
                                                (stage & 1) * 1024) + lane);
  };
  auto load_micro = [&](uint2 (&mu)[4], int g) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      mu[ni] = *reinterpret_cast<const uint2*>(args.micro + (wtile0[ni] + g) * kTileMicroBytes +
                                               (q >> 1) * 128 + l16 * 8);
  };

  float4_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float4_t part[4][4];

  uint4 wc0[4], wc1[4];   // codes of the current / next half-group
  uint2 mu_cur[4], mu_nxt[4];

  // prologue: stage 0 in flight
  dma_stage(g_abuf0, 0);
  load_codes(wc0, 0);
  load_micro(mu_cur, 0);

  // one pipeline stage: 4 MFMA steps over the LDS buffer, weight codes wc, steps 4h..4h+3
  auto compute_stage = [&](const uint4* buf, const uint4 (&wc)[4], const uint2 (&mu)[4], int h) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      frag af[4], wf[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = __builtin_bit_cast(frag, buf[(mi * 4 + t) * 64 + lane]);
      const int tt = h * 4 + t;  // step within the group: micro-block 2tt + (q >> 1)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const uint32_t cw = t == 0 ? wc[ni].x : t == 1 ? wc[ni].y : t == 2 ? wc[ni].z : wc[ni].w;
        const uint32_t mw = h == 0 ? mu[ni].x : mu[ni].y;
        float mu_f;
        switch (t) {
          case 0: mu_f = __builtin_amdgcn_cvt_f32_fp8((int)mw, 0); break;
          case 1: mu_f = __builtin_amdgcn_cvt_f32_fp8((int)mw, 1); break;
          case 2: mu_f = __builtin_amdgcn_cvt_f32_fp8((int)mw, 2); break;
          default: mu_f = __builtin_amdgcn_cvt_f32_fp8((int)mw, 3); break;
        }
        wf[ni] = Op::weight(cw, mu_f);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          part[mi][ni] = Op::mfma(af[mi], wf[ni], tt == 0 ? float4_t{0.0f, 0.0f, 0.0f, 0.0f} : part[mi][ni]);
      __builtin_amdgcn_sched_barrier(0);  // one step's operands live at a time
    }
  };

  // vm operations issued per stage by each wave (all counted by the waits below)
  constexpr int kDmaPerStage = 4, kCodesPerStage = 4, kMicroPerGroup = 4;

  for (int g = 0; g < groups; ++g) {
    // ---------- first half of group g (buffer 0) ----------
    dma_stage(g_abuf1, 2 * g + 1);
    load_codes(wc1, 2 * g + 1);
    // wait for stage 2g (issued one stage ago): the 8 operations just issued may pend
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kVmcntWait<kDmaPerStage + kCodesPerStage>::value);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(g_abuf0, wc0, mu_cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();  // every wave is done reading buffer 0
    __builtin_amdgcn_sched_barrier(0);

    // ---------- second half of group g (buffer 1) ----------
    const bool more = g + 1 < groups;
    if (more) {
      dma_stage(g_abuf0, 2 * g + 2);
      load_codes(wc0, 2 * g + 2);
      load_micro(mu_nxt, g + 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kVmcntWait<kDmaPerStage + kCodesPerStage + kMicroPerGroup>::value);
    } else {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kVmcntWait<0>::value);
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(g_abuf1, wc1, mu_cur, 1);

    // ---------- fold group g ----------
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      float sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sa[i] = args.a_scale ? g_sa[(mi * 16 + 4 * q + i) * groups + g] : 1.0f;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const float mw = fp16_value_hw(g_mw[((wave * 4 + ni) * groups + g) * 16 + l16]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mi][ni][i] = fmaf(sa[i] * mw, part[mi][ni][i], acc[mi][ni][i]);
      }
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) mu_cur[ni] = mu_nxt[ni];
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();  // every wave is done reading buffer 1
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- store ----
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      if (!w_ok[ni]) continue;
      const int64_t col = n0 + 16 * ni + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row_begin + 16 * mi + 4 * q + i;
        if (r >= row_end) continue;
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

bool gemm_supports(int64_t k) { return (k >> 8) <= kMaxGroupsLds; }

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (!gemm_supports(g.k)) return hipErrorInvalidValue;
  const int64_t tiles_n = (g.n + kBN - 1) / kBN;
  int64_t tiles_m;
  if (g.expert_offsets) tiles_m = (g.m + kBM - 1) / kBM + g.n_experts;  // upper bound
  else tiles_m = (g.m + kBM - 1) / kBM;
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
