// Dense product with 128-row wave tiles on gfx950 MFMA (large products):
//
//   C[r, n] = sum_g sA[r,g] * M_W[n,g] * sum_{k in g} A'[r,k] * (e2m1(W[n,k]) * mu_W[n,k/16])
//
// with the operands and per-group factors of the other product kernels (A' the exact FP16
// activation operand of the activation pass, or raw bf16 for W4A16; the weight operand
// e2m1 * mu exact in FP16 / bf16; v_mfma_f32_16x16x32 with float32 accumulation; the
// running sums kept in units of the current group's factors and rescaled at each group
// boundary). Every output element sees the same operations in the same order as in the
// other forms, so the results are bit-identical to them.
//
// What is different is the shape of the work, chosen from measurements on the device:
//   - the SIMD hides about two VALU instructions behind each 16x16x32 MFMA; every one
//     beyond costs ~4 cycles. A wave therefore owns 128 rows x 32 columns (8 x 2 MFMA
//     tiles): each decoded weight fragment (9 VALU) feeds 8 MFMAs, not 4;
//   - the micro-scale operands of two steps are formed by one shift and one mask, and the
//     per-group factor products are formed during the group, so only the multiplies of
//     the rescale land at the group boundary;
//   - LDS reads run at ~190 B/clk per CU: with 32 columns per wave each 1 KB activation
//     fragment feeds two MFMAs, 128 B/clk at the full MFMA rate.
// Workgroup: 8 waves side by side along n (two per SIMD), tile 128 x 256, one per CU.
// Pipeline: stages of 128 k (half a group, 4 MFMA steps) in a three-slot ring of LDS
// buffers, filled by LDS-DMA two stages ahead: the activation tile (128 x 128, 32 KB, in
// MFMA-fragment order; wave w copies row block w) and the weight codes (each wave its two
// row blocks, 1 KB each, contiguous in the tiled layout). One barrier per stage, before its
// last step, publishes the next stage so that the last step already loads the next
// stage's first fragments; it also frees the current slot, which then receives stage
// s + 3. Micro- and macro-scales come straight to registers one group ahead.
// "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200", section
// "The Mathematical Breakthrough of Microscopic FP4 Scaling", item 3: the scales are
// applied to the blocks right before the dot products.
#include <type_traits>

#include "fp4_device.h"
#include "fp4_kernels.h"
#include "gemm_ops.h"

using namespace fp4dev;
using namespace fp4gemm;
using fp4lib::GemmArgs;

namespace {

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format
constexpr int kWaves = 8;               // two per SIMD
constexpr int kMI = 8;                  // 16-row blocks per wave
constexpr int kNI = 2;                  // 16-column blocks per wave
constexpr int kBM = 16 * kMI;           // 128 rows per workgroup
constexpr int kBN = 16 * kNI * kWaves;  // 256 columns per workgroup
constexpr int kSteps = 4;               // 32-k MFMA steps per stage (128 k)
constexpr int kAChunks = kMI * kSteps * 64;  // 16-byte chunks of an activation stage: [mi][t][lane]
constexpr int kWChunks = kWaves * kNI * 64;  // of a weight stage: [wave][ni][lane]
constexpr int kCopies = kSteps + kNI;        // LDS-DMA instructions per wave and stage
constexpr int kLoads = 2 * kNI;              // register loads at a group's first barrier

__shared__ uint4 g_ra0[kAChunks];
__shared__ uint4 g_ra1[kAChunks];
__shared__ uint4 g_ra2[kAChunks];
__shared__ uint4 g_rw0[kWChunks];
__shared__ uint4 g_rw1[kWChunks];
__shared__ uint4 g_rw2[kWChunks];
// row-factor ratios of the FP16 operand path, [G][128]: a static object (k <= 8192), so the
// compiler can tell its reads from the slots the LDS-DMA copies are filling
constexpr int kMaxGroups = 32;
__shared__ float g_sa[kMaxGroups * kBM];

template <int B>
__device__ __forceinline__ uint4* a_slot() {
  if constexpr (B == 0) return g_ra0;
  else if constexpr (B == 1) return g_ra1;
  else return g_ra2;
}
template <int B>
__device__ __forceinline__ uint4* w_slot() {
  if constexpr (B == 0) return g_rw0;
  else if constexpr (B == 1) return g_rw1;
  else return g_rw2;
}

template <int A_BF16, int C_BF16>
__global__ __launch_bounds__(64 * kWaves, 1) void k_gemm_r8(GemmArgs args) {
  typedef OpTraits<A_BF16> Op;
  typedef typename Op::frag frag;
  const int groups = (int)(args.k >> 8);
  const int stages = 2 * groups;
  const int64_t nblocks = args.n >> 4;
  const int tiles_n = (int)((args.n + kBN - 1) / kBN);

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; each XCD gets a
  // contiguous run of tiles (n fastest), so its L2 keeps the same activation rows.
  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int tn = bid % tiles_n, tm = bid / tiles_n;
  const int64_t row_begin = (int64_t)tm * kBM, row_end = args.m;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t wb0 = (int64_t)tn * (kBN / 16) + wave * kNI;  // the wave's first 16-column block

  // ---- row-factor ratios of the FP16 operand path: f_g / f_{g+1}, the last group f_{G-1};
  // thread t covers row t % 128 and groups t / 128 + 4 j (a loop of uniform trip count)
  if (!A_BF16) {
    const int r = threadIdx.x & (kBM - 1);
    const float* f = args.a_scale + min(row_begin + r, row_end - 1) * groups;
    for (int g0 = 0; g0 < groups; g0 += kWaves * 64 / kBM) {
      const int g = g0 + (int)(threadIdx.x >> 7);
      if (g < groups) g_sa[g * kBM + r] = g + 1 < groups ? f[g] / f[g + 1] : f[g];
    }
  }

  // ---- buffer resources: per-lane byte offsets fixed for the whole k loop ----
  const uint16_t* a16 = static_cast<const uint16_t*>(args.a);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a16 + row_begin * args.lda), (short)0, (int)0xFFFFFFFF, kRsrcWord3);
  const int64_t a_row = min(row_begin + 16 * wave + l16, row_end - 1);  // wave w copies row block w
  const uint32_t a_voff = (uint32_t)(((a_row - row_begin) * args.lda + 8 * q) * 2);
  const int64_t blocks_left = nblocks - wb0 > 0 ? nblocks - wb0 : 0;
  const int64_t tiles_left = blocks_left * groups;
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(args.codes + wb0 * groups * kTileCodeBytes), (short)0,
      (int)min(tiles_left * kTileCodeBytes, (int64_t)0xFFFFFFFF), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mu_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(args.micro + wb0 * groups * kTileMicroBytes), (short)0,
      (int)min(tiles_left * kTileMicroBytes, (int64_t)0xFFFFFFFF), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mw_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(args.macro + wb0 * groups * kTileMacro), (short)0,
      (int)min(tiles_left * kTileMacro * 2, (int64_t)0xFFFFFFFF), kRsrcWord3);
  // copies of a stage past the last go through empty resources: zeros into the free slot,
  // no memory traffic, and every stage issues the same number of copies (the waits count)
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc((void*)a16, (short)0, 0, kRsrcWord3);
  const uint32_t mu_voff = (uint32_t)((q >> 1) * 128 + l16 * 8);

  auto copy_stage = [&](uint4* abuf, uint4* wbuf, int s) {  // stage s = 2 g + h
    const bool past = s >= stages;
    const int sc = past ? 0 : s;
    const int g = sc >> 1, h = sc & 1;
    const __amdgpu_buffer_rsrc_t ar = past ? none : a_rsrc;
    const __amdgpu_buffer_rsrc_t wr = past ? none : w_rsrc;
#pragma unroll
    for (int t = 0; t < kSteps; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void_ptr)(abuf + (wave * kSteps + t) * 64), 16, a_voff,
                                               (uint32_t)(sc * 256 + 64 * t), 0, 0);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_ptr)(wbuf + (wave * kNI + ni) * 64), 16,
                                               (uint32_t)lane * 16,
                                               (uint32_t)((ni * groups + g) * kTileCodeBytes + h * 1024), 0, 0);
  };
  // micro-scale bytes of group g (byte t = step t of the group) and macro-scale bits
  auto load_mu = [&](uint2 (&mu)[kNI], int g) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(mu_rsrc, mu_voff, (uint32_t)((ni * groups + g) * kTileMicroBytes), 0);
      mu[ni] = make_uint2(v[0], v[1]);
    }
  };
  auto load_mw = [&](uint32_t (&mw)[kNI], int g) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
      mw[ni] = __builtin_amdgcn_raw_buffer_load_b16(mw_rsrc, (uint32_t)l16 * 2, (uint32_t)((ni * groups + g) * kTileMacro * 2), 0);
  };
  // column factor of macro-scale bits (a zero factor counts as 1: its codes are 0)
  auto col_factor = [](uint32_t bits) {
    const float v = fp16_value_hw(bits & 0xFFFFu);
    return v != 0.0f ? v : 1.0f;
  };
  constexpr float kUnit = OpTraits<A_BF16>::kMicroUnit;

  // ---- prologue: macro-scales of groups 0 and 1, stages 0..2 in flight, stage 0 in ----
  uint32_t mw0[kNI], mw1[kNI], mw2[kNI];
  uint2 mu[kNI], mun[kNI];
  load_mw(mw0, 0);
  copy_stage(a_slot<0>(), w_slot<0>(), 0);
  load_mu(mu, 0);
  load_mw(mw1, min(1, groups - 1));
  copy_stage(a_slot<1>(), w_slot<1>(), 1);
  copy_stage(a_slot<2>(), w_slot<2>(), 2);
  __builtin_amdgcn_s_waitcnt(kVmcntWait<2 * kCopies>::value);  // stage 0 landed
  __syncthreads();                                              // ... for every wave; ratio table written

  float4_t x[kMI][kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) x[mi][ni] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // operands of step 0
  frag af[kMI], wf[kNI];
  uint4 cw[kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) af[mi] = __builtin_bit_cast(frag, a_slot<0>()[(mi * kSteps + 0) * 64 + lane]);
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    cw[ni] = w_slot<0>()[(wave * kNI + ni) * 64 + lane];
    wf[ni] = Op::template weight_step<0>(cw[ni].x, mu[ni].x);
  }

  // factor products p[mi][ni][i] = ratio_row * ratio_col of the boundary after the current
  // group (after the last group: the final factors), pn for the next group's
  float p[kMI][kNI][4];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[mi][ni][i] = 1.0f;
  const float* sa_lane = g_sa + 4 * q;  // + g * 128 + 16 mi: rows 16 mi + 4 q .. + 3
  // column ratio of the boundary after group g (after the last group: the final factor)
  auto col_ratios = [&](float (&rw)[kNI], int g, const uint32_t (&m_cur)[kNI], const uint32_t (&m_nxt)[kNI]) {
    const bool last = g + 1 >= groups;  // (selects, not branches: the step stays one region)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
      rw[ni] = col_factor(m_cur[ni]) * (last ? kUnit : __builtin_amdgcn_rcpf(col_factor(m_nxt[ni])));
  };
  auto products = [&](float (&pp)[kMI][kNI][4], int g, const float (&rw)[kNI], int mi_lo, int mi_hi) {
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      if (mi < mi_lo || mi >= mi_hi) continue;
      float4 ra = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
      if (!A_BF16) ra = *reinterpret_cast<const float4*>(sa_lane + g * kBM + 16 * mi);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        if (A_BF16) {
          pp[mi][ni][0] = pp[mi][ni][1] = pp[mi][ni][2] = pp[mi][ni][3] = rw[ni];
        } else {
          pp[mi][ni][0] = ra.x * rw[ni];
          pp[mi][ni][1] = ra.y * rw[ni];
          pp[mi][ni][2] = ra.z * rw[ni];
          pp[mi][ni][3] = ra.w * rw[ni];
        }
      }
    }
  };

  // One MFMA step: the step's 16 MFMAs (row block major); each activation fragment is
  // reloaded for the next step right after its two MFMAs (from `anext` at step `tnext`),
  // and the next step's weight fragments are decoded meanwhile. The rescale of a group
  // boundary is split over the two steps around it: POST (a group's last step) multiplies
  // row blocks 0..3 by the products `pp` once their last MFMAs of the group are done; PRE
  // (the next group's first step) multiplies row blocks 4..7 before their first MFMAs.
  auto mfma_step = [&](auto pre_c, auto post_c, const uint4* anext, int tnext, frag (&wn)[kNI],
                       const float (&pp)[kMI][kNI][4]) {
    constexpr bool PRE = decltype(pre_c)::value, POST = decltype(post_c)::value;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) x[mi][ni] = Op::mfma(af[mi], wf[ni], x[mi][ni]);
      if constexpr (PRE) {
        if (mi < kMI / 2) {
#pragma unroll
          for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[mi + kMI / 2][ni][i] *= pp[mi + kMI / 2][ni][i];
        }
      }
      if constexpr (POST) {
        if (mi >= kMI / 2) {
#pragma unroll
          for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[mi - kMI / 2][ni][i] *= pp[mi - kMI / 2][ni][i];
        }
      }
      af[mi] = __builtin_bit_cast(frag, anext[(mi * kSteps + tnext) * 64 + lane]);
    }
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) wf[ni] = wn[ni];
    // MFMA, VALU, MFMA, VALU, LDS read per row block (up to 6 VALU in each slot)
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
  };

  typedef std::integral_constant<bool, true> kTrue;
  typedef std::integral_constant<bool, false> kFalse;

  // Stage s in ring slot B (s % 3), H = s & 1 (H == 0: the first stage of group g).
  //   steps 0..2: MFMAs with the fragments reloaded from this slot; step 3 (after the
  //   barrier) reloads from the next slot and decodes the next stage's first weights;
  //   H == 0 (RESCALE: every group but the first): step 0 finishes the previous boundary's
  //   rescale; H == 1: the products of this group's boundary are formed in steps 0..2 and
  //   step 3 starts its rescale.
  // Wait before the barrier: stage s + 1's copies (issued after barrier s - 2) must have
  // landed; younger than them are the register loads of barrier s - 1 (when s - 1 is a
  // group's first stage) and the copies of barrier s - 1.
  float pn[kMI][kNI][4];
  auto run_stage = [&](auto b_c, auto h_c, auto rescale_c, int s) {
    constexpr int B = decltype(b_c)::value, H = decltype(h_c)::value;
    constexpr bool RESCALE = decltype(rescale_c)::value;
    constexpr int BN1 = (B + 1) % 3;
    typedef std::integral_constant<bool, H == 0 && RESCALE> kPre;
    typedef std::integral_constant<bool, H == 1> kPost;
    const int g = s >> 1;
    uint4* abuf = a_slot<B>();
    frag wn[kNI];
    float rw[kNI];
    // step 0
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) wn[ni] = Op::template weight_step<1>(cw[ni].y, H ? mu[ni].y : mu[ni].x);
    if (H == 1) {
      col_ratios(rw, g, mw0, mw1);
      products(pn, g, rw, 0, 3);
    }
    mfma_step(kPre{}, kFalse{}, abuf, 1, wn, p);
    __builtin_amdgcn_sched_barrier(0);
    // step 1
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) wn[ni] = Op::template weight_step<2>(cw[ni].z, H ? mu[ni].y : mu[ni].x);
    if (H == 1) products(pn, g, rw, 3, 6);
    mfma_step(kFalse{}, kFalse{}, abuf, 2, wn, p);
    __builtin_amdgcn_sched_barrier(0);
    // step 2
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) wn[ni] = Op::template weight_step<3>(cw[ni].w, H ? mu[ni].y : mu[ni].x);
    if (H == 1) products(pn, g, rw, 6, 8);
    mfma_step(kFalse{}, kFalse{}, abuf, 3, wn, p);
    __builtin_amdgcn_sched_barrier(0);
    // barrier: stage s + 1 published, this slot free
    constexpr int kWait = kCopies + (H == 1 ? kLoads : 0);
    __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<kWait>::value);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (H == 0) {  // a group's first stage: micro-scales of the next group, macro of the one after
      load_mu(mun, min(g + 1, groups - 1));
      load_mw(mw2, min(g + 2, groups - 1));
    }
    copy_stage(a_slot<B>(), w_slot<B>(), s + 3);
    __builtin_amdgcn_sched_barrier(0);
    // step 3: the next stage's code words and first weight fragments
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      cw[ni] = w_slot<BN1>()[(wave * kNI + ni) * 64 + lane];
      // next stage: same group (H == 0: second micro-scale word) or the next group's first
      wn[ni] = Op::template weight_step<0>(cw[ni].x, H ? mun[ni].x : mu[ni].y);
    }
    mfma_step(kFalse{}, kPost{}, a_slot<BN1>(), 0, wn, pn);
    __builtin_amdgcn_sched_barrier(0);
    if (H == 1) {  // next group: rotate the scales and the products
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        mu[ni] = mun[ni];
        mw0[ni] = mw1[ni];
        mw1[ni] = mw2[ni];
      }
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[mi][ni][i] = pn[mi][ni][i];
    }
  };
  typedef std::integral_constant<int, 0> C0;
  typedef std::integral_constant<int, 1> C1;
  typedef std::integral_constant<int, 2> C2;
  // group 0 (no boundary before it), then six stages per pass (slots cycle by 3, halves by
  // 2) starting at stage 2 (slot 2); every pass ends on a group boundary
  run_stage(C0{}, C0{}, kFalse{}, 0);
  run_stage(C1{}, C1{}, kFalse{}, 1);
  for (int s = 2; s < stages; s += 6) {
    run_stage(C2{}, C0{}, kTrue{}, s);
    run_stage(C0{}, C1{}, kTrue{}, s + 1);
    if (s + 2 >= stages) break;
    run_stage(C1{}, C0{}, kTrue{}, s + 2);
    run_stage(C2{}, C1{}, kTrue{}, s + 3);
    if (s + 4 >= stages) break;
    run_stage(C0{}, C0{}, kTrue{}, s + 4);
    run_stage(C1{}, C1{}, kTrue{}, s + 5);
  }
  // the ring's last copies (zeros from the empty resource) complete before exit
  __builtin_amdgcn_s_waitcnt(kVmcntWait<0>::value);

  // ---- final factors (the last group's products; row blocks 0..3 have them), store ----
  const int64_t n0 = wb0 * 16;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      if (wb0 + ni >= nblocks) continue;
      const int64_t col = n0 + 16 * ni + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row_begin + 16 * mi + 4 * q + i;
        if (r >= row_end) continue;
        // row blocks 0..3 were multiplied by the final factors in the last step
        const float v = mi < kMI / 2 ? x[mi][ni][i] : x[mi][ni][i] * p[mi][ni][i];
        if (C_BF16)
          static_cast<uint16_t*>(args.c)[r * args.ldc + col] = (uint16_t)bf16_rne_bits(v);
        else
          static_cast<float*>(args.c)[r * args.ldc + col] = v;
      }
    }
  }
}

}  // namespace

namespace fp4lib {

// LDS of the form (all static): three activation and weight slots (144 KB) and the
// row-factor ratios of up to 32 groups (16 KB).
bool gemm_r8_supports(int64_t m, int64_t n, int64_t k) {
  return m >= 1 && n >= 16 && n % 16 == 0 && k >= 256 && k % 256 == 0 && (k >> 8) <= kMaxGroups;
}

hipError_t launch_gemm_r8(const GemmArgs& g, hipStream_t st) {
  if (!gemm_r8_supports(g.m, g.n, g.k) || g.expert_offsets || g.w_e4m3) return hipErrorInvalidValue;
  const int64_t blocks = ((g.m + kBM - 1) / kBM) * ((g.n + kBN - 1) / kBN);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * kWaves);
  const size_t lds = 0;
  if (g.a_is_bf16) {
    if (g.c_is_bf16) hipLaunchKernelGGL((k_gemm_r8<1, 1>), grid, block, lds, st, g);
    else hipLaunchKernelGGL((k_gemm_r8<1, 0>), grid, block, lds, st, g);
  } else {
    if (g.c_is_bf16) hipLaunchKernelGGL((k_gemm_r8<0, 1>), grid, block, lds, st, g);
    else hipLaunchKernelGGL((k_gemm_r8<0, 0>), grid, block, lds, st, g);
  }
  return hipGetLastError();
}

}  // namespace fp4lib
