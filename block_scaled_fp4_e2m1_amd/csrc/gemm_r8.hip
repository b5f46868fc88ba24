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

// Packed activations (W4A4): per wave and stage, its 16 rows' E2M1 codes (64 chunks of
// 16 bytes: lane L's chunk is row L % 16, bytes 16 (L / 16) of the row's 64) and their
// micro-scales (16 chunks: lane L's 4 bytes are row L % 16, bytes 4 ((L / 16) % 2) of the
// row's 8; lanes 32..63 repeat lanes 0..31), in the same three-slot ring as the weights.
// The decoded FP16 stages then alternate between two activation slots.
constexpr int kPackChunks = 80;
__shared__ uint4 g_pa0[kWaves * kPackChunks];
__shared__ uint4 g_pa1[kWaves * kPackChunks];
__shared__ uint4 g_pa2[kWaves * kPackChunks];
template <int B>
__device__ __forceinline__ uint4* p_slot() {
  if constexpr (B == 0) return g_pa0;
  else if constexpr (B == 1) return g_pa1;
  else return g_pa2;
}

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

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// A_MODE: 0 the FP16 operand of the activation pass, 1 raw bf16 activations (W4A16),
// 2 packed E2M1 activations (W4A4) decoded here into FP16 operands identical to the
// activation pass's (code * mu, exact).
template <int A_MODE, int C_BF16>
__global__ __launch_bounds__(64 * kWaves, 1) void k_gemm_r8(GemmArgs args) {
  constexpr int A_BF16 = A_MODE == 1;
  constexpr bool PACKED = A_MODE == 2;
  constexpr int kCp = PACKED ? 2 + kNI : kCopies;  // LDS-DMA instructions per wave and stage
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

  // ---- row-factor ratios of the FP16 operand path: f_g / f_{g+1}, the last group f_{G-1}.
  // Thread t covers row t % 128 and the t / 128-th quarter of the groups (at most 8 of 32);
  // its row factors are loaded here, all at once, and divided after the prologue copies are
  // issued, so the loads' latency is paid once and overlaps the first stages' transfers.
  constexpr int kQuarter = kMaxGroups / 4;
  const int ratio_row = threadIdx.x & (kBM - 1);
  const int g_first = (int)(threadIdx.x >> 7) * ((groups + 3) >> 2);
  float fq[kQuarter + 1];
  if (!A_BF16) {
    const int64_t f_row = min(row_begin + ratio_row, row_end - 1);
    if (PACKED) {  // the group factor is the macro-scale (1 for an all-zero group)
      const uint16_t* f = args.a_macro + f_row * groups;
#pragma unroll
      for (int j = 0; j <= kQuarter; ++j) {
        const float v = fp16_value_hw(f[min(g_first + j, groups - 1)]);
        fq[j] = v != 0.0f ? v : 1.0f;
      }
    } else {
      const float* f = args.a_scale + f_row * groups;
#pragma unroll
      for (int j = 0; j <= kQuarter; ++j) fq[j] = f[min(g_first + j, groups - 1)];
    }
  }

  // ---- buffer resources: per-lane byte offsets fixed for the whole k loop ----
  const uint16_t* a16 = static_cast<const uint16_t*>(args.a);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a16 + row_begin * args.lda), (short)0, (int)0xFFFFFFFF, kRsrcWord3);
  const int64_t a_row = min(row_begin + 16 * wave + l16, row_end - 1);  // wave w copies row block w
  const uint32_t a_voff = (uint32_t)(((a_row - row_begin) * args.lda + 8 * q) * 2);
  // packed: codes (k / 2 bytes per row) and micro-scales (k / 16 per row) of row 16 w + L % 16
  const int64_t p_row = min(row_begin + 16 * wave + l16, row_end - 1);
  const __amdgpu_buffer_rsrc_t pc_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint8_t*>(args.a) + (PACKED ? row_begin * (args.k >> 1) : 0)), (short)0,
      (int)0xFFFFFFFF, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t pm_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(PACKED ? args.a_micro + row_begin * (args.k >> 4) : args.micro), (short)0, (int)0xFFFFFFFF, kRsrcWord3);
  const uint32_t pc_voff = (uint32_t)((p_row - row_begin) * (args.k >> 1) + 16 * q);
  const uint32_t pm_voff = (uint32_t)((p_row - row_begin) * (args.k >> 4) + 4 * (q & 1));
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

  // copy J (0..3: the activation chunk of step J; 4, 5: the codes of column block J - 4)
  // of stage s into ring slot (abuf, wbuf)
  auto copy_part = [&](auto j_c, auto b_c, int s) {  // ring slot B, stage s = 2 g + h
    constexpr int J = decltype(j_c)::value, B = decltype(b_c)::value;
    uint4* wbuf = w_slot<B>();
    const bool past = s >= stages;
    const int sc = past ? 0 : s;
    const int g = sc >> 1, h = sc & 1;
    if constexpr (PACKED && J < 2) {  // this wave's rows: codes, then micro-scales
      uint4* pb = p_slot<B>() + wave * kPackChunks;
      if constexpr (J == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(past ? none : pc_rsrc, (lds_void_ptr)pb, 16, pc_voff,
                                                 (uint32_t)(sc * 64), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(past ? none : pm_rsrc, (lds_void_ptr)(pb + 64), 4, pm_voff,
                                                 (uint32_t)(sc * 8), 0, 0);
    } else if constexpr (PACKED) {
      constexpr int ni = J - 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(past ? none : w_rsrc, (lds_void_ptr)(wbuf + (wave * kNI + ni) * 64), 16,
                                               (uint32_t)lane * 16,
                                               (uint32_t)((ni * groups + g) * kTileCodeBytes + h * 1024), 0, 0);
    } else if constexpr (J < kSteps) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(past ? none : a_rsrc, (lds_void_ptr)(a_slot<B>() + (wave * kSteps + J) * 64),
                                               16, a_voff, (uint32_t)(sc * 256 + 64 * J), 0, 0);
    } else {
      constexpr int ni = J - kSteps;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(past ? none : w_rsrc, (lds_void_ptr)(wbuf + (wave * kNI + ni) * 64),
                                               16, (uint32_t)lane * 16,
                                               (uint32_t)((ni * groups + g) * kTileCodeBytes + h * 1024), 0, 0);
    }
  };
  auto copy_stage = [&](auto b_c, int s) {
    static_for<0, kCp>([&](auto j_c) { copy_part(j_c, b_c, s); });
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

  // Packed activations: lane (p, l16) of a wave decodes row l16's 32 codes of step p
  // (k = 32 p .. 32 p + 31; p = q) into the FP16 fragment chunks of lanes (q', l16), q' =
  // 0..3: codes times mu in FP16 as the activation pass forms them (the micro byte shifted
  // into FP16 bit positions is mu * 2^-8; times 256 is mu, exactly).
  uint4 pk = make_uint4(0u, 0u, 0u, 0u);
  uint32_t pk_mu = 0u, pk_m2[2] = {0u, 0u}, pk_out[4] = {0u, 0u, 0u, 0u};
  auto pk_read = [&](auto pb_c) {
    const uint4* pb = p_slot<decltype(pb_c)::value>() + wave * kPackChunks;
    pk = pb[lane];
    pk_mu = reinterpret_cast<const uint32_t*>(pb + 64)[l16 + 16 * (q >> 1)];
  };
  auto pk_scales = [&]() {
    const uint32_t sh = 16 * (q & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // micro-blocks 2 p (codes 0..15 of the piece), 2 p + 1
      const uint32_t b = (pk_mu >> (sh + 8 * h)) & 0xFFu;
      const half2_t unit = {(_Float16)256.0f, (_Float16)256.0f};
      pk_m2[h] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, (b << 7) | (b << 23)) * unit);
    }
  };
  auto pk_decode_part = [&](auto fs_c, auto w_c, auto part_c) {
    constexpr int FS = decltype(fs_c)::value, W = decltype(w_c)::value, PART = decltype(part_c)::value;
    const uint32_t word = W == 0 ? pk.x : W == 1 ? pk.y : W == 2 ? pk.z : pk.w;
    pk_out[PART] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, PART) *
                                                    __builtin_bit_cast(half2_t, pk_m2[W >> 1]));
    if constexpr (PART == 3) {
      // A plain LDS store here would make the compiler wait for every LDS-DMA copy in flight
      // (it cannot tell these slots from the copies' ring, which they never overlap); the
      // store is issued directly instead: it has no result, its operands are ALU results,
      // and the stage barrier's explicit lgkmcnt(0) covers its completion.
      typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
      const u32x4 v = {pk_out[0], pk_out[1], pk_out[2], pk_out[3]};
      const uint32_t addr = (uint32_t)(uintptr_t)(lds_void_ptr)(a_slot<FS>() + (wave * kSteps + q) * 64 + W * 16 + l16);
      asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
    }
  };

  // ---- prologue: macro-scales of groups 0 and 1, stages 0..2 in flight, stage 0 in ----
  uint32_t mw0[kNI], mw1[kNI], mw2[kNI];
  uint2 mu[kNI], mun[kNI];
  // (register loads first, in this order: the wait below then covers them too)
  load_mw(mw0, 0);
  load_mu(mu, 0);
  load_mw(mw1, min(1, groups - 1));
  __builtin_amdgcn_sched_barrier(0);
  copy_stage(std::integral_constant<int, 0>{}, 0);
  copy_stage(std::integral_constant<int, 1>{}, 1);
  copy_stage(std::integral_constant<int, 2>{}, 2);
  __builtin_amdgcn_sched_barrier(0);
  if (!A_BF16) {
    const int g_end = min(g_first + ((groups + 3) >> 2), groups);
#pragma unroll
    for (int j = 0; j < kQuarter; ++j) {
      const int g = g_first + j;
      if (g < g_end) g_sa[g * kBM + ratio_row] = g + 1 < groups ? fq[j] / fq[j + 1] : fq[j];
    }
  }
  // stage 0 landed and the ratio table written, for every wave (a plain barrier: a fence
  // would also wait for stages 1 and 2)
  __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<2 * kCp>::value);
  if constexpr (PACKED) {  // stage 0's activations: this wave's rows, decoded into slot 0
    pk_read(std::integral_constant<int, 0>{});
    pk_scales();
    static_for<0, 4>([&](auto w_c) {
      static_for<0, 4>([&](auto part_c) { pk_decode_part(std::integral_constant<int, 0>{}, w_c, part_c); });
    });
    __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<2 * kCp>::value);
  }
  asm volatile("" ::: "memory");  // (no memory access moves across the barrier)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  float4_t x[kMI][kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) x[mi][ni] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // operands of step 0
  frag af[kMI], wf[kNI];
  uint4 cw[kNI], cwn[kNI];  // code words of the current and the next stage
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) af[mi] = __builtin_bit_cast(frag, a_slot<0>()[(mi * kSteps + 0) * 64 + lane]);
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    cw[ni] = w_slot<0>()[(wave * kNI + ni) * 64 + lane];
    wf[ni] = Op::template weight_step<0>(cw[ni].x, mu[ni].x);
  }

  // factor products pp[mi][ni][i] = ratio_row * ratio_col of the boundary after the current
  // group (after the last group: the final factors); formed in four steps of the group
  // (row blocks 2j, 2j + 1 in the j-th), consumed by the rescale around the boundary
  float pp[kMI][kNI][4];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[mi][ni][i] = 1.0f;
  float rw[kNI];
  float4 ra[2], ra_nx[2];  // row ratios of the current / next product step
  uint32_t wpart[kNI][4];
  typename Op::micro_t msplat[kNI];
  const float* sa_lane = g_sa + 4 * q;  // + g * 128 + 16 mi: rows 16 mi + 4 q .. + 3


  // One MFMA step (T = 0..3 of a stage in ring slot B; H = 0 / 1 the group's first / second
  // stage) as eight regions, one per row block R, each fenced so that the compiler keeps the
  // VALU work where it is placed:
  //   - the row block's two MFMAs, then the reload of its activation fragment for the next
  //     step (this slot, or the next slot in step 3, after the barrier); in step 3, regions
  //     0..5 also issue the copies that refill this slot;
  //   - a quarter of the next step's weight decode: column block R / 4, code pair R % 4;
  //   - around a group boundary, the rescale of row blocks whose last MFMA of the group is
  //     at least two regions back: H == 1, T == 3 multiplies row blocks 0..5 (regions
  //     2..7), the next group's T == 0 row blocks 6, 7 (regions 0, 1, before their MFMAs);
  //   - in four steps per group (H == 0: T = 1, 2; H == 1: T = 0, 1), the factor products
  //     of two row blocks (regions 3..6), their row ratios loaded one step earlier (regions
  //     6, 7), and the column ratios once per group (first of the four steps, region 1).
  auto step = [&](auto b_c, auto t_c, auto h_c, auto rescale_c, int g, int s_copy) {
    constexpr int B = decltype(b_c)::value, T = decltype(t_c)::value, H = decltype(h_c)::value;
    constexpr bool RESCALE = decltype(rescale_c)::value;
    constexpr int TN = (T + 1) & 3;  // the next step (within the stage, or the next stage's first)
    constexpr bool PRE = H == 0 && T == 0 && RESCALE;
    constexpr bool POST = H == 1 && T == 3;
    constexpr bool PROD = H == 0 ? (T == 1 || T == 2) : (T == 0 || T == 1);
    constexpr int PS = H == 0 ? T - 1 : T + 2;  // which of the four product steps
    // the step before each product step loads that step's row ratios (regions 6, 7)
    constexpr bool RA_NEXT = !A_BF16 && (H == 0 ? T != 2 : T == 0);
    constexpr int PS_NEXT = H == 0 ? (T == 3 ? 2 : T) : 3;
    const uint4* anext;
    if constexpr (PACKED) anext = T < 3 ? a_slot<H>() : a_slot<1 - H>();  // FP16 stages alternate
    else anext = T < 3 ? a_slot<B>() : a_slot<(B + 1) % 3>();
    static_for<0, kMI>([&](auto r_c) {
      constexpr int R = decltype(r_c)::value;
      constexpr int NI = R / 4, P = R % 4;
      x[R][0] = Op::mfma(af[R], wf[0], x[R][0]);
      x[R][1] = Op::mfma(af[R], wf[1], x[R][1]);
      af[R] = __builtin_bit_cast(frag, anext[(R * kSteps + TN) * 64 + lane]);
      // step 3: this slot is free (the barrier before the step); the copies that refill it
      // go out one per region (all waves at once right after the barrier stall on issue)
      if constexpr (T == 3 && R < kCp)
        copy_part(std::integral_constant<int, R>{}, b_c, s_copy);
      if constexpr (T == 2 && R == 0) {  // the next stage's code words (this wave's own copies)
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni) cwn[ni] = w_slot<(B + 1) % 3>()[(wave * kNI + ni) * 64 + lane];
      }
      if constexpr (PACKED) {  // the next stage's activations: this wave's rows, decoded
        if constexpr (T == 0 && R == 5) pk_read(std::integral_constant<int, (B + 1) % 3>{});
        if constexpr (T == 0 && R == 7) pk_scales();
        if constexpr (T == 1 || T == 2)
          pk_decode_part(std::integral_constant<int, 1 - H>{}, std::integral_constant<int, 2 * (T - 1) + R / 4>{},
                         std::integral_constant<int, R % 4>{});
      }
      // next step's weights: micro-scale word of this stage (H == 0: first word), or of the
      // next stage (same group's second word, or the next group's first)
      if constexpr (P == 0) {
        const uint32_t word = T < 3 ? (H ? mu[NI].y : mu[NI].x) : (H ? mun[NI].x : mu[NI].y);
        msplat[NI] = Op::template micro_step<TN>(word);
      }
      const uint32_t code = T == 0 ? cw[NI].y : T == 1 ? cw[NI].z : T == 2 ? cw[NI].w : cwn[NI].x;
      wpart[NI][P] = Op::template weight_part<P>(code, msplat[NI]);
      if constexpr (PRE && R < 2) {
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[6 + R][ni][i] *= pp[6 + R][ni][i];
      }
      if constexpr (POST && R >= 2) {
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[R - 2][ni][i] *= pp[R - 2][ni][i];
      }
      if constexpr (RA_NEXT && R >= 6)
        ra_nx[R - 6] = *reinterpret_cast<const float4*>(sa_lane + g * kBM + 16 * (2 * PS_NEXT + R - 6));
      if constexpr (PROD) {
        if constexpr (R == 0 && !A_BF16) {
          ra[0] = ra_nx[0];
          ra[1] = ra_nx[1];
        }
        if constexpr (R == 1 && PS == 0) {  // column ratios of the boundary after group g
          const bool last = g + 1 >= groups;  // (selects, not branches)
#pragma unroll
          for (int ni = 0; ni < kNI; ++ni)
            rw[ni] = col_factor(mw0[ni]) * (last ? kUnit : __builtin_amdgcn_rcpf(col_factor(mw1[ni])));
        }
        if constexpr (R >= 3 && R <= 6) {
          constexpr int U = R - 3, MI = 2 * PS + U / 2, CI = U % 2;
          if constexpr (A_BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pp[MI][CI][i] = rw[CI];
          } else {
            pp[MI][CI][0] = ra[U / 2].x * rw[CI];
            pp[MI][CI][1] = ra[U / 2].y * rw[CI];
            pp[MI][CI][2] = ra[U / 2].z * rw[CI];
            pp[MI][CI][3] = ra[U / 2].w * rw[CI];
          }
        }
      }
      // issue order: MFMA, VALU, MFMA, LDS reads, VALU
      constexpr int kDec = (P == 0 ? (A_BF16 ? 1 : 3) : 0) + (A_BF16 ? 4 : 2);
      constexpr int kRes = ((PRE && R < 2) || (POST && R >= 2)) ? 8 : 0;
      constexpr int kProd = PROD && !A_BF16 && R >= 3 && R <= 6 ? 4 : 0;
      constexpr int kRat = PROD && R == 1 && PS == 0 ? 12 : 0;
      constexpr int kPk = PACKED ? ((T == 1 || T == 2) ? 2 : (T == 0 && R == 7) ? 8 : 0) : 0;
      constexpr int kV = kDec + kRes + kProd + kRat + kPk;
      constexpr int kDs = 1 + (T == 2 && R == 0 ? kNI : 0) + (RA_NEXT && R >= 6 ? 1 : 0) +
                          (PACKED && T == 0 && R == 5 ? 2 : 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, (kV + 1) / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kV / 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      // (keeps the decode in this step: otherwise it sinks past a loop exit that follows)
      asm volatile("" : : "v"(wpart[ni][0]), "v"(wpart[ni][1]), "v"(wpart[ni][2]), "v"(wpart[ni][3]));
      wf[ni] = __builtin_bit_cast(frag, make_uint4(wpart[ni][0], wpart[ni][1], wpart[ni][2], wpart[ni][3]));
    }
  };

  typedef std::integral_constant<bool, true> kTrue;
  typedef std::integral_constant<bool, false> kFalse;
  typedef std::integral_constant<int, 0> C0;
  typedef std::integral_constant<int, 1> C1;
  typedef std::integral_constant<int, 2> C2;
  typedef std::integral_constant<int, 3> C3;

  // Stage s in ring slot B (s % 3), H = s & 1. Before step 2 this wave's copies of stage
  // s + 1 must have landed (its code words are read in step 2): younger than them are the
  // copies of barrier s - 1 and, when s - 1 is a group's first stage, its register loads.
  // The barrier before step 3 publishes stage s + 1 to every wave and frees this slot (all
  // its reads done: lgkmcnt 0), which then receives stage s + 3.
  auto run_stage = [&](auto b_c, auto h_c, auto rescale_c, int s) {
    constexpr int H = decltype(h_c)::value;
    const int g = s >> 1;
    constexpr int kWait = kCp + (H == 1 ? kLoads : 0);
    if constexpr (PACKED) {  // the next stage's packed rows are read in step 0
      __builtin_amdgcn_s_waitcnt(kVmcntWait<kWait>::value);
      __builtin_amdgcn_sched_barrier(0);
    }
    step(b_c, C0{}, h_c, rescale_c, g, 0);
    step(b_c, C1{}, h_c, rescale_c, g, 0);
    if constexpr (!PACKED) {
      __builtin_amdgcn_s_waitcnt(kVmcntWait<kWait>::value);
      __builtin_amdgcn_sched_barrier(0);
    }
    step(b_c, C2{}, h_c, rescale_c, g, 0);
    __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<kWait>::value);
    asm volatile("" ::: "memory");  // (no memory access moves across the barrier)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (H == 0) {  // a group's first stage: micro-scales of the next group, macro of the one after
      load_mu(mun, min(g + 1, groups - 1));
      load_mw(mw2, min(g + 2, groups - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    step(b_c, C3{}, h_c, rescale_c, g, s + 3);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) cw[ni] = cwn[ni];
    if (H == 1) {  // next group: rotate the scales
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        mu[ni] = mun[ni];
        mw0[ni] = mw1[ni];
        mw1[ni] = mw2[ni];
      }
    }
  };
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

  // ---- final factors (the last group's products; row blocks 0..5 have them), store ----
  // (the store addresses are formed here: opaque copies of the lane index and first row
  // keep the compiler from computing them before the loop, where they would hold registers)
  int lane_e = lane;
  int64_t row0 = row_begin;
  asm volatile("" : "+v"(lane_e), "+s"(row0));
  const int qe = lane_e >> 4, l16e = lane_e & 15;
  const int64_t n0 = wb0 * 16;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      if (wb0 + ni >= nblocks) continue;
      const int64_t col = n0 + 16 * ni + l16e;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + 16 * mi + 4 * qe + i;
        if (r >= row_end) continue;
        // row blocks 0..5 were multiplied by the final factors in the last step
        const float v = mi < kMI - 2 ? x[mi][ni][i] : x[mi][ni][i] * pp[mi][ni][i];
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
  if (g.a_packed) {
    if (g.c_is_bf16) hipLaunchKernelGGL((k_gemm_r8<2, 1>), grid, block, lds, st, g);
    else hipLaunchKernelGGL((k_gemm_r8<2, 0>), grid, block, lds, st, g);
  } else if (g.a_is_bf16) {
    if (g.c_is_bf16) hipLaunchKernelGGL((k_gemm_r8<1, 1>), grid, block, lds, st, g);
    else hipLaunchKernelGGL((k_gemm_r8<1, 0>), grid, block, lds, st, g);
  } else {
    if (g.c_is_bf16) hipLaunchKernelGGL((k_gemm_r8<0, 1>), grid, block, lds, st, g);
    else hipLaunchKernelGGL((k_gemm_r8<0, 0>), grid, block, lds, st, g);
  }
  return hipGetLastError();
}

}  // namespace fp4lib
