// Dense and grouped (mixture-of-experts) products on gfx950 MFMA.
//
//   C[r, n] = sum_g sA[r,g] * M_W[n,g] * sum_{k in g} A'[r,k] * (e2m1(W[n,k]) * mu_W[n,k/16])
//
// A' is the activation operand with everything but its per-256 factor sA applied: for
// W4A4 / W4A8 it is the FP16 output of the activation pass (exact), for W4A16 the raw
// bf16 activations (sA = 1). The weight operand e2m1 * mu is exact in FP16 (at most 6
// significant bits, range [2^-10, 2688]) and in bf16, so every MFMA product is exact and
// only the float32 accumulation rounds. The per-256 factors cannot be folded into the
// 16-bit operands exactly; the running sums are instead kept in units of the current
// group's factors and rescaled at each group boundary (see the kernel comment).
//
// Tiling: waves side by side along n, each owning 64 rows x 16 NI weight rows as 4 x NI
// tiles of v_mfma_f32_16x16x32_{f16,bf16}. Large dense products run 16 waves of 32
// columns (64 x 512 per workgroup, one per CU); small ones 8 waves of 16 columns (64 x 128,
// two per CU); grouped ones 8 waves of 32 columns (64 x 256, two per CU). Every form runs
// four waves per SIMD, which hides more of the pipeline's latency than two, and a wider
// workgroup copies each activation tile into LDS once for more weight columns.
// Weight fragments come straight from the tiled layout (each lane's 16 bytes are one
// MFMA operand row for four k-steps); activation fragments are 16-byte row pieces.
//
// Sensitive layers (W8A8): the same pipeline with E4M3 weight elements in their tiled
// layout and the FP16 A8 activation operand: W' = e4m3 * mu * 2^-3 is exact in FP16 as
// well, so the products stay exact; each of 8 waves then covers 16 weight rows (tile
// 64 x 128) so that the doubled weight bytes fit the same LDS buffers. "NVIDIA Ships TensorRT-LLM
// 0.16", deployment advice on outliers: FP8 kept on the most sensitive layers.
//
// Grouped form: the workgroup grid enumerates (expert, 64-row tile) pairs; each
// workgroup finds its expert by a prefix sum over the per-expert tile counts, so one
// launch covers every expert whatever the routing produced (including empty experts).
// "llama.cpp Put Precision Policy Inside the Model", section "One model can need more
// than one precision": the same W4A4/W4A8 routing serves dense and mixture-of-experts.
#include <type_traits>

#include "fp4_device.h"
#include "fp4_kernels.h"
#include "gemm_ops.h"

using namespace fp4dev;
using fp4lib::GemmArgs;

namespace {

using namespace fp4gemm;

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
// Main product kernel. Workgroup: waves side by side along n (8 or 16 by weight mode);
// tile 64 rows x 16 NI weight rows per wave; each wave owns a 64 x 16 NI block as 4 x NI
// MFMA tiles, so every weight fragment is decoded by exactly one wave. Four waves per
// SIMD (at most 128 registers): two 8-wave workgroups or one 16-wave workgroup per CU.
// The 64-row activation tile of a stage is copied once per workgroup, each wave moving
// part of one 16-row slice.
// The k loop runs in stages of half a 256-column group:
//   - the activation tile (64 x 128, 16 KB, MFMA-fragment order) and the weight codes
//     (NI row blocks x 1 KB per wave, contiguous in the tiled layout) are copied into LDS
//     by LDS-DMA, double-buffered in separate LDS objects, one stage ahead;
//   - micro-scales of the next group are prefetched into registers;
//   - per-row activation factors and the tile's macro-scales for every group are
//     copied into LDS once, at the start (dynamic LDS, sized by the group count).
// One barrier per stage: it both publishes stage s and frees the buffers of stage s-1
// for the copies of stage s+1. Inside a stage, the weight decode and LDS reads of MFMA
// step t+1 are interleaved 3 VALU : 1 MFMA with the 16 MFMAs of step t.
// Per-group factors without separate partial sums: the running sum X is kept in units
// of the current group's factor s_g = sA[row, g] * M_W[col, g]. Between groups g and
// g+1, X is multiplied by s_g / s_{g+1} (a per-row ratio times a per-column ratio; a
// zero factor counts as 1, its group contributes nothing) and the next group's MFMAs
// accumulate straight into X; at the store X is multiplied by s_last itself. The ratios
// are computed in the last MFMA step of group g (VALU otherwise idle) and each tile's
// multiply is issued just before its first MFMA of group g+1, where it waits on nothing.
// The extra float32 roundings are a few units of 2^-24 per group. (On the FP16 path the
// weight operand carries mu * 2^-8, so the column factor is 256 * M_W.)
// Each wave copies and reads only its own weight codes, so the code words and step-0
// weight fragments of stage s+1 are read and decoded during the last MFMA step of stage
// s, after a wait on the wave's own copies; only the activation tile needs the barrier.
// ---------------------------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format

constexpr int kBM = 64;              // rows per workgroup
constexpr int kStageK = 128;         // k per pipeline stage
constexpr int kAStage = kBM * kStageK * 2 / 16;  // 16-byte chunks: [mi 4][t 4][64]
constexpr int kWStage = 256 * kStageK / 2 / 16;  // 16-byte chunks: [wave 4][piece 4][64]

__shared__ uint4 g_a0[kAStage];
__shared__ uint4 g_a1[kAStage];
__shared__ uint4 g_w0[kWStage];
__shared__ uint4 g_w1[kWStage];
__shared__ uint4 g_w0x[2 * kWStage];  // the 16-wave form: [wave 16][piece 2][64]
__shared__ uint4 g_w1x[2 * kWStage];
__shared__ uint4 g_adummy[2 * 64];  // the 10-wave form: target of its two spare waves' copies
// the 10-wave form's stage ring has four slots: two more activation and weight buffers
constexpr int kW10Slots = 10 * 64;  // 16-byte chunks: [wave 10][piece 1][64]
__shared__ uint4 g_a2[kAStage];
__shared__ uint4 g_a3[kAStage];
__shared__ uint4 g_w2[kW10Slots];
__shared__ uint4 g_w3[kW10Slots];
constexpr size_t kW10StaticLds = (4 * kAStage + 2 * kWStage + 2 * kW10Slots + 2 * 64) * 16;
// the E4M3 10-wave form: two 1 KB pieces per wave, four weight slots of its own
constexpr int kW10eSlots = 10 * 2 * 64;
__shared__ uint4 g_we0[kW10eSlots];
__shared__ uint4 g_we1[kW10eSlots];
__shared__ uint4 g_we2[kW10eSlots];
__shared__ uint4 g_we3[kW10eSlots];
constexpr size_t kW10eStaticLds = (4 * kAStage + 4 * kW10eSlots + 2 * 64) * 16;

// dynamic LDS: float sa[G][64] then uint16 mw[BN/16][G][16], the latter rounded up to the
// 256-byte pieces it is copied in
size_t gemm_dynamic_lds(int groups, int bn = 256) {
  return (size_t)groups * kBM * 4 + (((size_t)(bn / 16) * groups * 16 * 2 + 255) & ~(size_t)255);
}

// Weight-side shape of the pipeline, by weight mode WM:
//   0  E2M1, 2 row blocks of 16 weight rows per wave and 8 waves (workgroup tile
//      64 x 256), one 1 KB LDS-DMA piece per row block and stage: grouped products, and
//      dense ones whose 64 x 512 tables do not fit LDS;
//   1  E4M3 (W8A8), 1 row block per wave and 8 waves (tile 64 x 128), two 1 KB pieces
//      per row block and stage, so the doubled weight bytes fit the same LDS buffers;
//   2  E2M1 narrow, 1 row block per wave and 8 waves (tile 64 x 128): twice the
//      workgroups of the wide grid and twice its waves per workgroup, for products whose
//      wide grid cannot fill the chip;
//   3  E2M1, 2 row blocks per wave and 16 waves (tile 64 x 512, one workgroup per CU):
//      one activation stage feeds twice the weight columns of mode 0; dense products
//      whose 64 x 512 grid still gives every CU a workgroup;
//   4  E2M1, 1 row block per wave and 10 waves (tile 64 x 160, one workgroup per CU):
//      narrow products whose 64 x 128 grid would give some CUs two workgroups while the
//      64 x 160 grid gives each at most one (512 x 5120: 256 tiles instead of 320);
//   5  E4M3, the same 10-wave 64 x 160 shape for W8A8 products of that kind.
template <int WM>
struct WShape {
  static constexpr bool E4M3 = WM == 1 || WM == 5;
  static constexpr int NI = (WM == 0 || WM == 3) ? 2 : 1;  // row blocks per wave
  static constexpr int WAVES = WM == 3 ? 16 : (WM == 4 || WM == 5) ? 10 : 8;  // waves per workgroup
  static constexpr int BN = 16 * NI * WAVES;               // weight rows per workgroup
  static constexpr int kTile = E4M3 ? kTile8CodeBytes : kTileCodeBytes;
  static constexpr int kPieces = E4M3 ? 2 * NI : NI;  // 1 KB LDS-DMA pieces per wave and stage
  static constexpr int kRing = WAVES == 10 ? 4 : 2;  // stage buffers (copies run kRing - 1 ahead)
};

// Activation and weight buffers of ring slot B (distinct objects, so the compiler can tell
// the slot being read from the slots being filled).
template <int B>
__device__ __forceinline__ uint4* a_slot() {
  if constexpr (B == 0) return g_a0;
  else if constexpr (B == 1) return g_a1;
  else if constexpr (B == 2) return g_a2;
  else return g_a3;
}
template <int WM, int B>
__device__ __forceinline__ uint4* w_slot() {
  if constexpr (WM == 3) {
    if constexpr (B == 0) return g_w0x;
    else return g_w1x;
  } else if constexpr (WM == 5) {
    if constexpr (B == 0) return g_we0;
    else if constexpr (B == 1) return g_we1;
    else if constexpr (B == 2) return g_we2;
    else return g_we3;
  } else if constexpr (B == 0) return g_w0;
  else if constexpr (B == 1) return g_w1;
  else if constexpr (B == 2) return g_w2;
  else return g_w3;
}

template <int A_BF16, int WM>
struct StepOperands {
  typedef typename OpTraits<A_BF16>::frag frag;
  frag af[4], wf[WShape<WM>::NI];
};

// weight fragment of row block ni for MFMA step T (0..3) of a stage, from the stage's code
// words: E2M1 dword T of word ni; E4M3 dwords 2 (T % 2), +1 of word 2 ni + T / 2
template <int A_BF16, int WM, int T>
__device__ __forceinline__ typename OpTraits<A_BF16>::frag weight_frag(const uint4 (&cw)[4], int ni, uint32_t mu_op) {
  typedef OpTraits<A_BF16> Op;
  if constexpr (WShape<WM>::E4M3) {
    const uint4 w = cw[2 * ni + (T >> 1)];
    return (T & 1) ? Op::weight8(w.z, w.w, mu_op) : Op::weight8(w.x, w.y, mu_op);
  } else {
    const uint32_t c = T == 0 ? cw[ni].x : T == 1 ? cw[ni].y : T == 2 ? cw[ni].z : cw[ni].w;
    return Op::weight(c, mu_op);
  }
}

// operands of step T (0..3) of a stage: activation fragments from LDS, weight fragments
// decoded from the stage's code words with micro-scale byte (4h+T)
template <int A_BF16, int WM, int T>
__device__ __forceinline__ void stage_operands(const uint4* abuf, const uint4 (&cw)[4],
                                               int lane, const uint2 (&mu)[4], int h,
                                               StepOperands<A_BF16, WM>& o) {
  typedef OpTraits<A_BF16> Op;
  typedef typename Op::frag frag;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) o.af[mi] = __builtin_bit_cast(frag, abuf[(mi * 4 + T) * 64 + lane]);
#pragma unroll
  for (int ni = 0; ni < WShape<WM>::NI; ++ni) {
    const uint32_t mw = h == 0 ? mu[ni].x : mu[ni].y;
    o.wf[ni] = weight_frag<A_BF16, WM, T>(cw, ni, Op::micro_operand((mw >> (8 * T)) & 0xFFu));
  }
}

template <int A_BF16, int WM>
__device__ __forceinline__ void stage_mfma(const StepOperands<A_BF16, WM>& o, float4_t (&x)[4][WShape<WM>::NI]) {
  typedef OpTraits<A_BF16> Op;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < WShape<WM>::NI; ++ni) x[mi][ni] = Op::mfma(o.af[mi], o.wf[ni], x[mi][ni]);
}

// Interleave for the MFMAs of a step with the next step's operand preparation: the four
// activation-fragment LDS reads go right after the first MFMAs (their latency then hides
// behind the rest of the step), the weight decode 3 VALU per MFMA.
template <int WM>
__device__ __forceinline__ void interleave_step() {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
  }
#pragma unroll
  for (int i = 4; i < 4 * WShape<WM>::NI; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
  }
}

// per-row (ra) and per-column (rw) ratios s_g / s_{g+1} for the boundary after group g
template <int WM>
struct Rescale {
  float ra[4][4];
  float rw[WShape<WM>::NI];
};

// Last MFMA step of a stage (step 3): its MFMAs interleaved with
//   - the code words and step-0 weight fragments of the next stage (read from the
//     wave's own LDS buffer after waiting for its own copies: at most VMCNT younger
//     loads may stay in flight), and
//   - for the last stage of a group (RATIOS), the group-boundary ratios, applied in the
//     next group's first step (the operands of step 2 are dead here).
template <int A_BF16, int WM, bool RATIOS, int VMCNT, typename RatioFn>
__device__ __forceinline__ void last_step(const StepOperands<A_BF16, WM>& o, float4_t (&x)[4][WShape<WM>::NI],
                                          RatioFn&& ratios, Rescale<WM>& r, const uint4* nwbuf, int wave,
                                          int lane, const uint32_t (&mw_next)[4], uint4 (&cw)[4],
                                          typename OpTraits<A_BF16>::frag (&wf0)[WShape<WM>::NI]) {
  typedef OpTraits<A_BF16> Op;
  constexpr int NI = WShape<WM>::NI;
  __builtin_amdgcn_s_waitcnt(kVmcntWait<VMCNT>::value);
#pragma unroll
  for (int d = 0; d < WShape<WM>::kPieces; ++d) cw[d] = nwbuf[(wave * WShape<WM>::kPieces + d) * 64 + lane];
  if (RATIOS) ratios(r);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) x[mi][ni] = Op::mfma(o.af[mi], o.wf[ni], x[mi][ni]);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    wf0[ni] = weight_frag<A_BF16, WM, 0>(cw, ni, Op::micro_operand(mw_next[ni] & 0xFFu));
#pragma unroll
  for (int i = 0; i < 4 * NI; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, RATIOS ? 5 : 3, 0);  // VALU
  }
}

// One stage: 4 MFMA steps. On entry cw holds the stage's code words and wf0 its step-0
// weight fragments; on exit they hold the next stage's. RESCALE: the first stage of a
// group multiplies each running sum by the boundary ratios r just before that tile's
// first MFMA of the group (no wait on MFMA results: those sums were finished a step
// earlier). RATIOS: the last stage of a group computes the next ratios into r.
template <int A_BF16, int WM, bool RESCALE, bool RATIOS, int VMCNT, typename RatioFn>
__device__ __forceinline__ void compute_stage(const uint4* abuf, uint4 (&cw)[4],
                                              typename OpTraits<A_BF16>::frag (&wf0)[WShape<WM>::NI], int wave,
                                              int lane, const uint2 (&mu)[4], int h,
                                              float4_t (&x)[4][WShape<WM>::NI], RatioFn&& ratios, Rescale<WM>& r,
                                              const uint4* nwbuf, const uint2 (&mu_next)[4], int h_next) {
  typedef OpTraits<A_BF16> Op;
  typedef typename Op::frag frag;
  constexpr int NI = WShape<WM>::NI;
  StepOperands<A_BF16, WM> o0, o1;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) o0.af[mi] = __builtin_bit_cast(frag, abuf[(mi * 4 + 0) * 64 + lane]);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) o0.wf[ni] = wf0[ni];
  __builtin_amdgcn_sched_barrier(0);
  if (RESCALE) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[mi][ni][i] *= A_BF16 ? r.rw[ni] : r.ra[mi][i] * r.rw[ni];
        x[mi][ni] = Op::mfma(o0.af[mi], o0.wf[ni], x[mi][ni]);
      }
    stage_operands<A_BF16, WM, 1>(abuf, cw, lane, mu, h, o1);
    __builtin_amdgcn_sched_group_barrier(0x002, A_BF16 ? 4 : 8, 0);  // VALU: tile 0's rescale
#pragma unroll
    for (int i = 0; i < 4 * NI; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, A_BF16 ? 6 : 10, 0);  // VALU
    }
  } else {
    stage_mfma<A_BF16, WM>(o0, x);
    stage_operands<A_BF16, WM, 1>(abuf, cw, lane, mu, h, o1);
    interleave_step<WM>();
  }
  __builtin_amdgcn_sched_barrier(0);
  stage_mfma<A_BF16, WM>(o1, x);
  stage_operands<A_BF16, WM, 2>(abuf, cw, lane, mu, h, o0);
  interleave_step<WM>();
  __builtin_amdgcn_sched_barrier(0);
  stage_mfma<A_BF16, WM>(o0, x);
  stage_operands<A_BF16, WM, 3>(abuf, cw, lane, mu, h, o1);
  interleave_step<WM>();
  __builtin_amdgcn_sched_barrier(0);
  uint32_t mw_next[4];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) mw_next[ni] = h_next == 0 ? mu_next[ni].x : mu_next[ni].y;
  last_step<A_BF16, WM, RATIOS, VMCNT>(o1, x, ratios, r, nwbuf, wave, lane, mw_next, cw, wf0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int A_BF16, int C_BF16, int GROUPED, int WM>
__device__ __forceinline__ void gemm_body(const GemmArgs& args) {
  static_assert(!WShape<WM>::E4M3 || (!A_BF16 && !GROUPED), "E4M3 weights: dense, FP16 activation operand");
  static_assert((WM != 3 && WM != 4 && WM != 5) || !GROUPED, "the 16- and 10-wave forms are dense");
  constexpr int NI = WShape<WM>::NI, BN = WShape<WM>::BN, kTile = WShape<WM>::kTile;
  constexpr int kWaves = WShape<WM>::WAVES;
  constexpr int kRing = WShape<WM>::kRing;
  constexpr int kSlotChunks = WM == 3 ? 2 * kWStage : WM == 4 ? kW10Slots : WM == 5 ? kW10eSlots : kWStage;
  static_assert(kWaves * WShape<WM>::kPieces * 64 <= kSlotChunks, "weight slots");
  constexpr int kPieces = WShape<WM>::kPieces;
  constexpr bool kE4M3 = WShape<WM>::E4M3;
  extern __shared__ uint8_t g_dyn[];
  const int groups = (int)(args.k >> 8);
  // the four-slot ring runs four stages (two groups) per pass: plan_gemm selects these
  // forms only for an even group count and launch_gemm refuses an odd one, so this exit
  // (which keeps a misuse from reading past the ring) is never taken
  if (kRing == 4 && (groups & 1)) return;
  const int64_t n = args.n;
  const int64_t nblocks = n >> 4;
  const int tiles_n = (int)((n + BN - 1) / BN);
  float* g_sa = reinterpret_cast<float*>(g_dyn);                               // [g][64]
  uint16_t* g_mw = reinterpret_cast<uint16_t*>(g_dyn + (size_t)groups * kBM * 4);  // [BN/16][g][16]

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

  // wave index as a wave-uniform (scalar) value: LDS-DMA destinations derive from it
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t n0 = (int64_t)tn * BN + wave * 16 * NI;  // first output column of this wave
  const int64_t nb_tile0 = w_row_base / 16 + (int64_t)tn * (BN / 16);  // first row block of the tile

  // ---- one-time tables: activation factors [g][row] and the tile's macro-scales ----
  if (!A_BF16) {  // the FP16 operand path always carries activation factors
    int64_t src_row = min(row_begin + lane, row_end - 1);  // lane = row of the tile
    if (GROUPED && args.row_token) src_row = args.row_token[src_row];
    for (int g = wave; g < groups; g += kWaves)  // one 64-row column of factors per DMA
      __builtin_amdgcn_global_load_lds((global_void_ptr)(args.a_scale + src_row * groups + g),
                                       (lds_void_ptr)(g_sa + g * kBM), 4, 0, 0);
  }
  {
    // the tile's BN/16 row blocks x G groups x 16 rows of macro-scales are contiguous
    const int mw_elems = (BN / 16) * groups * 16;  // uint16 count
    const int64_t mw_first = nb_tile0 * groups * 16;
    const int64_t mw_last = (w_row_base / 16 + nblocks) * groups * 16;  // exclusive bound
    for (int c0 = wave * 64 * 2; c0 < mw_elems; c0 += kWaves * 64 * 2) {  // 4-byte lanes = 2 entries
      const int64_t src = min(mw_first + c0 + 2 * lane, mw_last - 2);
      __builtin_amdgcn_global_load_lds((global_void_ptr)(args.macro + src), (lds_void_ptr)(g_mw + c0), 4, 0, 0);
    }
  }

  // Operand copies go through raw buffer resources: the per-lane byte offset is fixed for
  // the whole k loop and the per-stage part is a scalar offset, so the loop spends no
  // vector instructions on addresses. Reads past a resource's size return zero.
  // ---- activation copies: wave w moves row tile mi = w % 4 (16 rows); the row tile's 4
  // pieces per stage are split over its 2 (8 waves) or 4 (16 waves) waves ----
  const uint16_t* a16 = static_cast<const uint16_t*>(args.a);
  // The 10-wave form copies with waves 0..7 as the 8-wave forms do; waves 8 and 9 issue the
  // same two copies through an empty resource (zeros, no memory traffic) into a dummy
  // buffer, so that every wave runs the same code and wait counts.
  constexpr int kCopyWaves = kWaves == 10 ? 8 : kWaves;
  constexpr int kAPieces = 16 / kCopyWaves;  // per wave and stage
  const bool a_spare = kWaves == 10 && wave >= kCopyWaves;  // wave-uniform
  const int a_mi = wave & 3, a_t0 = a_spare ? 0 : (wave >> 2) * kAPieces;
  int64_t a_src_row = min(row_begin + a_mi * 16 + l16, row_end - 1);
  if (GROUPED && args.row_token) a_src_row = args.row_token[a_src_row];
  // gathered rows are addressed from the start of A (the launcher keeps A under 4 GiB);
  // otherwise from the workgroup's first row
  const int64_t a_base_row = (GROUPED && args.row_token) ? 0 : row_begin;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a16 + a_base_row * args.lda), (short)0, a_spare ? 0 : (int)0xFFFFFFFF, kRsrcWord3);
  const uint32_t a_voff = (uint32_t)(((a_src_row - a_base_row) * args.lda + 8 * q) * 2);

  // ---- weights: NI row blocks (16 columns each) per wave, consecutive in the tiled layout ----
  bool w_ok[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) w_ok[ni] = n0 / 16 + ni < nblocks;
  const int64_t wb0 = w_row_base / 16 + n0 / 16;               // the wave's first row block
  const int64_t w_blocks_left = w_row_base / 16 + nblocks - wb0;  // row blocks up to the end
  const int64_t w_tiles_left = w_blocks_left > 0 ? w_blocks_left * groups : 0;
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(args.codes + wb0 * groups * kTile), (short)0,
      (int)min(w_tiles_left * kTile, (int64_t)0xFFFFFFFF), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mu_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(args.micro + wb0 * groups * kTileMicroBytes), (short)0,
      (int)min(w_tiles_left * kTileMicroBytes, (int64_t)0xFFFFFFFF), kRsrcWord3);
  const uint32_t mu_voff = (uint32_t)((q >> 1) * 128 + l16 * 8);
  // A copy for a stage past the last one (four-slot ring) goes through empty resources:
  // zeros into a free slot, no memory traffic, the same wait counts.
  const __amdgpu_buffer_rsrc_t a_none = __builtin_amdgcn_make_buffer_rsrc((void*)a16, (short)0, 0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t w_none =
      __builtin_amdgcn_make_buffer_rsrc((void*)args.codes, (short)0, 0, kRsrcWord3);
  auto copy_stage = [&](uint4* abuf, uint4* wbuf, int s, bool past) {  // stage s = 2 g + h
    const int g = s >> 1, h = s & 1;
    const uint32_t a_soff = (uint32_t)s * (kStageK * 2);
    const __amdgpu_buffer_rsrc_t ar = past ? a_none : a_rsrc;
    const __amdgpu_buffer_rsrc_t wr = past ? w_none : w_rsrc;
#pragma unroll
    for (int tt = 0; tt < kAPieces; ++tt) {
      const int t = a_t0 + tt;
      uint4* adst = abuf + (a_mi * 4 + t) * 64;
      if constexpr (kWaves == 10) adst = a_spare ? g_adummy + tt * 64 : adst;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void_ptr)adst, 16, a_voff, a_soff + 64 * t, 0, 0);
    }
    // piece d: row block d (E2M1) or d / 2, half d % 2 of the stage's 2 KB (E4M3)
#pragma unroll
    for (int d = 0; d < kPieces; ++d) {
      const int ni = kE4M3 ? d >> 1 : d;
      const uint32_t soff = (uint32_t)((ni * groups + g) * kTile + h * (kTile / 2) + (kE4M3 ? (d & 1) * 1024 : 0));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_ptr)(wbuf + (wave * kPieces + d) * 64), 16,
                                               (uint32_t)lane * 16, soff, 0, 0);
    }
  };
  auto load_micro = [&](uint2 (&mu)[4], int g) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(mu_rsrc, mu_voff,
                                                         (uint32_t)((ni * groups + g) * kTileMicroBytes), 0);
      mu[ni] = make_uint2(v[0], v[1]);
    }
  };

  float4_t x[4][NI];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) x[mi][ni] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const float* sa_lane = g_sa + 4 * q;                               // + g*64 + mi*16: rows 4q..4q+3
  const uint16_t* mw_lane = g_mw + (wave * NI) * groups * 16 + l16;   // + (ni*G + g)*16
  // column factor M_W of group g (a zero factor counts as 1: its columns' codes are 0)
  auto col_factor = [&](int ni, int g) {
    const float v = fp16_value_hw(mw_lane[(ni * groups + g) * 16]);
    return v != 0.0f ? v : 1.0f;
  };
  // unit the weight operand leaves in the column factor: 2^8 (E2M1 * mu * 2^-8 in FP16),
  // 8 (E4M3 * mu * 2^-3), 1 on the bf16 path
  constexpr float kUnit = kE4M3 ? OpTraits<0>::kMicroUnit8 : OpTraits<A_BF16>::kMicroUnit;
  // ratios s_g / s_{g+1} for the boundary after group g, with s_G = 1: after the last
  // group the "ratio" is the final factor itself. Row ratios come from the table built
  // in the prologue; the weight operand's unit cancels except in the final factor.
  auto ratios_after = [&](int g, Rescale<WM>& r) {
    const bool last = g + 1 >= groups;
    if constexpr (kRing == 4) {
      // The tables live in dynamic LDS, which the compiler cannot tell apart from the
      // ring's static slots: a plain read here made it wait for every copy in flight
      // (vmcnt 0, the copies issued three stages ahead included). These reads are
      // issued as one block that waits for its own results (lgkmcnt 0) instead; the
      // tables were complete before the loop (prologue wait and barrier).
      static_assert(NI == 1, "one row block per wave in the four-slot forms");
      const int gn = min(g + 1, groups - 1);
      const uint32_t mw_a = (uint32_t)(uintptr_t)(lds_void_ptr)(mw_lane + g * 16);
      const uint32_t mw_b = (uint32_t)(uintptr_t)(lds_void_ptr)(mw_lane + gn * 16);
      uint32_t h0, h1;
      if constexpr (!A_BF16) {
        const uint32_t sa = (uint32_t)(uintptr_t)(lds_void_ptr)(sa_lane + g * kBM);
        float4_t v0, v1, v2, v3;
        asm volatile(
            "ds_read_b128 %0, %6\n\tds_read_b128 %1, %6 offset:64\n\tds_read_b128 %2, %6 offset:128\n\t"
            "ds_read_b128 %3, %6 offset:192\n\tds_read_u16 %4, %7\n\tds_read_u16 %5, %8\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(h0), "=&v"(h1)
            : "v"(sa), "v"(mw_a), "v"(mw_b));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r.ra[0][i] = v0[i];
          r.ra[1][i] = v1[i];
          r.ra[2][i] = v2[i];
          r.ra[3][i] = v3[i];
        }
      } else {
        asm volatile("ds_read_u16 %0, %2\n\tds_read_u16 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(h0), "=&v"(h1)
                     : "v"(mw_a), "v"(mw_b));
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int i = 0; i < 4; ++i) r.ra[mi][i] = 1.0f;
      }
      const float f0 = fp16_value_hw(h0), f1 = fp16_value_hw(h1);  // a zero factor counts as 1
      const float c0 = f0 != 0.0f ? f0 : 1.0f, c1 = f1 != 0.0f ? f1 : 1.0f;
      r.rw[0] = c0 * (last ? kUnit : __builtin_amdgcn_rcpf(c1));
      return;
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      r.rw[ni] = last ? col_factor(ni, g) * kUnit
                      : col_factor(ni, g) * __builtin_amdgcn_rcpf(col_factor(ni, g + 1));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      float4 v = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
      if (!A_BF16) v = *reinterpret_cast<const float4*>(sa_lane + g * kBM + mi * 16);
      r.ra[mi][0] = v.x; r.ra[mi][1] = v.y; r.ra[mi][2] = v.z; r.ra[mi][3] = v.w;
    }
  };

  uint2 mu_cur[4], mu_nxt[4];
  const int stages = 2 * groups;
  // Two slots: stage 0, its micro-scales, wait for all. Four slots: stage 0, the
  // micro-scales, stages 1 and 2, wait for all but stage 2, so that every stage later
  // finds the same loads younger than the copies it waits for (see run_stage).
  copy_stage(a_slot<0>(), w_slot<WM, 0>(), 0, false);
  __builtin_amdgcn_sched_barrier(0);
  load_micro(mu_cur, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kRing == 4) {
    copy_stage(a_slot<1>(), w_slot<WM, 1>(), 1, false);
    copy_stage(a_slot<2>(), w_slot<WM, 2>(), 2, false);
  }
  // stage 0's code words and step-0 weight fragments (the wave's own copies)
  uint4 cw[4];
  typename OpTraits<A_BF16>::frag wf0[NI];
  __builtin_amdgcn_s_waitcnt(kVmcntWait<kRing == 4 ? kAPieces + kPieces : 0>::value);
  if (!A_BF16) {
    // row factors [g][row] -> ratios f_g / f_{g+1} (last group: f_{G-1}), in place; each
    // lane of wave 0 walks one row upwards in g, reading f_{g+1} before it is replaced
    __syncthreads();  // every wave's factor copies have landed
    if (wave == 0) {
      float f = g_sa[lane];
      for (int g = 0; g + 1 < groups; ++g) {
        const float fn = g_sa[(g + 1) * kBM + lane];
        g_sa[g * kBM + lane] = f / fn;
        f = fn;
      }
    }
  }
#pragma unroll
  for (int d = 0; d < kPieces; ++d) cw[d] = w_slot<WM, 0>()[(wave * kPieces + d) * 64 + lane];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    wf0[ni] = weight_frag<A_BF16, WM, 0>(cw, ni, OpTraits<A_BF16>::micro_operand(mu_cur[ni].x & 0xFFu));

  // stage s in buffers (s & 1): the barrier publishes its activation tile (every wave's
  // copies are complete) and frees the other buffers, which then receive stage s + 1
  // while stage s computes. H = s & 1 is a compile-time constant: the second stage of
  // every group ends with the group-boundary rescale.
  // boundary ratios carried from the last stage of a group into the first of the next
  // (1 before the first group; after the last group they are the final factors)
  Rescale<WM> resc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) resc.ra[i][j] = 1.0f;
  }
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) resc.rw[ni] = 1.0f;
  // Stage s reads ring slot B = s % kRing and first issues the copies of stage
  // s + kRing - 1 into the slot stage s - 1 used (free after the barrier). Its last step
  // waits for stage s + 1's copies, with these loads younger than them:
  //   two slots:  the micro-scale loads of stage s (H == 0 stages only), issued after
  //               the copies;
  //   four slots: the copies of stages s + 2 and s + 3, and the micro-scale loads of
  //               the one H == 0 stage among s - 1 and s, issued before that stage's
  //               copies (so the next group's micro-scales never wait behind a stage
  //               of copies).
  // The four-slot barrier is a bare s_barrier after lgkmcnt 0: every wave has waited
  // for its own copies of stage s (previous stage's last step), and its reads of the
  // slot about to be refilled are complete. __syncthreads() would add a workgroup fence,
  // which waits for the copies still in flight, two and three stages ahead.
  auto run_stage = [&](auto h_const, auto b_const, int s) {
    constexpr int H = decltype(h_const)::value, B = decltype(b_const)::value;
    constexpr int kWait = kRing == 2 ? (H == 0 ? NI : 0) : 2 * (kAPieces + kPieces) + NI;
    // (the micro-scale loads are unconditional in H == 0 stages, the last group
    // re-reading its own, so that the count of loads younger than the awaited copies is
    // fixed; it holds because every iteration runs this same code: in a separately
    // compiled last iteration these loads would be dead, the compiler would drop them,
    // and the wait would let copies through unfinished)
    if constexpr (kRing == 2) {
      __syncthreads();
      if (s + 1 < stages) copy_stage(a_slot<(B + 1) % 2>(), w_slot<WM, (B + 1) % 2>(), s + 1, false);
      __builtin_amdgcn_sched_barrier(0);
      if (H == 0) load_micro(mu_nxt, min((s >> 1) + 1, groups - 1));
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<63>::value);
      asm volatile("" ::: "memory");  // (no memory access moves across the barrier)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (H == 0) load_micro(mu_nxt, min((s >> 1) + 1, groups - 1));
      __builtin_amdgcn_sched_barrier(0);
      copy_stage(a_slot<(B + 3) % 4>(), w_slot<WM, (B + 3) % 4>(), min(s + 3, stages - 1), s + 3 >= stages);
    }
    __builtin_amdgcn_sched_barrier(0);
    // next stage: same group (H == 0: micro-scale word 1 of mu_cur) or the next group
    // (H == 1: word 0 of mu_nxt)
    compute_stage<A_BF16, WM, H == 0, H == 1, kWait>(
        a_slot<B>(), cw, wf0, wave, lane, mu_cur, H, x, [&](Rescale<WM>& rr) { ratios_after(s >> 1, rr); },
        resc, w_slot<WM, (B + 1) % kRing>(), H == 0 ? mu_cur : mu_nxt, 1 - H);
    if (H == 1) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) mu_cur[ni] = mu_nxt[ni];
    }
  };
  typedef std::integral_constant<int, 0> C0;
  typedef std::integral_constant<int, 1> C1;
  if constexpr (kRing == 2) {
    for (int s = 0; s < stages; s += 2) {
      run_stage(C0{}, C0{}, s);
      run_stage(C1{}, C1{}, s + 1);
    }
  } else {
    for (int s = 0; s < stages; s += 4) {  // stages % 4 == 0 (checked above)
      run_stage(C0{}, C0{}, s);
      run_stage(C1{}, C1{}, s + 1);
      run_stage(C0{}, std::integral_constant<int, 2>{}, s + 2);
      run_stage(C1{}, std::integral_constant<int, 3>{}, s + 3);
    }
  }

  // the ring's last copies (zeros from empty resources) are complete before the
  // workgroup's LDS can be handed to another
  __builtin_amdgcn_s_waitcnt(kVmcntWait<0>::value);

  // ---- apply the final factors, store ----
  // The stores go through a raw buffer over the tile's valid rows: each store's row offset
  // is a scalar, the lane's offset is fixed, and a row at or past row_end lies outside the
  // buffer, where the hardware drops the store (no per-element branch or 64-bit address;
  // the boundary keeps 128 x ldc x 4 bytes below 2^31).
  constexpr int kES = C_BF16 ? 2 : 4;
  const int64_t tile_rows = min((int64_t)kBM, row_end - row_begin);
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char*>(args.c) + row_begin * args.ldc * kES, (short)0, (int)(tile_rows * args.ldc * kES),
      kRsrcWord3);
  const uint32_t c_voff = (uint32_t)(((int64_t)(4 * q) * args.ldc + n0 + l16) * kES);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      if (!w_ok[ni]) continue;
#pragma unroll
      for (int i = 0; i < 4; i += 2) {  // rows 4q + i and 4q + i + 1: one bf16 conversion
        const uint32_t c_soff = (uint32_t)(((int64_t)(16 * mi + i) * args.ldc + 16 * ni) * kES);
        const uint32_t c_soff1 = c_soff + (uint32_t)(args.ldc * kES);
        const float v0 = x[mi][ni][i] * (A_BF16 ? resc.rw[ni] : resc.ra[mi][i] * resc.rw[ni]);
        const float v1 = x[mi][ni][i + 1] * (A_BF16 ? resc.rw[ni] : resc.ra[mi][i + 1] * resc.rw[ni]);
        if (C_BF16) {
          const uint32_t b = bf16x2_rne(v0, v1);
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)b, c_rsrc, c_voff, c_soff, 0);
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(b >> 16), c_rsrc, c_voff, c_soff1, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v0), c_rsrc, c_voff, c_soff, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v1), c_rsrc, c_voff, c_soff1, 0);
        }
      }
    }
  }
}
// Kernels: the 8-wave forms run two workgroups per CU, the 16-wave form one; either way
// four waves per SIMD. The 10-wave form runs one workgroup per CU (three waves on two
// SIMDs, two on the others).
template <int A_BF16, int C_BF16, int GROUPED, int WM>
__global__ __launch_bounds__(512, 2) void k_gemm(GemmArgs args) {
  gemm_body<A_BF16, C_BF16, GROUPED, WM>(args);
}

template <int A_BF16, int C_BF16>
__global__ __launch_bounds__(1024, 1) void k_gemm_w16(GemmArgs args) {
  gemm_body<A_BF16, C_BF16, 0, 3>(args);
}

template <int A_BF16, int C_BF16>
__global__ __launch_bounds__(640, 1) void k_gemm_w10(GemmArgs args) {
  gemm_body<A_BF16, C_BF16, 0, 4>(args);
}

template <int C_BF16>
__global__ __launch_bounds__(640, 1) void k_gemm_w10e(GemmArgs args) {
  gemm_body<0, C_BF16, 0, 5>(args);
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

bool gemm_supports(int64_t k) { return gemm_dynamic_lds((int)(k >> 8)) <= 64 * 1024; }

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    cus[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0 ? v : 256;
  }
  return cus[dev];
}

// Kernel form and grid of a product (the selection launch_gemm makes); false when the
// shape is outside what the kernels cover (k tables over the LDS budget, grid too large).
struct GemmPlan {
  bool r8, narrow, wide16, w10;
  int64_t bn, blocks;
  unsigned threads;
  size_t lds;
};

static bool plan_gemm(int64_t m, int64_t n, int64_t k, bool grouped, int n_experts, bool e4m3, GemmPlan& p) {
  if (m < 1 || n < 16 || n % 16 || !gemm_supports(k)) return false;
  if (e4m3 && grouped) return false;
  if (grouped && n_experts < 1) return false;
  int64_t tiles_m;
  if (grouped) tiles_m = (m + kBM - 1) / kBM + n_experts;  // upper bound
  else tiles_m = (m + kBM - 1) / kBM;
  const int64_t cus = device_cus();
  // dense E2M1 products whose 128 x 256 tiles give every CU a workgroup take the
  // 128-row-wave form (a decoded weight fragment feeds 8 MFMAs instead of 4)
  p.r8 = !e4m3 && !grouped && gemm_r8_supports(m, n, k) && ((m + 127) / 128) * ((n + 255) / 256) >= cus;
  if (p.r8) {
    p.narrow = p.wide16 = p.w10 = false;
    p.bn = 256;
    p.blocks = ((m + 127) / 128) * ((n + 255) / 256);
    p.threads = 512;
    p.lds = 0;
    return p.blocks <= 0x7FFFFFFF;
  }
  // dense E2M1 products whose 64 x 256 tiles cannot give every CU two workgroups take the
  // narrow 64 x 128 tile
  p.narrow = !e4m3 && !grouped && tiles_m * ((n + WShape<0>::BN - 1) / WShape<0>::BN) < 2 * cus;
  // dense E2M1 products whose 64 x 512 tiles still give every CU a workgroup take the
  // 16-wave form: four waves per SIMD, one activation stage for twice the weight columns
  p.wide16 = !e4m3 && !grouped && !p.narrow &&
             tiles_m * ((n + WShape<3>::BN - 1) / WShape<3>::BN) >= cus &&
             gemm_dynamic_lds((int)(k >> 8), WShape<3>::BN) <= 160 * 1024 - 96 * 1024;
  // narrow products take the 10-wave 64 x 160 form when it puts fewer weight columns on
  // the busiest SIMD: 48 per 64 x 160 tile on a CU (3 waves of 16), 32 per 64 x 128
  // tile (two workgroups of 8 waves share a CU); W8A8 products, whose E4M3 tile is
  // always 64 x 128, likewise, with weight slots of twice the size. The form's four-slot
  // ring runs four stages (two groups) per pass: an even group count is a precondition.
  p.w10 = false;
  if (p.narrow || (e4m3 && !grouped)) {
    const int64_t t128 = tiles_m * ((n + WShape<2>::BN - 1) / WShape<2>::BN);
    const int64_t t160 = tiles_m * ((n + WShape<4>::BN - 1) / WShape<4>::BN);
    const int groups = (int)(k >> 8);
    const size_t lds = (e4m3 ? kW10eStaticLds : kW10StaticLds) + gemm_dynamic_lds(groups, WShape<4>::BN);
    p.w10 = 48 * ((t160 + cus - 1) / cus) < 32 * ((t128 + cus - 1) / cus) && groups % 2 == 0 &&
            lds <= 160 * 1024;
  }
  p.bn = p.w10 ? WShape<4>::BN : e4m3 ? WShape<1>::BN : p.narrow ? WShape<2>::BN
         : p.wide16 ? WShape<3>::BN : WShape<0>::BN;
  p.blocks = tiles_m * ((n + p.bn - 1) / p.bn);
  if (p.blocks <= 0 || p.blocks > 0x7FFFFFFF) return false;
  p.threads = p.wide16 ? 1024 : p.w10 ? 640 : 512;
  p.lds = gemm_dynamic_lds((int)(k >> 8), (int)p.bn);
  return true;
}

bool gemm_packed_a4(int64_t m, int64_t n, int64_t k) {
  GemmPlan p;
  return plan_gemm(m, n, k, false, 0, false, p) && p.r8;
}

bool gemm_plan_ok(int64_t m, int64_t n, int64_t k, int grouped, int n_experts, int w_e4m3) {
  GemmPlan p;
  return plan_gemm(m, n, k, grouped != 0, n_experts, w_e4m3 != 0, p);
}

const char* gemm_kernel_name(int64_t m, int64_t n, int64_t k, int grouped, int n_experts, int w_e4m3) {
  GemmPlan p;
  if (!plan_gemm(m, n, k, grouped != 0, n_experts, w_e4m3 != 0, p)) return nullptr;
  if (p.r8) return "k_gemm_r8 (128 x 256, 8 waves of 128 x 32)";
  if (p.wide16) return "k_gemm_w16 (64 x 512, 16 waves)";
  if (p.w10) return w_e4m3 ? "k_gemm_w10e (64 x 160, 10 waves, E4M3)" : "k_gemm_w10 (64 x 160, 10 waves)";
  if (w_e4m3) return "k_gemm (64 x 128, 8 waves, E4M3)";
  if (p.narrow) return "k_gemm (64 x 128, 8 waves)";
  return grouped ? "k_gemm (64 x 256, 8 waves, grouped)" : "k_gemm (64 x 256, 8 waves)";
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.w_e4m3 && g.a_is_bf16) return hipErrorInvalidValue;
  GemmPlan p;
  if (!plan_gemm(g.m, g.n, g.k, g.expert_offsets != nullptr, g.n_experts, g.w_e4m3 != 0, p))
    return hipErrorInvalidValue;
  if (p.r8) return launch_gemm_r8(g, st);
  if (g.a_packed) return hipErrorInvalidValue;  // packed activations: the 128-row-wave form only
  const bool narrow = p.narrow, wide16 = p.wide16, w10 = p.w10;
  const dim3 grid((unsigned)p.blocks), block(p.threads);
  const size_t lds = p.lds;
#define FP4_GEMM(A, C, G, W) hipLaunchKernelGGL((k_gemm<A, C, G, W>), grid, block, lds, st, g)
  const int grouped = g.expert_offsets != nullptr;
  if (wide16) {
#define FP4_GEMM16(A, C) hipLaunchKernelGGL((k_gemm_w16<A, C>), grid, block, lds, st, g)
    if (g.a_is_bf16) { if (g.c_is_bf16) FP4_GEMM16(1, 1); else FP4_GEMM16(1, 0); }
    else { if (g.c_is_bf16) FP4_GEMM16(0, 1); else FP4_GEMM16(0, 0); }
#undef FP4_GEMM16
  } else if (w10 && (g.k >> 8) % 2) {
    // the four-slot ring's precondition (plan_gemm never selects it for an odd group count;
    // refused here too rather than launched into the kernel's guard)
    return hipErrorInvalidValue;
  } else if (w10 && g.w_e4m3) {
    if (g.c_is_bf16) hipLaunchKernelGGL((k_gemm_w10e<1>), grid, block, lds, st, g);
    else hipLaunchKernelGGL((k_gemm_w10e<0>), grid, block, lds, st, g);
  } else if (w10) {
#define FP4_GEMM10(A, C) hipLaunchKernelGGL((k_gemm_w10<A, C>), grid, block, lds, st, g)
    if (g.a_is_bf16) { if (g.c_is_bf16) FP4_GEMM10(1, 1); else FP4_GEMM10(1, 0); }
    else { if (g.c_is_bf16) FP4_GEMM10(0, 1); else FP4_GEMM10(0, 0); }
#undef FP4_GEMM10
  } else if (g.w_e4m3) {
    if (g.c_is_bf16) FP4_GEMM(0, 1, 0, 1); else FP4_GEMM(0, 0, 0, 1);
  } else if (narrow) {
    if (g.a_is_bf16) { if (g.c_is_bf16) FP4_GEMM(1, 1, 0, 2); else FP4_GEMM(1, 0, 0, 2); }
    else { if (g.c_is_bf16) FP4_GEMM(0, 1, 0, 2); else FP4_GEMM(0, 0, 0, 2); }
  } else if (g.a_is_bf16) {
    if (g.c_is_bf16) { if (grouped) FP4_GEMM(1, 1, 1, 0); else FP4_GEMM(1, 1, 0, 0); }
    else { if (grouped) FP4_GEMM(1, 0, 1, 0); else FP4_GEMM(1, 0, 0, 0); }
  } else {
    if (g.c_is_bf16) { if (grouped) FP4_GEMM(0, 1, 1, 0); else FP4_GEMM(0, 1, 0, 0); }
    else { if (grouped) FP4_GEMM(0, 0, 1, 0); else FP4_GEMM(0, 0, 0, 0); }
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
