// Decode product (W4A16, m <= 8 activation rows) for gfx950.
//
// C[m, n] = sum_g M[n,g] * sum_{b in g} mu[n,b] * sum_{k in b} e2m1(W[n,k]) * A[m,k]
//
// Decoding is memory-bound (the weights are read once), so the kernel is built around
// the weight stream: the tiled layout gives every lane two 16-byte loads per 16x256 tile
// (1 KB contiguous per wave instruction). The contraction runs on
// v_mfma_f32_16x16x32_bf16 with W as the 16-row operand. Its 16 output columns are used
// as 8 activation rows x 2 micro-blocks: column (m, p) sees activation row m only in the
// 16 k-slots of micro-block p (zeros elsewhere), so each MFMA returns separate partial
// sums per micro-block. The E4M3 micro-scale is then applied to those partial sums in
// float32 and the FP16 macro-scale once per 256 columns -- the weight operand itself is
// just the E2M1 value (one hardware conversion per two codes, exact in bf16), so the
// per-element work stays far below the bandwidth budget.
//
// Work split: a workgroup of RBW x KS waves owns RBW 16-row blocks over the whole of k;
// wave (rb, ks) streams row block rb over its run of at most GPW 256-column groups. The
// activations (m <= 8 rows) are copied once per workgroup into LDS by LDS-DMA loads (no
// registers), in MFMA-fragment order, so a wave's operand read is 512 contiguous bytes.
// Operand lanes outside their micro-block read from a small zero region instead (no
// branches). The KS partial results of a row block meet in LDS. With k = 4096 and
// n = 14336 a workgroup holds 4 row blocks x 4 runs of 1024 columns (16 waves, 92 KB of
// LDS), one per CU on 224 CUs, and the weight stream of the whole launch is in flight at
// once.
//
// Issue order. A compute unit's memory pipe drains at its share of HBM bandwidth, and a
// wave cannot run past a load it has not yet issued, so loads are issued in the order
// their data is needed and computing starts before the last of them: the activation
// copies, the micro-scales (LDS-DMA) and macro-scales of the wave's run, then the codes of
// its first two groups; the codes of group g + 2 are issued once group g is computed.
#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;

namespace {

constexpr int kMaxWaves = 16;  // waves per workgroup (row blocks x waves along k)
constexpr int kMaxKS = 8;      // waves along k per row block
constexpr int kZeroBytes = 4096;  // zero region: covers the per-group operand offsets
constexpr size_t kMaxLds = 160 * 1024;  // LDS of one compute unit

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

template <int GPW>
struct GemvRegs {
  uint4 code[GPW][2];   // 64 codes per lane per tile
  uint32_t mac[GPW];    // macro-scale of the lane's weight row (low 16 bits)
};

// LDS: [A chunks: (k/8) x 8 rows x 16 B][zero region][micro-scale tiles: one 256-byte
// slot per (wave, group)][float red[KS][RBW*16][8]]
template <int kRBW, int GPW, int OUT_BF16>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemv_bf16(  // <= 128 VGPRs
    const uint16_t* __restrict__ a, int64_t lda, int m, int64_t k,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ micro,
    const uint16_t* __restrict__ macro, int64_t n, void* __restrict__ c, int64_t ldc) {
  extern __shared__ uint4 smem[];
  const int nwaves = blockDim.x >> 6;
  const int ks_count = nwaves / kRBW;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int rb = wave % kRBW, ks = wave / kRBW;
  const int q = lane >> 4;        // k-slot group of the operands, row quad of the output
  const int l16 = lane & 15;      // weight row of the lane (operand and output column)
  const int mrow = l16 & 7;       // activation row this lane feeds (operand row = p*8+m)
  const int p_op = l16 >> 3;      // micro-block parity of the operand row this lane feeds
  const int p = q >> 1;           // micro-block parity of this lane's output rows 4q..4q+3
  const int64_t groups = k >> 8;
  const int64_t nblocks = n >> 4;
  const int64_t nb = (int64_t)blockIdx.x * kRBW + rb;
  const int64_t g0 = (int64_t)ks * GPW;
  const bool act_lane = ((q >> 1) == p_op) && (mrow < m);
  const int a_chunks = (int)(k >> 3) * 8;
  uint4* zero = smem + a_chunks;
  uint4* mu_lds = zero + kZeroBytes / 16;                 // [nwaves][GPW][256 B]
  float* red = reinterpret_cast<float*>(mu_lds + nwaves * GPW * (kTileMicroBytes / 16));

  for (int i = threadIdx.x; i < kZeroBytes / 16; i += blockDim.x) zero[i] = make_uint4(0, 0, 0, 0);

  // ---- activations: LDS-DMA copies, chunk (c8, row) -> smem[c8 * 8 + row] ----
  // Each wave instruction fills 64 consecutive chunks; rows >= m copy row m-1 (those
  // chunks are never read).
  for (int s = wave; s < a_chunks / 64; s += nwaves) {
    const int i = s * 64 + lane;
    const int c8 = i >> 3, row = min(i & 7, m - 1);
    __builtin_amdgcn_global_load_lds((global_void_ptr)(a + row * lda + (int64_t)c8 * 8),
                                     (lds_void_ptr)(smem + s * 64), 16, 0, 0);
  }

  // ---- this wave's GPW tiles (consecutive in memory). A row block past the end (odd
  // block count) re-reads the last one and is not stored, so every load is
  // unconditional and every wait can be counted. Micro-scales go to LDS by DMA (one
  // 256-byte tile per instruction) and macro-scales to registers, ahead of the code
  // stream; the codes of the first kAhead groups follow. ----
  const int64_t tile0 = min(nb, nblocks - 1) * groups + g0;
  uint4* mu_wave = mu_lds + wave * GPW * (kTileMicroBytes / 16);
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
    __builtin_amdgcn_global_load_lds(
        (global_void_ptr)(micro + (tile0 + gi) * kTileMicroBytes + lane * 4),
        (lds_void_ptr)(mu_wave + gi * (kTileMicroBytes / 16)), 4, 0, 0);
  GemvRegs<GPW> R;
  const uint4* cp = reinterpret_cast<const uint4*>(codes + tile0 * kTileCodeBytes) + lane;
  const uint16_t* hp = macro + tile0 * kTileMacro + l16;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) R.mac[gi] = hp[gi * kTileMacro];
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kAhead = GPW < 2 ? GPW : 2;  // code groups in flight ahead of the compute
#pragma unroll
  for (int gi = 0; gi < kAhead; ++gi) {
    R.code[gi][0] = load_nt16(cp + gi * (kTileCodeBytes / 16));
    R.code[gi][1] = load_nt16(cp + gi * (kTileCodeBytes / 16) + 64);
  }
  // wait for the activation and micro-scale copies, the macro-scales and the zero-region
  // writes (issued first; the 2 * kAhead code loads may still be in flight), then a bare
  // barrier: LDS is coherent inside the workgroup, and no global data needs ordering here.
  // (sched_barrier keeps the code loads above the wait: the count depends on it)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<2 * kAhead>::value);
  asm volatile("" ::: "memory");  // (no memory access moves across the barrier)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // operand chunk of step t of local group gi: a_lane + gi * a_step + t * 32 chunks
  const uint4* a_lane = act_lane ? smem + (g0 * 32 + q) * 8 + mrow : zero;
  const int a_step = act_lane ? 32 * 8 : 0;

  // ---- compute. Each MFMA step is pinned in order (decode, MFMA, micro-scale FMA) so
  // the scheduler cannot front-load MFMAs and park their results; the activation
  // fragment of the next step is read one step ahead, and the codes of group gi + kAhead
  // are requested after group gi (the compiler's waits then take each group's codes as
  // they arrive). ----
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const float4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  uint4 a_next = a_lane[0];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const uint4* ag = a_lane + gi * a_step;
    // micro-scales of the lane's weight row, blocks 2t+p (t = 0..7): 8 bytes
    const uint2 mu8 = *reinterpret_cast<const uint2*>(
        reinterpret_cast<const uint8_t*>(mu_wave + gi * (kTileMicroBytes / 16)) + p * 128 + l16 * 8);
    float accg[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float2_t mu_pair;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint4 a_cur = a_next;
      if (t < 7) a_next = ag[(t + 1) * 32];
      else if (gi + 1 < GPW) a_next = (ag + a_step)[0];
      const uint4 cw4 = R.code[gi][t >> 2];
      const uint32_t cw = (t & 3) == 0 ? cw4.x : (t & 3) == 1 ? cw4.y : (t & 3) == 2 ? cw4.z : cw4.w;
      const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 0);
      const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 1);
      const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 2);
      const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 3);
      const bf16x8_t wf = {w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
      const float4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a_cur), wf,
                                                                 zero4, 0, 0, 0);
      const uint32_t mw = (t < 4) ? mu8.x : mu8.y;
      // two micro-scales per conversion
      if ((t & 3) == 0) mu_pair = __builtin_amdgcn_cvt_pk_f32_fp8((int)mw, false);
      if ((t & 3) == 2) mu_pair = __builtin_amdgcn_cvt_pk_f32_fp8((int)mw, true);
      const float mu_f = mu_pair[t & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) accg[i] = fmaf(mu_f, d[i], accg[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float M = fp16_value_hw(R.mac[gi] & 0xFFFFu);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(M, accg[i], acc[i]);
    if (gi + kAhead < GPW) {
      __builtin_amdgcn_sched_barrier(0);
      R.code[gi + kAhead][0] = load_nt16(cp + (gi + kAhead) * (kTileCodeBytes / 16));
      R.code[gi + kAhead][1] = load_nt16(cp + (gi + kAhead) * (kTileCodeBytes / 16) + 64);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- fold the two micro-block columns, then the k-split waves, then store ----
  // output rows 4q+i = (p, m = 4(q&1)+i); the two parities meet across lane ^ 32
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], 32);
  if (p == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((ks * kRBW + rb) * 16 + l16) * 8 + 4 * q + i] = acc[i];
  }
  __syncthreads();
  for (int o = threadIdx.x; o < kRBW * 16 * 8; o += blockDim.x) {
    const int nl = o % (kRBW * 16), mm = o / (kRBW * 16);
    if (mm >= m) continue;
    const int64_t nn = (int64_t)blockIdx.x * kRBW * 16 + nl;
    if (nn >= n) continue;
    const int r = nl >> 4, row = nl & 15;
    float s = 0.0f;
    for (int w = 0; w < ks_count; ++w) s += red[((w * kRBW + r) * 16 + row) * 8 + mm];
    if (OUT_BF16)
      static_cast<uint16_t*>(c)[mm * ldc + nn] = (uint16_t)bf16_rne_bits(s);
    else
      static_cast<float*>(c)[mm * ldc + nn] = s;
  }
}

// groups per wave: a divisor of the group count, at most 4 (register budget), with at
// most kMaxKS waves along k; 0 when no such split exists
int gemv_gpw(int64_t groups) {
  for (int gpw : {4, 2, 1})
    if (groups % gpw == 0 && groups / gpw <= kMaxKS && (gpw == 1 || groups / gpw >= 2)) return gpw;
  return 0;
}

}  // namespace

namespace fp4lib {

bool gemv_supports(int64_t m, int64_t n, int64_t k) {
  if (!(m >= 1 && m <= 8 && (n % 16) == 0 && (k % 256) == 0)) return false;
  const int gpw = gemv_gpw(k >> 8);
  if (gpw == 0) return false;
  return true;
}

hipError_t launch_gemv_bf16(const uint16_t* a, int64_t lda, int64_t m, int64_t k,
                            const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                            int64_t n, void* c, int out_bf16, int64_t ldc, hipStream_t st) {
  if (!gemv_supports(m, n, k)) return hipErrorInvalidValue;
  const int64_t groups = k >> 8;
  const int gpw = gemv_gpw(groups);
  const int ks = (int)((groups + gpw - 1) / gpw);
  const int64_t nblocks = n >> 4;
  // Row blocks per workgroup. Each workgroup copies all of A once, so wider workgroups
  // copy less per weight byte: four row blocks while that still keeps 3/4 of the CUs
  // busy, two while it leaves a workgroup per CU, else one (measured at k = 4096:
  // n = 12288..28672 run fastest with four, n = 8192 with two).
  auto lds_bytes = [&](int rbw) {
    return (size_t)k * 16 + kZeroBytes + (size_t)ks * rbw * gpw * kTileMicroBytes +
           (size_t)ks * rbw * 16 * 8 * sizeof(float);
  };
  const int64_t cus = device_cus();
  int rbw = 1;
  if (4 * ks <= kMaxWaves && 4 * (nblocks / 4) >= 3 * cus && lds_bytes(4) <= kMaxLds) rbw = 4;
  else if (2 * ks <= kMaxWaves && nblocks / 2 >= cus && lds_bytes(2) <= kMaxLds) rbw = 2;
  const dim3 grid((unsigned)((nblocks + rbw - 1) / rbw)), block(64 * rbw * ks);
  const size_t lds = lds_bytes(rbw);
#define FP4_GEMV(R, G, B) \
  hipLaunchKernelGGL((k_gemv_bf16<R, G, B>), grid, block, lds, st, a, lda, (int)m, k, codes, micro, macro, n, c, ldc)
#define FP4_GEMV_G(R, B) \
  do { if (gpw == 1) FP4_GEMV(R, 1, B); else if (gpw == 2) FP4_GEMV(R, 2, B); else FP4_GEMV(R, 4, B); } while (0)
#define FP4_GEMV_R(B) \
  do { if (rbw == 4) FP4_GEMV_G(4, B); else if (rbw == 2) FP4_GEMV_G(2, B); else FP4_GEMV_G(1, B); } while (0)
  if (out_bf16) FP4_GEMV_R(1); else FP4_GEMV_R(0);
#undef FP4_GEMV_R
#undef FP4_GEMV_G
#undef FP4_GEMV
  return hipGetLastError();
}

}  // namespace fp4lib
