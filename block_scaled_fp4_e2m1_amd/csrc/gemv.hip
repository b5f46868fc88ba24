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
// Work split: a workgroup of KS waves owns RB 16-row blocks; wave w owns a contiguous run
// of at most GPW 256-column groups; partial results meet in LDS.
#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;

namespace {

template <int RB, int GPW>
struct GemvRegs {
  uint4 code[GPW][RB][2];   // 64 codes per lane per tile
  uint4 mu[GPW][RB][2];     // 32 micro-scales: rows 4q..4q+3, blocks of parity p
  uint2 mac[GPW][RB];       // 4 macro-scales: rows 4q..4q+3
  uint4 act[GPW][8];        // activation fragment per 32-column step
};

template <int RB, int GPW, int OUT_BF16>
__global__ __launch_bounds__(1024) void k_gemv_bf16(const uint16_t* __restrict__ a, int64_t lda,
                                                    int m, int64_t k,
                                                    const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ micro,
                                                    const uint16_t* __restrict__ macro,
                                                    int64_t n, void* __restrict__ c, int64_t ldc) {
  extern __shared__ float red[];  // [KS][RB*16][8]
  const int ks = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;        // k-slot group of the operands, row quad of the output
  const int col = lane & 15;      // output column = (activation row, micro-block parity)
  const int mrow = col & 7, p = col >> 3;
  const int64_t groups = k >> 8;
  const int64_t nblocks = n >> 4;
  const int64_t nb0 = (int64_t)blockIdx.x * RB;
  const int64_t g0 = (int64_t)wave * GPW;
  const bool act_lane = ((q >> 1) == p) && (mrow < m);

  GemvRegs<RB, GPW> R;
  // ---- issue every load of this wave first (weights stream, activations hit L2) ----
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int64_t g = g0 + gi;
    const bool gv = g < groups;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const bool v = gv && (nb0 + r) < nblocks;
      const int64_t tile = (nb0 + r) * groups + g;
      if (v) {
        const uint4* cp = reinterpret_cast<const uint4*>(codes + tile * kTileCodeBytes) + lane;
        R.code[gi][r][0] = load_nt16(cp);
        R.code[gi][r][1] = load_nt16(cp + 64);
        const uint4* mp = reinterpret_cast<const uint4*>(micro + tile * kTileMicroBytes + p * 128 + q * 32);
        R.mu[gi][r][0] = mp[0];
        R.mu[gi][r][1] = mp[1];
        R.mac[gi][r] = *reinterpret_cast<const uint2*>(macro + tile * kTileMacro + 4 * q);
      } else {
        R.code[gi][r][0] = R.code[gi][r][1] = make_uint4(0, 0, 0, 0);
        R.mu[gi][r][0] = R.mu[gi][r][1] = make_uint4(0, 0, 0, 0);
        R.mac[gi][r] = make_uint2(0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (gv && act_lane)
        R.act[gi][t] = *reinterpret_cast<const uint4*>(a + mrow * lda + g * kGroup + 32 * t + 8 * q);
      else
        R.act[gi][t] = make_uint4(0, 0, 0, 0);
    }
  }

  // ---- compute ----
  float acc[RB][4];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.0f;

  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      // micro-scales of rows 4q+i, block 2t+p, as float: mus[i][t]
      float mus[4][8];
      const uint32_t mw[8] = {R.mu[gi][r][0].x, R.mu[gi][r][0].y, R.mu[gi][r][0].z, R.mu[gi][r][0].w,
                              R.mu[gi][r][1].x, R.mu[gi][r][1].y, R.mu[gi][r][1].z, R.mu[gi][r][1].w};
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)mw[d], false);
        const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)mw[d], true);
        mus[d >> 1][(d & 1) * 4 + 0] = lo[0];
        mus[d >> 1][(d & 1) * 4 + 1] = lo[1];
        mus[d >> 1][(d & 1) * 4 + 2] = hi[0];
        mus[d >> 1][(d & 1) * 4 + 3] = hi[1];
      }
      float accg[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint4 cw4 = R.code[gi][r][t >> 2];
        const uint32_t cw = (t & 3) == 0 ? cw4.x : (t & 3) == 1 ? cw4.y : (t & 3) == 2 ? cw4.z : cw4.w;
        const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 0);
        const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 1);
        const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 2);
        const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 3);
        const bf16x8_t wf = {w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, R.act[gi][t]);
        const float4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, af, zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) accg[i] = fmaf(mus[i][t], d[i], accg[i]);
      }
      const uint2 mc = R.mac[gi][r];
      const float M[4] = {fp16_value(mc.x & 0xFFFFu), fp16_value(mc.x >> 16),
                          fp16_value(mc.y & 0xFFFFu), fp16_value(mc.y >> 16)};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][i] = fmaf(M[i], accg[i], acc[r][i]);
    }
  }

  // ---- fold the two micro-block columns, then the waves, then store ----
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] += __shfl_xor(acc[r][i], 8);
  if (p == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * RB * 16 + r * 16 + 4 * q + i) * 8 + mrow] = acc[r][i];
  }
  __syncthreads();
  for (int o = threadIdx.x; o < RB * 16 * 8; o += blockDim.x) {
    const int nl = o % (RB * 16), mm = o / (RB * 16);
    if (mm >= m) continue;
    const int64_t nn = nb0 * 16 + nl;
    if (nn >= n) continue;
    float s = 0.0f;
    for (int w = 0; w < ks; ++w) s += red[(w * RB * 16 + nl) * 8 + mm];
    if (OUT_BF16)
      static_cast<uint16_t*>(c)[mm * ldc + nn] = (uint16_t)bf16_rne_bits(s);
    else
      static_cast<float*>(c)[mm * ldc + nn] = s;
  }
}

constexpr int kRB = 1;

int gemv_gpw(int64_t groups) {
  // groups per wave so that at most 16 waves cover k
  if (groups <= 16) return 1;
  if (groups <= 32) return 2;
  return 0;
}

}  // namespace

namespace fp4lib {

bool gemv_supports(int64_t m, int64_t n, int64_t k) {
  return m >= 1 && m <= 8 && (n % 16) == 0 && (k % 256) == 0 && gemv_gpw(k >> 8) > 0;
}

hipError_t launch_gemv_bf16(const uint16_t* a, int64_t lda, int64_t m, int64_t k,
                            const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                            int64_t n, void* c, int out_bf16, int64_t ldc, hipStream_t st) {
  if (!gemv_supports(m, n, k)) return hipErrorInvalidValue;
  const int64_t groups = k >> 8;
  const int gpw = gemv_gpw(groups);
  const int ks = (int)((groups + gpw - 1) / gpw);
  const int64_t nblocks = n >> 4;
  const dim3 grid((unsigned)((nblocks + kRB - 1) / kRB)), block(64 * ks);
  const size_t lds = (size_t)ks * kRB * 16 * 8 * sizeof(float);
#define FP4_GEMV(G, B) \
  hipLaunchKernelGGL((k_gemv_bf16<kRB, G, B>), grid, block, lds, st, a, lda, (int)m, k, codes, micro, macro, n, c, ldc)
  if (out_bf16) {
    if (gpw == 1) FP4_GEMV(1, 1); else FP4_GEMV(2, 1);
  } else {
    if (gpw == 1) FP4_GEMV(1, 0); else FP4_GEMV(2, 0);
  }
#undef FP4_GEMV
  return hipGetLastError();
}

}  // namespace fp4lib
