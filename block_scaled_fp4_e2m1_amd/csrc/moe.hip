// Mixture-of-experts steps around the grouped product on gfx950: top-k routing with the
// permutation of routed rows, and the weighted combine of the expert outputs.
//
// "llama.cpp Put Precision Policy Inside the Model", section "One model can need more
// than one precision": the W4A4 / W4A8 routing covers mixture-of-experts products. The
// router stays float32 (ClusterBid FP4 cost guide, section "Where Does FP4 Hurt
// Accuracy?": routers are among the parts quantization hurts most).
//
// Routing (every step deterministic, no atomics):
//   1. k_route_topk: one wave per token. Each lane holds up to kMaxPerLane logits; k
//      rounds of a wave-wide argmax (larger logit first, lower expert id on ties) pick the
//      experts; weights are the softmax over the k selected logits, in float32. The wave
//      also writes the token's expert set as bit-planes, one 64-bit ballot per 64 experts
//      and plane: plane 0 marks the chosen experts, planes 1..4 hold the bits of each
//      chosen expert's rank j among the token's choices.
//   2. k_route_count: one workgroup per expert counts the tokens with its bit in plane 0.
//   3. k_route_scatter: one workgroup per expert: its first row is the sum of the counts
//      of the experts before it; tokens are visited in rounds of 256 (thread i takes token
//      256 * round + i), all plane loads of a batch of rounds in flight together; a block
//      scan of the hit bits ranks each hit in token order, and the hit writes row_token,
//      token_rows (at its rank j, read from the planes) and the expert's offsets.
// Combine: out[t, :] = sum_j weight[t, j] * y[token_rows[t, j], :], float32 in rank order
// j = 0 .. k-1, one thread per 8 consecutive columns of a token.
#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;

namespace {

constexpr int kMaxPerLane = 16;   // E <= 1024 experts
constexpr int kRouteThreads = 256;
constexpr int kPlanes = 5;        // chosen + 4 rank bits (top_k <= 16)


__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// One step of the in-row reduction: take the (value, id) of the lane that the DPP control
// names when it is better.
template <int CTRL>
__device__ __forceinline__ void dpp_better(float& bv, int& be) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
}

// Wave-wide best (value, id): DPP inside each row of 16 lanes (swap within pairs and
// quads, then rotate the row by 4 and by 8), then the four row results by readlane.
// Every lane returns the same pair.
__device__ __forceinline__ void wave_best(float& bv, int& be) {
  dpp_better<0xB1>(bv, be);   // quad_perm [1,0,3,2]
  dpp_better<0x4E>(bv, be);   // quad_perm [2,3,0,1]
  dpp_better<0x124>(bv, be);  // row_ror:4
  dpp_better<0x128>(bv, be);  // row_ror:8
  float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * row));
    const int oe = __builtin_amdgcn_readlane(be, 16 * row);
    if (better(ov, oe, rv, re)) { rv = ov; re = oe; }
  }
  bv = rv;
  be = re;
}

__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int64_t tokens,
                                                    int n_experts, int top_k,
                                                    int32_t* __restrict__ topk_ids,
                                                    float* __restrict__ topk_w,
                                                    uint32_t* __restrict__ planes) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tokens) return;  // whole waves leave together
  // NaN ranks with -inf (below every number); a per-lane mask of taken experts makes each
  // round pick a distinct valid expert whatever the logits hold, so the permutation below
  // always covers every routed row.
  const int words = (n_experts + 63) >> 6;
  float v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    const float x = e < n_experts ? logits[t * n_experts + e] : -INFINITY;
    v[i] = x == x ? x : -INFINITY;
  }
  uint32_t taken = 0;
  uint64_t slot_rank = 0;  // 4 bits per slot: the round that took the slot's expert
  // lane j keeps the j-th pick
  float my_v = -INFINITY, v_max = 0.0f;
  int my_e = 0;
  for (int j = 0; j < top_k; ++j) {
    // lane-local best (experts of this lane are lane, lane + 64, ...: increasing ids);
    // the sentinel id loses to every untaken expert, -inf ones included
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if (i < words) {  // uniform: slots past the last expert word hold nothing
        const int e = lane + 64 * i;
        if (e < n_experts && !((taken >> i) & 1u) && better(v[i], e, bv, be)) { bv = v[i]; be = e; }
      }
    }
    wave_best(bv, be);
    if (lane == j) { my_v = bv; my_e = be; }
    if (j == 0) v_max = bv;
    // the owning lane retires the chosen expert (top_k <= n_experts: one is always left)
    if ((be & 63) == lane) {
      taken |= 1u << (be >> 6);
      slot_rank |= (uint64_t)j << (4 * (be >> 6));
    }
  }
  const float ex = lane < top_k ? expf(my_v - v_max) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
  if (lane < top_k) {
    topk_ids[t * top_k + lane] = my_e;
    topk_w[t * top_k + lane] = ex / sum;
  }
  // planes as 32-bit words, token-minor: word (p, w) of token t at planes[(p * W + w) * T + t]
  // (W = 2 * words) holds bit (e & 31) for expert e = 32 w + (e & 31); p = 0 marks the
  // chosen experts, p = 1..4 hold bit p-1 of their rank. Lane l writes word l (+64, +128).
  const int w32 = 2 * words;
  uint32_t val[3] = {0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    if (i < words) {
      const uint32_t chosen = (taken >> i) & 1u;
      const uint32_t rank = (uint32_t)(slot_rank >> (4 * i)) & 15u;
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) {
        const uint64_t b = __ballot(p == 0 ? chosen : (chosen & (rank >> (p - 1))));
        const int idx = p * w32 + 2 * i;  // low half; idx + 1 the high half
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
          if (lane + 64 * pass == idx) val[pass] = (uint32_t)b;
          if (lane + 64 * pass == idx + 1) val[pass] = (uint32_t)(b >> 32);
        }
      }
    }
  }
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int idx = lane + 64 * pass;
    if (idx < kPlanes * w32) planes[(int64_t)idx * tokens + t] = val[pass];
  }
}

// block-wide sum of one int per thread (256 threads)
__device__ __forceinline__ int block_sum(int v, int* scratch) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  const int total = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  return total;
}

// Plane p's 32-bit word that holds expert e's bit, for token t (token-minor layout).
__device__ __forceinline__ uint32_t plane_word(const uint32_t* __restrict__ planes, int64_t tokens,
                                               int64_t t, int words, int p, int e) {
  return planes[((int64_t)p * 2 * words + (e >> 5)) * tokens + t];
}

__global__ __launch_bounds__(kRouteThreads) void k_route_count(const uint32_t* __restrict__ planes,
                                                               int64_t tokens, int n_experts,
                                                               int32_t* __restrict__ counts) {
  __shared__ int scratch[4];
  const int e = blockIdx.x;
  const int words = (n_experts + 63) >> 6;
  int c = 0;
#pragma unroll 8
  for (int64_t t = threadIdx.x; t < tokens; t += kRouteThreads)
    c += (int)((plane_word(planes, tokens, t, words, 0, e) >> (e & 31)) & 1u);
  c = block_sum(c, scratch);
  if (threadIdx.x == 0) counts[e] = c;
}

constexpr int kScanRounds = 16;  // rounds of 256 tokens per batch of the scatter

__global__ __launch_bounds__(kRouteThreads) void k_route_scatter(const uint32_t* __restrict__ planes,
                                                                 int64_t tokens, int top_k,
                                                                 int n_experts,
                                                                 const int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ row_token,
                                                                 int32_t* __restrict__ token_rows) {
  __shared__ int scratch[4];
  __shared__ int cnt[kScanRounds][4];          // hits per (round, wave)
  __shared__ int round_base[kScanRounds + 1];  // first row of each round
  const int e = blockIdx.x;
  const int words = (n_experts + 63) >> 6;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // first routed row of expert e
  int before = 0;
  for (int i = threadIdx.x; i < e; i += kRouteThreads) before += counts[i];
  int base = block_sum(before, scratch);
  if (threadIdx.x == 0) {
    offsets[e] = base;
    if (e == n_experts - 1) offsets[n_experts] = base + counts[e];
  }
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t b0 = 0; b0 < tokens; b0 += (int64_t)kRouteThreads * kScanRounds) {
    // every plane load of the batch first (independent): hit bit and rank per round
    uint32_t word[kScanRounds][kPlanes];
#pragma unroll
    for (int i = 0; i < kScanRounds; ++i) {
      const int64_t t = b0 + (int64_t)i * kRouteThreads + threadIdx.x;
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) word[i][p] = t < tokens ? plane_word(planes, tokens, t, words, p, e) : 0u;
    }
    uint32_t bits = 0;
    uint64_t ranks = 0;  // 4 bits per round
#pragma unroll
    for (int i = 0; i < kScanRounds; ++i) {
      bits |= ((word[i][0] >> (e & 31)) & 1u) << i;
      uint32_t j = 0;
#pragma unroll
      for (int p = 1; p < kPlanes; ++p) j |= ((word[i][p] >> (e & 31)) & 1u) << (p - 1);
      ranks |= (uint64_t)j << (4 * i);
    }
#pragma unroll
    for (int i = 0; i < kScanRounds; ++i) {
      const uint64_t bal = __ballot((bits >> i) & 1u);
      if (lane == 0) cnt[i][wave] = (int)__popcll(bal);
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the round totals
      const int tot = lane < kScanRounds ? cnt[lane][0] + cnt[lane][1] + cnt[lane][2] + cnt[lane][3] : 0;
      int incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (lane < kScanRounds) round_base[lane] = base + incl - tot;
      if (lane == kScanRounds - 1) round_base[kScanRounds] = base + incl;
    }
    __syncthreads();
    // token order = (round, wave, lane): rank = round start + earlier waves + earlier lanes
#pragma unroll
    for (int i = 0; i < kScanRounds; ++i) {
      const uint32_t hit = (bits >> i) & 1u;
      const uint64_t bal = __ballot(hit);
      if (hit) {
        int r = round_base[i] + (int)__popcll(bal & below);
        for (int w = 0; w < wave; ++w) r += cnt[i][w];
        const int64_t t = b0 + (int64_t)i * kRouteThreads + threadIdx.x;
        const int j = (int)((ranks >> (4 * i)) & 15u);
        row_token[r] = (int32_t)t;
        token_rows[t * top_k + j] = r;
      }
    }
    base = round_base[kScanRounds];
    __syncthreads();  // cnt and round_base are rewritten by the next batch
  }
}

template <int IN_BF16, int OUT_BF16>
__global__ __launch_bounds__(256) void k_moe_combine(const void* __restrict__ y, int64_t ldy,
                                                     const int32_t* __restrict__ token_rows,
                                                     const float* __restrict__ topk_w,
                                                     int64_t tokens, int top_k, int64_t hidden,
                                                     void* __restrict__ out, int64_t ldo) {
  const int64_t t = blockIdx.x;
  const int64_t c = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8;
  if (t >= tokens || c >= hidden) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const int64_t r = token_rows[t * top_k + j];
    const float w = topk_w[t * top_k + j];
    float v[8];
    if (IN_BF16) {
      const uint4 p = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y) + r * ldy + c);
      const uint32_t q[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(q[i] << 16);
        v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(y) + r * ldy + c);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, v[i], acc[i]);
  }
  if (OUT_BF16) {
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = bf16x2_rne(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + t * ldo + c) = make_uint4(q[0], q[1], q[2], q[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + t * ldo + c);
    p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

}  // namespace

namespace fp4lib {

bool route_supports(int n_experts, int top_k) {
  return n_experts >= 1 && n_experts <= 64 * kMaxPerLane && top_k >= 1 && top_k <= 16 &&
         top_k <= n_experts;
}

size_t route_workspace_bytes(int64_t tokens, int n_experts) {
  const size_t counts = ((size_t)n_experts * 4 + 255) & ~(size_t)255;
  return counts + (size_t)tokens * (size_t)((n_experts + 63) >> 6) * 8 * kPlanes;
}

hipError_t launch_moe_route(const float* logits, int64_t tokens, int n_experts, int top_k,
                            int32_t* topk_ids, float* topk_w, int32_t* offsets, int32_t* row_token,
                            int32_t* token_rows, void* workspace, hipStream_t st) {
  if (!route_supports(n_experts, top_k) || tokens < 1) return hipErrorInvalidValue;
  int32_t* counts = static_cast<int32_t*>(workspace);
  uint32_t* planes = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) +
                                                 (((size_t)n_experts * 4 + 255) & ~(size_t)255));
  hipLaunchKernelGGL(k_route_topk, dim3((unsigned)((tokens + 3) / 4)), dim3(256), 0, st, logits, tokens,
                     n_experts, top_k, topk_ids, topk_w, planes);
  hipLaunchKernelGGL(k_route_count, dim3((unsigned)n_experts), dim3(kRouteThreads), 0, st, planes,
                     tokens, n_experts, counts);
  hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)n_experts), dim3(kRouteThreads), 0, st, planes,
                     tokens, top_k, n_experts, counts, offsets, row_token, token_rows);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void* y, int in_bf16, int64_t ldy, const int32_t* token_rows,
                              const float* topk_w, int64_t tokens, int top_k, int64_t hidden,
                              void* out, int out_bf16, int64_t ldo, hipStream_t st) {
  if (hidden % 8 || tokens < 1 || tokens > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tokens, (unsigned)((hidden / 8 + 255) / 256)), block(256);
#define FP4_COMB(I, O) \
  hipLaunchKernelGGL((k_moe_combine<I, O>), grid, block, 0, st, y, ldy, token_rows, topk_w, tokens, top_k, hidden, out, ldo)
  if (in_bf16) { if (out_bf16) FP4_COMB(1, 1); else FP4_COMB(1, 0); }
  else { if (out_bf16) FP4_COMB(0, 1); else FP4_COMB(0, 0); }
#undef FP4_COMB
  return hipGetLastError();
}

}  // namespace fp4lib
