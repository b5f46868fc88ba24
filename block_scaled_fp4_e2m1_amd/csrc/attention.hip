// Decode attention over a KV cache kept in the two-level block-scaled FP4 format on gfx950,
// and the append that quantizes new tokens into the cache.
//
// "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200": the codec
// (section "The Mathematical Breakthrough of Microscopic FP4 Scaling"). "The FP4
// Inflection: Rethinking AI Inference Architecture", section "What does this mean for
// model serving engines?": FP4 KV caches (smaller footprint, less bandwidth, new attention
// kernels). "AdaLLM Breakthrough: First NVFP4-Only Inference Engine for RTX 4090
// Unveiled": a quantized KV cache read by its own decode kernel.
//
// Codec reading: each token's key (value) vector over all KV heads, kv_heads * 128
// elements, is one codec row: E4M3 micro-scale per 16 elements, FP16 macro-scale per 256
// (a pair of heads). head_dim is 128.
//
// Cache layout (per sequence b, KV head h, T = max_tokens, a multiple of 32):
//   k_codes [b][h][T][64 B]: a token-head's 128 codes, dword 4g + s holding d = 32s + 8g ..
//           +7 (low nibble first), so that lane group g of an MFMA reads 16 contiguous bytes;
//   k_micro [b][h][T][8]      the token-head's 8 micro-scales (block d / 16);
//   k_macro [b][h/2][T]       FP16 macro-scale of the token's 256-group (head pair);
//   v_codes [b][h][T/32][128 d][16 B]: a 32-token tile transposed, byte 16d + m holding
//           slots 2m (low nibble) and 2m+1 of column d;
//   v_micro [b][h][T/32][8 blk][32 slots];
//   v_macro [b][h/2][T].
// Slot 8g + i of a tile is token 4g + i (i < 4) or 16 + 4g + i - 4 (i >= 4): the k order in
// which the P.V step meets the tile's tokens, so one dword gives a lane its 8 tokens.
//
// Attention (k_attn_decode): one workgroup per (sequence, KV head, chunk of 2048 tokens),
// 4 waves of 512 tokens, 32-token tiles copied by LDS-DMA into a two-stage ring per wave
// (the next tile lands while the current one is computed). Per tile and wave:
//   S^T = K' . Q'^T by 8 MFMA 16x16x32 f16 (rows: 16 tokens; columns: the KV head's query
//   heads, up to 16); K' = e2m1 * mu * 2^-8 is exact in FP16; Q' = q * 2^e with one power
//   of two per head (exact), so the scores are exact products accumulated in float32;
//   online softmax per head in base 2;
//   O^T += V'^T . P''^T by 16 MFMAs (rows: 16 head-dim columns; k: 32 slots); V' = e2m1 *
//   mu (per-slot micro-scales, exact in FP16), P'' = p * 2^12 * M_V[t] / M_ref
//   (M_ref the largest value macro-scale of the wave's tokens) as an FP16 pair hi + lo,
//   one MFMA each, so the weights keep ~22 bits.
// Waves are combined through LDS; chunks by k_attn_combine.
#include "fp4_device.h"
#include "fp4_kernels.h"

#include <type_traits>

using namespace fp4dev;

namespace {

constexpr int kHeadDim = 128;
constexpr int kTile = 32;          // tokens per tile
#ifndef FP4_ATTN_WAVE_TOKENS
#define FP4_ATTN_WAVE_TOKENS 512
#endif
#ifndef FP4_ATTN_STAGES
#define FP4_ATTN_STAGES 2
#endif
constexpr int kWaveTokens = FP4_ATTN_WAVE_TOKENS;  // tokens per wave
constexpr int kChunk = 4 * kWaveTokens;            // tokens per attention workgroup
constexpr int kPartial = kHeadDim + 2;  // O[128], m, l per (sequence, head, chunk)

// slot of token t (0..31) inside its tile, and back
__device__ __forceinline__ int token_slot(int t) {
  return t < 16 ? 8 * (t >> 2) + (t & 3) : 8 * ((t - 16) >> 2) + 4 + ((t - 16) & 3);
}

// --------------------------------------------------------------------------------------
// Append: one workgroup per (sequence, tile touched by the new tokens). All 256 threads
// copy the tile's V codes into LDS and back (16 dwords each in flight for 8 heads); wave 0
// quantizes the tile's new key rows and wave 1 its value rows, each one token after
// another (the V nibbles of two tokens share bytes; only wave 1 touches them).

constexpr int kAppendThreads = 256;

template <int IN_BF16>
__global__ __launch_bounds__(kAppendThreads) void k_kv_append(fp4lib::KvCacheArgs c, const void* __restrict__ k_new,
                                                  const void* __restrict__ v_new, int64_t ld,
                                                  const int32_t* __restrict__ positions, int n_new) {
  extern __shared__ uint32_t vtile[];  // kv_heads x 512 dwords: the tile's V codes
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = threadIdx.x & 63;
  const int64_t T = c.max_tokens;
  const int64_t pos0 = positions[b];
  if (pos0 < 0) return;
  const int64_t tile = pos0 / kTile + blockIdx.y;
  const int64_t t_lo = max(pos0, tile * kTile);
  const int64_t t_hi = min(min(pos0 + n_new, tile * kTile + kTile), T);
  if (t_lo >= t_hi) return;
  const int H = c.kv_heads;
  const int mv_count = H * (kHeadDim / 16);  // micro-vectors per token row
  const int64_t tiles = T / kTile;
  uint8_t* const vt8 = reinterpret_cast<uint8_t*>(vtile);

  // the tile's current V codes (tokens of the tile that are not rewritten keep theirs)
  const bool whole = t_lo == tile * kTile && t_hi == tile * kTile + kTile;
  for (int i0 = 0; i0 < H * 512; i0 += kAppendThreads * 16) {
    uint32_t tmp[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {  // independent loads first
      const int i = i0 + u * kAppendThreads + tid;
      tmp[u] = 0u;
      if (!whole && i < H * 512) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(
            c.v_codes + (((int64_t)b * H + (i >> 9)) * tiles + tile) * 2048);
        tmp[u] = src[i & 511];
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * kAppendThreads + tid;
      if (i < H * 512) vtile[i] = tmp[u];
    }
  }
  __syncthreads();

  const int which = tid >> 6;  // 0: keys, 1: values, 2-3: copy only
  if (which < 2) for (int64_t t = t_lo; t < t_hi; ++t) {
    const int64_t row = (int64_t)b * n_new + (t - pos0);
    const int slot = token_slot((int)(t - tile * kTile));
    for (int base = 0; base < mv_count; base += 64) {  // uniform trip count: shuffles stay whole
      const int mv = base + lane;
      const bool live = mv < mv_count;
      const int h = mv >> 3, j = mv & 7;  // head, micro-vector inside the head
      {
        const void* src = which ? v_new : k_new;
        float v[16];
        if (live) {
          Raw16<IN_BF16> raw;
          load_raw16<IN_BF16>(src, row * ld + (int64_t)mv * 16, raw);
          unpack16<IN_BF16>(raw, v);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = 0.0f;
        }
        uint32_t m_bits, mu_byte;
        float m_val;
        const float s = block_scales(v, 6.0f, m_bits, mu_byte, m_val);
        uint32_t w0, w1;
        e2m1_encode16(v, s, w0, w1);
        if (live) {
        const int64_t th = (int64_t)b * H + h;          // (sequence, head)
        const int64_t pair = (int64_t)b * (H / 2) + (h >> 1);
        if (which == 0) {
          uint32_t* kc = reinterpret_cast<uint32_t*>(c.k_codes + (th * T + t) * 64);
          kc[(2 * (j & 1)) * 4 + (j >> 1)] = w0;      // d = 16j .. 16j+7
          kc[(2 * (j & 1) + 1) * 4 + (j >> 1)] = w1;  // d = 16j+8 .. 16j+15
          c.k_micro[(th * T + t) * 8 + j] = (uint8_t)mu_byte;
          if ((mv & 15) == 0) c.k_macro[pair * T + t] = (uint16_t)m_bits;
        } else {
          c.v_micro[(th * tiles + tile) * 256 + j * 32 + slot] = (uint8_t)mu_byte;
          if ((mv & 15) == 0) c.v_macro[pair * T + t] = (uint16_t)m_bits;
          // 16 nibbles into 16 rows d of the transposed tile (rows are lane-private)
          uint8_t* hb = vt8 + h * 2048 + (slot >> 1);
          const int sh = (slot & 1) * 4;
          const uint8_t keep = (uint8_t)(0xF0u >> sh);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t code = ((e < 8 ? w0 : w1) >> (4 * (e & 7))) & 15u;
            uint8_t* p = hb + (16 * j + e) * 16;
            *p = (uint8_t)((*p & keep) | (code << sh));
          }
        }
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < H * 512; i += kAppendThreads) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(c.v_codes + (((int64_t)b * H + (i >> 9)) * tiles + tile) * 2048);
    dst[i & 511] = vtile[i];
  }
}

// --------------------------------------------------------------------------------------
// Attention.

__device__ __forceinline__ half8_t decode_uniform(uint32_t cw, uint32_t mu_op) {
  const half2_t m2 = __builtin_bit_cast(half2_t, mu_op);
  const half2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * m2;
  const half2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * m2;
  const half2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * m2;
  const half2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * m2;
  return half8_t{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
}

// 8 codes with one micro-scale each, the micro-scales given as FP16 pairs (slots 0-1, 2-3,
// 4-5, 6-7; every E4M3 value is an FP16 value): the products e2m1 * mu (at most 6
// significant bits, 2^-10 .. 2688) are exact in FP16
__device__ __forceinline__ half8_t decode_per_slot_h(uint32_t cw, uint4 m) {
  const half2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * __builtin_bit_cast(half2_t, m.x);
  const half2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * __builtin_bit_cast(half2_t, m.y);
  const half2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * __builtin_bit_cast(half2_t, m.z);
  const half2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * __builtin_bit_cast(half2_t, m.w);
  return half8_t{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format

// One 32-token tile of one wave in LDS, each part laid out in the order its reader lanes
// want it (the DMA lane that fetches a piece is the lane that later reads it):
//   kc[mt][l]: token 16 mt + (l & 15), K code bytes 16 (l >> 4) .. +15;
//   vc[h][l]:  V code row (column) d = 64 h + l, its 16 bytes (32 slots);
//   km:        the tile's K micro-scales, token-major (8 bytes per token);
//   vm:        the tile's V micro-scales, [block][slot].
struct TileStage {
  uint4 kc[2][64];
  uint4 vc[2][64];
  uint32_t km[64];
  uint32_t vm[64];
};

constexpr int kStages = FP4_ATTN_STAGES;  // ring depth: tiles in flight per wave
static_assert(kStages == 2 || kStages == 3, "ring depth");
constexpr int kDmaPerTile = 6;
static_assert(kDmaPerTile * (kStages - 1) < 64, "vmcnt range");

// One LDS object per ring stage (indexed by wave) and per macro row: reads of one stage
// and copies into another are then provably disjoint, so the compiler adds no wait of its
// own for the copies in flight.
__shared__ TileStage g_st0[4];
__shared__ TileStage g_st1[4];
__shared__ TileStage g_st2[kStages > 2 ? 4 : 1];
__shared__ uint16_t g_kM[4][kWaveTokens];  // macro-scales of each wave's tokens
__shared__ uint16_t g_vM[4][kWaveTokens];
// the current tile's V micro-scales of each wave as FP16 pairs, [block][slot / 2]: every
// byte is converted once per tile here instead of by each of the 16 lanes that read it
__shared__ uint32_t g_vmh[4][128];
__shared__ float g_m[4][16];
__shared__ float g_l[4][16];

template <int S>
__device__ __forceinline__ TileStage& stage_ref(int wave) {
  if constexpr (S == 0) return g_st0[wave];
  else if constexpr (S == 1 || kStages == 2) return g_st1[wave];
  else return g_st2[wave];
}

// After the token loop a wave's results O[head][128] go to its own stage 0 (heads 0..8,
// 9 x 512 bytes = one TileStage) and stage 1 (heads 9..15).
__device__ __forceinline__ float* o_row(int wave, int h) {
  return h < 9 ? reinterpret_cast<float*>(&g_st0[wave]) + h * kHeadDim
               : reinterpret_cast<float*>(&g_st1[wave]) + (h - 9) * kHeadDim;
}
static_assert(sizeof(TileStage) == 9 * kHeadDim * 4, "nine head rows per stage");

__device__ __forceinline__ float fp16_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__global__ __launch_bounds__(256, 3) void k_attn_decode(fp4lib::KvCacheArgs c, const uint16_t* __restrict__ q,
                                                     int q_heads, const int32_t* __restrict__ lengths,
                                                     float scale_log2, float* __restrict__ partial,
                                                     int chunks) {
  // chunks are the grid's slowest dimension: every sequence's first chunks are dispatched
  // before anyone's later (often partial) chunks, so the short workgroups fill the end of
  // the launch instead of delaying long ones behind them
  const int chunk = blockIdx.z, kvh = blockIdx.x, b = blockIdx.y;
  const int H = c.kv_heads;
  const int64_t T = c.max_tokens;
  const int64_t L = min((int64_t)max(lengths[b], 0), T);
  const int64_t chunk_lo = (int64_t)chunk * kChunk;
  if (chunk_lo >= L) return;  // whole workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 3;
  const int n = lane & 15, g = lane >> 4;
  const int group = q_heads / H;

  // Raw buffer resources over this (sequence, head)'s arrays: every copy below is bounded
  // by the array (reads past it return zero), so tiles past the cache can be requested.
  const int64_t th = (int64_t)b * H + kvh, pair = (int64_t)b * (H / 2) + (kvh >> 1);
  const __amdgpu_buffer_rsrc_t kc_r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.k_codes + th * T * 64), (short)0, (int)(T * 64), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t km_r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.k_micro + th * T * 8), (short)0, (int)(T * 8), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vc_r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.v_codes + th * (T / kTile) * 2048), (short)0, (int)(T * 64), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vm_r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.v_micro + th * (T / kTile) * 256), (short)0, (int)(T * 8), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t kM_r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.k_macro + pair * T), (short)0, (int)(T * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vM_r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.v_macro + pair * T), (short)0, (int)(T * 2), kRsrcWord3);

  const int64_t w_lo = chunk_lo + (int64_t)wave * kWaveTokens;
  const int64_t w_hi = min(L, w_lo + kWaveTokens);
  const int n_tiles = w_hi > w_lo ? (int)((w_hi - w_lo + kTile - 1) / kTile) : 0;

  // the query rows first (plain loads, older than every copy below)
  const bool q_real = n < group;
  uint4 qraw[4];
  {
    // padding columns load the KV head's first query row (no branch around the loads) and
    // are zeroed below
    const int qn = q_real ? n : 0;
    const uint16_t* qh = q + ((int64_t)b * q_heads + (int64_t)kvh * group + qn) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const uint4*>(qh + 32 * s + 8 * g);
  }

  // the wave's macro-scales (copies of 256 bytes), then the first kStages - 1 tiles
  const uint32_t w_lo32 = (uint32_t)w_lo;
#pragma unroll
  for (int i = 0; i < kWaveTokens / 128; ++i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kM_r, (lds_void_ptr)(g_kM[wave] + 128 * i), 4,
                                             (uint32_t)lane * 4, w_lo32 * 2 + 256 * i, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vM_r, (lds_void_ptr)(g_vM[wave] + 128 * i), 4,
                                             (uint32_t)lane * 4, w_lo32 * 2 + 256 * i, 0, 0);
  }
  const uint32_t kc_voff = (uint32_t)(n * 64 + 16 * g);
  // a tile past the wave's range gets an offset past every resource (2^31 > T * 64): the
  // copy returns zeros without touching memory and the wait counts stay fixed
  auto issue_tile = [&](TileStage& s, int it) {
    const uint32_t oob = it < n_tiles ? 0u : 0x80000000u;
    const uint32_t t0 = w_lo32 + (uint32_t)it * kTile;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kc_r, (lds_void_ptr)s.kc[mt], 16, kc_voff,
                                               (t0 * 64 + 1024 * mt) | oob, 0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vc_r, (lds_void_ptr)s.vc[h], 16, (uint32_t)lane * 16,
                                               ((t0 / kTile) * 2048 + 1024 * h) | oob, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(km_r, (lds_void_ptr)s.km, 4, (uint32_t)lane * 4, (t0 * 8) | oob, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vm_r, (lds_void_ptr)s.vm, 4, (uint32_t)lane * 4,
                                             ((t0 / kTile) * 256) | oob, 0, 0);
  };
  issue_tile(stage_ref<0>(wave), 0);
  if constexpr (kStages > 2) issue_tile(stage_ref<1>(wave), 1);

  // Q'^T operand: column n is query head kvh * group + n (zero for n >= group); k-step s,
  // lane group g holds d = 32s + 8g .. +7. One power of two per head brings max|q| into
  // [2^14, 2^15), so the bf16 -> FP16 conversion is exact.
  half8_t bq[4];
  float smul;  // score multiplier per column: scale * log2(e) * 2^8 (K' unit) / 2^e
  {
    float qv[4][8];
    float qmax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t w[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
      if (!q_real) w[0] = w[1] = w[2] = w[3] = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[s][2 * i] = __uint_as_float(w[i] << 16);
        qv[s][2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        qmax = fmaxf(qmax, fmaxf(fabsf(qv[s][2 * i]), fabsf(qv[s][2 * i + 1])));
      }
    }
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
    float sq = 1.0f;
    if (qmax > 0.0f && qmax == qmax) {
      const int ex = (int)((__float_as_uint(qmax) >> 23) & 0xFFu);  // biased exponent
      const int e = min(max(127 + 14 + 127 - max(ex, 1), 1), 254);   // 2^(14 - (ex - 127))
      sq = __uint_as_float((uint32_t)e << 23);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) bq[s][i] = (_Float16)(qv[s][i] * sq);
    smul = scale_log2 * 256.0f / sq;
  }

  // the macro copies were issued first: at most the kStages - 1 tiles behind them pending
  // (the q load above is a plain load the compiler already waited for)
  __builtin_amdgcn_s_waitcnt(kVmcntWait<kDmaPerTile * (kStages - 1)>::value);
  float mref = 0.0f;  // reference for the value macro-scales of this wave's tokens
#pragma unroll
  for (int part = 0; part < kWaveTokens / 256; ++part) {
    const int t = 256 * part + 4 * lane;  // token inside the wave
    const uint2 mm = *reinterpret_cast<const uint2*>(g_vM[wave] + t);
    const uint32_t hs[4] = {mm.x & 0xFFFFu, mm.x >> 16, mm.y & 0xFFFFu, mm.y >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (w_lo + t + i < w_hi) mref = fmaxf(mref, fp16_bits_to_float(hs[i]));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mref = fmaxf(mref, __shfl_xor(mref, o));
  if (!(mref > 0.0f) || mref != mref) mref = 1.0f;
  const float pv_mul = 4096.0f / mref;  // P'' = p * 2^12 * M_V / M_ref

  float m_run = -INFINITY, l_run = 0.0f;
  float4_t acc_o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc_o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};

  // one tile; S = it % kStages as a constant
  auto step = [&](auto s_const, int it) {
    constexpr int S = decltype(s_const)::value;
    issue_tile(stage_ref<(S + kStages - 1) % kStages>(wave), it + kStages - 1);  // stage of tile it - 1
    __builtin_amdgcn_s_waitcnt(kVmcntWait<kDmaPerTile * (kStages - 1)>::value);  // tile it has landed
    const TileStage& st = stage_ref<S>(wave);
    const int64_t t0 = w_lo + (int64_t)it * kTile;
    const int rem = (int)min(L - t0, (int64_t)kTile);  // tokens of this tile inside the sequence
    {
      // V micro-scales to FP16: lane l converts the tile's bytes 4l .. 4l + 3 (block l / 8,
      // slots 4 (l % 8) .. + 3), zeroing the slots of tokens past the length. Slots are not in
      // token order: slots 8j .. 8j + 3 hold tokens 4j .. 4j + 3, slots 8j + 4 .. 8j + 7 hold
      // tokens 16 + 4j .. 16 + 4j + 3 (the order of the scores in the P operand).
      const uint32_t vmw = st.vm[lane];
      uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vmw, 1.0f, false));
      uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vmw, 1.0f, true));
      if (rem < kTile) {
        const int s0 = 4 * (lane & 7);                           // the lane's first slot
        const int tok0 = 16 * ((s0 >> 2) & 1) + 4 * (s0 >> 3);  // its token
        p0 &= (tok0 < rem ? 0xFFFFu : 0u) | (tok0 + 1 < rem ? 0xFFFF0000u : 0u);
        p1 &= (tok0 + 2 < rem ? 0xFFFFu : 0u) | (tok0 + 3 < rem ? 0xFFFF0000u : 0u);
      }
      *reinterpret_cast<uint2*>(&g_vmh[wave][2 * lane]) = make_uint2(p0, p1);
    }

    // S^T for the two 16-token halves
    float4_t acc_s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      acc_s[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
      const uint4 kc = st.kc[mt][lane];
      const uint2 km = *reinterpret_cast<const uint2*>(&st.km[2 * (16 * mt + n)]);
      const uint32_t cw[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int blk = 2 * s + (g >> 1);  // micro-block of d = 32s + 8g
        const uint32_t mb = ((blk < 4 ? km.x : km.y) >> (8 * (blk & 3))) & 0xFFu;
        const half8_t a = decode_uniform(cw[s], (mb << 7) | (mb << 23));
        acc_s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[s], acc_s[mt], 0, 0, 0);
      }
    }
    // scores (base 2) of tokens t0 + 16 mt + 4g + i for query column n; only the last tile
    // of a sequence holds tokens past its length (wave-uniform test)
    float sc[8], vr[8];
    auto scores = [&](auto full_c) __attribute__((always_inline)) {
      constexpr bool kFull = decltype(full_c)::value;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int tk = it * kTile + 16 * mt + 4 * g;  // token index inside the wave
        const uint2 kM = *reinterpret_cast<const uint2*>(g_kM[wave] + tk);
        const uint2 vM = *reinterpret_cast<const uint2*>(g_vM[wave] + tk);
        const uint32_t kh[4] = {kM.x & 0xFFFFu, kM.x >> 16, kM.y & 0xFFFFu, kM.y >> 16};
        const uint32_t vh[4] = {vM.x & 0xFFFFu, vM.x >> 16, vM.y & 0xFFFFu, vM.y >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool live = kFull || 16 * mt + 4 * g + i < rem;
          sc[4 * mt + i] = live ? acc_s[mt][i] * (fp16_bits_to_float(kh[i]) * smul) : -INFINITY;
          vr[4 * mt + i] = live ? fp16_bits_to_float(vh[i]) * pv_mul : 0.0f;
        }
      }
    };
    if (rem == kTile) scores(std::true_type{});
    else scores(std::false_type{});
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float psum = 0.0f;
    half8_t bp, bp_lo;  // P'' as an FP16 pair: hi + lo carries ~22 bits of the float32 value
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pr = __builtin_amdgcn_exp2f(sc[i] - m_new);  // v_exp_f32; -inf gives 0
      psum += pr;
      const float x = pr * vr[i];
      const _Float16 hi = (_Float16)x;
      bp[i] = hi;
      bp_lo[i] = (_Float16)(x - (float)hi);
    }
    // rescale only when some column's running max grew (rare after the first tiles)
    if (__ballot(m_new > m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc_o[dt] *= alpha;
    }
    l_run += psum;
    m_run = m_new;

    // O^T += V'^T . P''^T, the micro-scales from the wave's FP16 table (written at the start
    // of this tile's step; in the last tile of a sequence the slots of tokens past the
    // length hold 0 there, since their cache bytes may hold anything)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      // column d = 16 dt + n is V code row 64 (dt / 4) + 16 (dt % 4) + n; its dword g holds
      // slots 8g .. 8g + 7
      const uint32_t vc = reinterpret_cast<const uint32_t*>(&st.vc[dt >> 2][16 * (dt & 3) + n])[g];
      const uint4 mh = *reinterpret_cast<const uint4*>(&g_vmh[wave][dt * 16 + 4 * g]);
      const half8_t a = decode_per_slot_h(vc, mh);
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bp, acc_o[dt], 0, 0, 0);
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bp_lo, acc_o[dt], 0, 0, 0);
    }
  };
  for (int it0 = 0; it0 < n_tiles; it0 += kStages) {
    step(std::integral_constant<int, 0>(), it0);
    if (it0 + 1 < n_tiles) step(std::integral_constant<int, 1>(), it0 + 1);
    if constexpr (kStages > 2)
      if (it0 + 2 < n_tiles) step(std::integral_constant<int, 2>(), it0 + 2);
  }
  // copies issued past the last tile must land before the ring is reused below
  __builtin_amdgcn_s_waitcnt(kVmcntWait<0>::value);

  // per-head sum over the four lane groups, then the wave's results into LDS
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const float o_mul = mref * (1.0f / 4096.0f);  // P'' unit 2^12 / M_ref (V' = e2m1 * mu)
  if (n < group) {  // into this wave's own stages (no other wave reads them before the barrier)
    if (g == 0) {
      g_m[wave][n] = m_run;
      g_l[wave][n] = l_run;
    }
    float* orow = o_row(wave, n);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * g + i] = acc_o[dt][i] * o_mul;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < group * kHeadDim; idx += 256) {
    const int h = idx / kHeadDim, d = idx % kHeadDim;
    float m = g_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) m = fmaxf(m, g_m[w][h]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = g_m[w][h] == -INFINITY ? 0.0f : exp2f(g_m[w][h] - m);
      o += f * o_row(w, h)[d];
      l += f * g_l[w][h];
    }
    float* dst = partial + (((int64_t)b * q_heads + (int64_t)kvh * group + h) * chunks + chunk) * kPartial;
    dst[d] = o;
    if (d == 0) {
      dst[kHeadDim] = m;
      dst[kHeadDim + 1] = l;
    }
  }
}

template <int OUT_BF16>
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ partial,
                                                      const int32_t* __restrict__ lengths, int q_heads,
                                                      int64_t max_tokens, int chunks, void* __restrict__ out) {
  const int bh = blockIdx.x;
  const int b = bh / q_heads;
  const int d = threadIdx.x;
  const int64_t L = min((int64_t)max(lengths[b], 0), max_tokens);
  const int used = (int)((L + kChunk - 1) / kChunk);
  const float* src = partial + (int64_t)bh * chunks * kPartial;
  // batches of 8 chunks, each batch's loads issued together, merged online
  float m = -INFINITY, o = 0.0f, l = 0.0f;
  for (int c0 = 0; c0 < used; c0 += 8) {
    float mc[8], oc[8], lc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool live = c0 + i < used;
      const float* p = src + (int64_t)(live ? c0 + i : 0) * kPartial;
      mc[i] = live ? p[kHeadDim] : -INFINITY;
      lc[i] = p[kHeadDim + 1];
      oc[i] = p[d];
    }
    float mb = mc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mb = fmaxf(mb, mc[i]);
    const float mn = fmaxf(m, mb);
    const float f = m == -INFINITY ? 0.0f : exp2f(m - mn);
    o *= f;
    l *= f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float w = mc[i] == -INFINITY ? 0.0f : exp2f(mc[i] - mn);
      o += w * oc[i];
      l += w * lc[i];
    }
    m = mn;
  }
  const float r = used > 0 ? o / l : 0.0f;
  if (OUT_BF16)
    static_cast<uint16_t*>(out)[(int64_t)bh * kHeadDim + d] = (uint16_t)bf16_rne_bits(r);
  else
    static_cast<float*>(out)[(int64_t)bh * kHeadDim + d] = r;
}

}  // namespace

namespace fp4lib {

bool kv_cache_supports(int max_tokens, int kv_heads, int head_dim) {
  return head_dim == kHeadDim && kv_heads >= 2 && kv_heads <= 32 && kv_heads % 2 == 0 &&
         max_tokens >= kTile && max_tokens % kTile == 0;
}

size_t attention_partial_bytes(int64_t n_seq, int q_heads, int64_t max_tokens) {
  const int64_t chunks = (max_tokens + kChunk - 1) / kChunk;
  return (size_t)n_seq * (size_t)q_heads * (size_t)chunks * kPartial * sizeof(float);
}

hipError_t launch_kv_append(const KvCacheArgs& c, const void* k_new, const void* v_new, int in_bf16,
                            int64_t ld, const int32_t* positions, int n_new, hipStream_t st) {
  if (!kv_cache_supports((int)c.max_tokens, c.kv_heads, kHeadDim) || n_new < 1 || c.n_seq < 1)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)c.n_seq, (unsigned)(n_new / kTile + 2)), block(kAppendThreads);
  const size_t lds = (size_t)c.kv_heads * 2048;
  if (in_bf16)
    hipLaunchKernelGGL(k_kv_append<1>, grid, block, lds, st, c, k_new, v_new, ld, positions, n_new);
  else
    hipLaunchKernelGGL(k_kv_append<0>, grid, block, lds, st, c, k_new, v_new, ld, positions, n_new);
  return hipGetLastError();
}

hipError_t launch_attention_decode(const KvCacheArgs& c, const uint16_t* q, int q_heads,
                                   const int32_t* lengths, float scale, float* partial, void* out,
                                   int out_bf16, hipStream_t st) {
  if (!kv_cache_supports((int)c.max_tokens, c.kv_heads, kHeadDim) || q_heads % c.kv_heads ||
      q_heads / c.kv_heads > 16 || c.n_seq < 1)
    return hipErrorInvalidValue;
  const int chunks = (int)((c.max_tokens + kChunk - 1) / kChunk);
  if (c.n_seq > 65535 || chunks > 65535) return hipErrorInvalidValue;  // grid y and z limits
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(k_attn_decode, dim3((unsigned)c.kv_heads, (unsigned)c.n_seq, (unsigned)chunks),
                     dim3(256), 0, st, c, q, q_heads, lengths, scale_log2, partial, chunks);
  const dim3 grid2((unsigned)(c.n_seq * q_heads)), block2(kHeadDim);
  if (out_bf16)
    hipLaunchKernelGGL(k_attn_combine<1>, grid2, block2, 0, st, partial, lengths, q_heads, c.max_tokens, chunks, out);
  else
    hipLaunchKernelGGL(k_attn_combine<0>, grid2, block2, 0, st, partial, lengths, q_heads, c.max_tokens, chunks, out);
  return hipGetLastError();
}

}  // namespace fp4lib
