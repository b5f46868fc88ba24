// Layout repack of a quantized tensor between the canonical (interchange) layout and the
// tiled layout the product kernels read, in either direction, for E2M1 and E4M3
// elements. It is an integer permutation of the code bytes, the E4M3 micro-scales and
// the FP16 macro-scales: no value is decoded, so repacking is exact and the two
// directions are inverse to each other. (The format: "NVIDIA Ships TensorRT-LLM 0.16:
// Native FP4 Quantization for Blackwell B200", section "The Mathematical Breakthrough of
// Microscopic FP4 Scaling", items 1-2; the tiled layout is this library's own, matched to
// the MFMA operand order.)
//
// Work mapping: a tile is 16 rows x 256 columns (2048 code bytes for E2M1, 4096 for
// E4M3). A 256-thread workgroup permutes 4 KB of codes per pass (two E2M1 tiles or one
// E4M3 tile): every thread loads one 16-byte chunk of the source tile in the source
// order (each row's run of the tile is whole 128-byte lines), the chunks meet in LDS, and
// every thread gathers one 16-byte chunk of the destination from LDS and stores it, so
// both global sides are 16-byte coalesced. The first 16 threads of each tile move its
// micro-scales (one row each: 16 bytes canonical, two 8-byte runs of even and odd blocks
// tiled) and its macro-scales (one 16-bit value each).
// HBM-bound: it reads and writes every byte of the tensor once.
#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;

namespace {

constexpr int kRepackThreads = 256;

// byte b of the 16 in (x, y, z, w)
__device__ __forceinline__ uint32_t byte_of(const uint4& v, int b) {
  const uint32_t w = b < 4 ? v.x : b < 8 ? v.y : b < 12 ? v.z : v.w;
  return (w >> (8 * (b & 3))) & 0xFFu;
}

template <int E4M3, int TO_TILED>
__global__ __launch_bounds__(kRepackThreads) void k_repack(const uint8_t* __restrict__ src_codes,
                                                           const uint8_t* __restrict__ src_micro,
                                                           const uint16_t* __restrict__ src_macro,
                                                           uint8_t* __restrict__ dst_codes,
                                                           uint8_t* __restrict__ dst_micro,
                                                           uint16_t* __restrict__ dst_macro, int64_t rows,
                                                           int64_t k) {
  constexpr int kTileBytes = E4M3 ? kTile8CodeBytes : kTileCodeBytes;
  constexpr int kChunks = kTileBytes / 16;             // 16-byte chunks per tile
  constexpr int kTilesPerBlock = kRepackThreads / kChunks;
  constexpr int kRunBytes = kTileBytes / 16;           // bytes of one row inside a tile
  constexpr int kRunChunks = kRunBytes / 16;
  __shared__ uint4 buf[kRepackThreads];

  const int64_t groups = k >> 8;
  const int64_t tiles = (rows >> 4) * groups;
  const int tid = threadIdx.x;
  const int lt = tid / kChunks;                    // tile of this workgroup
  const int ci = tid % kChunks;                    // chunk of that tile
  const int64_t T = (int64_t)blockIdx.x * kTilesPerBlock + lt;
  const bool live = T < tiles;                     // uniform per tile (whole waves)
  const int64_t rb = live ? T / groups : 0, g = live ? T - rb * groups : 0;
  const int64_t row_bytes = E4M3 ? k : k >> 1;     // canonical code bytes per row
  uint4* tbuf = buf + lt * kChunks;

  // ---- codes: source chunk ci -> LDS (source order) ----
  if (live) {
    const uint8_t* p;
    if (TO_TILED) {  // canonical chunk ci: row n = ci / kRunChunks, piece ci % kRunChunks
      const int n = ci / kRunChunks, pc = ci % kRunChunks;
      p = src_codes + (rb * 16 + n) * row_bytes + g * kRunBytes + pc * 16;
    } else {
      p = src_codes + T * kTileBytes + ci * 16;
    }
    tbuf[ci] = *reinterpret_cast<const uint4*>(p);
  }
  __syncthreads();
  if (live) {
    const uint32_t* w32 = reinterpret_cast<const uint32_t*>(tbuf);
    const uint2* w64 = reinterpret_cast<const uint2*>(tbuf);
    uint4 out;
    uint8_t* dp;
    if (TO_TILED) {
      // tiled chunk ci; the canonical run of row n starts at LDS byte n * kRunBytes
      if (!E4M3) {
        // ci = 64 h + 16 j + n: columns 32 (4h + u) + 8 j + 0..7, u = 0..3 -> one dword each
        const int h = ci >> 6, j = (ci >> 4) & 3, n = ci & 15;
        const int base = n * (kRunBytes / 4) + j;
        out = make_uint4(w32[base + 4 * (4 * h + 0)], w32[base + 4 * (4 * h + 1)],
                         w32[base + 4 * (4 * h + 2)], w32[base + 4 * (4 * h + 3)]);
      } else {
        // ci = 128 h + 64 p + 16 j + n: columns 32 (4h + 2p + u) + 8 j + 0..7, u = 0..1
        const int h = ci >> 7, pp = (ci >> 6) & 1, j = (ci >> 4) & 3, n = ci & 15;
        const int base = n * (kRunBytes / 8) + j;
        const uint2 a = w64[base + 4 * (4 * h + 2 * pp)], b = w64[base + 4 * (4 * h + 2 * pp + 1)];
        out = make_uint4(a.x, a.y, b.x, b.y);
      }
      dp = dst_codes + T * kTileBytes + ci * 16;
    } else {
      // canonical chunk ci = row n, piece pc; the tiled chunk (h, [p,] j, n) sits at LDS
      // chunk index h * 64 (+ p * 64) + 16 j + n
      const int n = ci / kRunChunks, pc = ci % kRunChunks;
      if (!E4M3) {
        // bytes 16 pc .. +15 of the row's run = columns 32 pc .. +31: t = pc, j = 0..3
        const int t = pc;
        const int c0 = (t >> 2) * 64 + n;
        out = make_uint4(w32[(c0 + 0) * 4 + (t & 3)], w32[(c0 + 16) * 4 + (t & 3)],
                         w32[(c0 + 32) * 4 + (t & 3)], w32[(c0 + 48) * 4 + (t & 3)]);
      } else {
        // bytes 16 pc .. +15 = columns 16 pc .. +15: t = pc / 2, j = 2 (pc % 2) + 0..1
        const int t = pc >> 1, j0 = 2 * (pc & 1);
        const int c0 = (t >> 2) * 128 + ((t >> 1) & 1) * 64 + n;
        const uint2 a = w64[(c0 + 16 * j0) * 2 + (t & 1)], b = w64[(c0 + 16 * (j0 + 1)) * 2 + (t & 1)];
        out = make_uint4(a.x, a.y, b.x, b.y);
      }
      dp = dst_codes + (rb * 16 + n) * row_bytes + g * kRunBytes + pc * 16;
    }
    *reinterpret_cast<uint4*>(dp) = out;
  }

  // ---- micro- and macro-scales: thread n < 16 of the tile moves row n's ----
  if (live && ci < 16) {
    const int n = ci;
    const int64_t r = rb * 16 + n;
    const int64_t tiled_off = T * kTileMicroBytes + n * 8;          // + p * 128: blocks 2t + p
    const int64_t canon_off = r * (k >> 4) + g * 16;                // blocks 0..15
    if (TO_TILED) {
      const uint4 v = *reinterpret_cast<const uint4*>(src_micro + canon_off);
      uint32_t e[4] = {0u, 0u, 0u, 0u};  // even blocks in e[0..1], odd in e[2..3]
#pragma unroll
      for (int b = 0; b < 16; ++b) e[(b & 1) * 2 + (b >> 3)] |= byte_of(v, b) << (8 * ((b >> 1) & 3));
      *reinterpret_cast<uint2*>(dst_micro + tiled_off) = make_uint2(e[0], e[1]);
      *reinterpret_cast<uint2*>(dst_micro + tiled_off + 128) = make_uint2(e[2], e[3]);
      dst_macro[T * kTileMacro + n] = src_macro[r * groups + g];
    } else {
      const uint2 ev = *reinterpret_cast<const uint2*>(src_micro + tiled_off);
      const uint2 od = *reinterpret_cast<const uint2*>(src_micro + tiled_off + 128);
      const uint4 both = make_uint4(ev.x, ev.y, od.x, od.y);  // bytes 0..7 even, 8..15 odd
      uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < 16; ++b) o[b >> 2] |= byte_of(both, (b & 1) * 8 + (b >> 1)) << (8 * (b & 3));
      *reinterpret_cast<uint4*>(dst_micro + canon_off) = make_uint4(o[0], o[1], o[2], o[3]);
      dst_macro[r * groups + g] = src_macro[T * kTileMacro + n];
    }
  }
}

}  // namespace

namespace fp4lib {

bool repack_supports(int64_t rows, int64_t k, int elem_e4m3) {
  if (rows < 16 || rows % 16 || k < 256 || k % 256) return false;
  const int64_t tiles = (rows / 16) * (k / 256);
  const int64_t per_block = elem_e4m3 ? 1 : 2;
  return (tiles + per_block - 1) / per_block <= 0x7FFFFFFF;
}

hipError_t launch_repack(const uint8_t* src_codes, const uint8_t* src_micro, const uint16_t* src_macro,
                         uint8_t* dst_codes, uint8_t* dst_micro, uint16_t* dst_macro, int64_t rows, int64_t k,
                         int elem_e4m3, int to_tiled, hipStream_t st) {
  if (!repack_supports(rows, k, elem_e4m3)) return hipErrorInvalidValue;
  const int64_t tiles = (rows / 16) * (k / 256);
  const int64_t per_block = elem_e4m3 ? 1 : 2;
  const dim3 grid((unsigned)((tiles + per_block - 1) / per_block)), block(kRepackThreads);
#define FP4_RP(E, T) \
  hipLaunchKernelGGL((k_repack<E, T>), grid, block, 0, st, src_codes, src_micro, src_macro, dst_codes, dst_micro, \
                     dst_macro, rows, k)
  if (elem_e4m3) { if (to_tiled) FP4_RP(1, 1); else FP4_RP(1, 0); }
  else { if (to_tiled) FP4_RP(0, 1); else FP4_RP(0, 0); }
#undef FP4_RP
  return hipGetLastError();
}

}  // namespace fp4lib
