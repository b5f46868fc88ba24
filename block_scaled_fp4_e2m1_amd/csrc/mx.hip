// MX-native FP4 on gfx950: quantization to E2M1 with one E8M0 power-of-two scale per 32
// elements, and the product on the block-scaled FP4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4,
// FP4 x FP4, scales applied by the matrix core).
//
// Not the pages' two-level format: its micro-scale (E4M3 per 16) and macro-scale (FP16 per
// 256) do not map onto the instruction's E8M0-per-32 scales without changing the numbers
// (the instruction, like the hardware conversions, only applies powers of two). This is
// the format that reaches the FP4 matrix peak; it is kept beside the pages' format to
// measure that speed and the accuracy difference.
//
// Quantization (OCP microscaling reading for MXFP4): per 32 consecutive elements of a row,
// e = floor(log2(max |x|)) - 2 clamped to [-127, 127] (-127 for an all-zero block), scale
// byte e + 127, codes = x / 2^e rounded to nearest E2M1 (ties to even, saturating at 6;
// the sign kept for values that round to 0).
//
// Tiled layout (rows padded to a multiple of 16, k % 128 == 0): tile T = (r / 16) *
// (k / 128) + c / 128 holds 16 rows x 128 columns; its 1024 code bytes are [kb 4][n 16][16]
// with kb = (c % 128) / 32, n = r % 16 (32 codes, low nibble first), its 64 scale bytes
// [kb 4][n 16]. Lane l = 16 kb + n of an MFMA reads the 16 bytes at l * 16 and the scale
// byte l: exactly its operand (row n, k = 32 kb .. +31) and that block's scale.
#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;

namespace {

constexpr int kMxBlock = 32;
constexpr int kMxTileK = 128;
constexpr int kMxTileCode = 1024;
constexpr int kMxTileScale = 64;

// One thread per 32-element block; consecutive threads walk (row block, k tile, kb, n) with
// n fastest, so 16 threads write 256 contiguous code bytes and 64 threads 64 scale bytes.
template <int IN_BF16>
__global__ __launch_bounds__(256) void k_mx_quantize(const void* __restrict__ x, int64_t ldx, int64_t rows,
                                                     int64_t k, int64_t padded_rows,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t kt_count = k / kMxTileK;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // block index in tile order
  if (idx >= padded_rows * (k / kMxBlock)) return;
  const int n = (int)(idx & 15), kb = (int)((idx >> 4) & 3);
  const int64_t tile = idx >> 6;  // (row block) * kt_count + k tile
  const int64_t rb = tile / kt_count, kt = tile - rb * kt_count;
  const int64_t r = rb * 16 + n, c0 = kt * kMxTileK + kb * kMxBlock;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  uint32_t sbyte = 0u;  // e = -127 for padding rows and all-zero blocks
  if (r < rows) {
    float v[32];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Raw16<IN_BF16> raw;
      load_raw16<IN_BF16>(x, r * ldx + c0 + 16 * h, raw);
      unpack16<IN_BF16>(raw, v + 16 * h);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    if (amax > 0.0f) {
      // floor(log2(amax)) from the float32 bits (normal or subnormal)
      const uint32_t bits = __float_as_uint(amax);
      const int ef = (int)(bits >> 23);
      const int fl = ef > 0 ? ef - 127 : (31 - __clz(bits & 0x7FFFFFu)) - 149;
      const int e = min(max(fl - 2, -127), 127);
      sbyte = (uint32_t)(e + 127);
      // X = 2^e as a float (2^-127 is a subnormal float)
      const float X = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
      const E2M1Thresholds th(X);  // t * X exact; above 5X (and past 6X) gives code 7 = 6
#pragma unroll
      for (int i = 0; i < 32; ++i)
        w[i >> 3] |= (th.mag(fabsf(v[i])) | (sign_of(v[i]) << 3)) << (4 * (i & 7));
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) w[i >> 3] |= (sign_of(v[i]) << 3) << (4 * (i & 7));
    }
  }
  *reinterpret_cast<uint4*>(codes + tile * kMxTileCode + (16 * kb + n) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[tile * kMxTileScale + 16 * kb + n] = (uint8_t)sbyte;
}

typedef int v8i __attribute__((ext_vector_type(8)));

// 128 x 128 output tile per workgroup, 4 waves of 64 x 64 (4 x 4 MFMAs of 16 x 16), one
// 128-wide k tile per step. Operands go straight to registers (each lane's 16-byte piece is
// its MFMA operand), kMxDepth - 1 steps ahead of the step being computed: a step's 16
// MFMAs take ~256 cycles per wave, shorter than a loaded L2 round trip.
constexpr int kMxDepth = 3;

template <int OUT_BF16>
__global__ __launch_bounds__(256, 2) void k_gemm_mx(const uint8_t* __restrict__ a_codes,
                                                 const uint8_t* __restrict__ a_scales, int64_t m,
                                                 const uint8_t* __restrict__ w_codes,
                                                 const uint8_t* __restrict__ w_scales, int64_t n, int64_t k,
                                                 void* __restrict__ c, int64_t ldc) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t kt_count = k / kMxTileK;
  const int64_t a_rb_count = (m + 15) / 16, w_rb_count = (n + 15) / 16;
  const int64_t m0 = (int64_t)blockIdx.y * 128 + (wave & 1) * 64;
  const int64_t n0 = (int64_t)blockIdx.x * 128 + (wave >> 1) * 64;
  // row blocks of this wave (clamped into the arrays; clamped rows are never stored)
  int64_t a_tile0[4], w_tile0[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_tile0[i] = min(m0 / 16 + i, a_rb_count - 1) * kt_count;
    w_tile0[i] = min(n0 / 16 + i, w_rb_count - 1) * kt_count;
  }
  uint4 af[kMxDepth][4], wf[kMxDepth][4];
  uint32_t as[kMxDepth][4], ws[kMxDepth][4];
  auto load = [&](int buf, int64_t kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t ta = a_tile0[i] + kt, tw = w_tile0[i] + kt;
      af[buf][i] = *reinterpret_cast<const uint4*>(a_codes + ta * kMxTileCode + lane * 16);
      wf[buf][i] = *reinterpret_cast<const uint4*>(w_codes + tw * kMxTileCode + lane * 16);
      as[buf][i] = a_scales[ta * kMxTileScale + lane];
      ws[buf][i] = w_scales[tw * kMxTileScale + lane];
    }
  };
  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int d = 0; d + 1 < kMxDepth; ++d)
    if (d < kt_count) load(d, d);
  for (int64_t kt = 0; kt < kt_count; kt += kMxDepth) {
#pragma unroll
    for (int h = 0; h < kMxDepth; ++h) {  // buffer h holds k tile kt + h
      if (kt + h >= kt_count) break;
      if (kt + h + kMxDepth - 1 < kt_count) load((h + kMxDepth - 1) % kMxDepth, kt + h + kMxDepth - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v8i a = {(int)af[h][i].x, (int)af[h][i].y, (int)af[h][i].z, (int)af[h][i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v8i b = {(int)wf[h][j].x, (int)wf[h][j].y, (int)wf[h][j].z, (int)wf[h][j].w, 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i][j], 4, 4, 0, (int)as[h][i], 0,
                                                                         (int)ws[h][j]);
        }
      }
    }
  }
  // lane l holds rows 4 (l / 16) + t, column l % 16 of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + 16 * j + (lane & 15);
      if (col >= n) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t row = m0 + 16 * i + 4 * (lane >> 4) + t;
        if (row >= m) continue;
        if (OUT_BF16)
          static_cast<uint16_t*>(c)[row * ldc + col] = (uint16_t)bf16_rne_bits(acc[i][j][t]);
        else
          static_cast<float*>(c)[row * ldc + col] = acc[i][j][t];
      }
    }
}

}  // namespace

namespace fp4lib {

int64_t mx_padded_rows(int64_t rows) { return (rows + 15) / 16 * 16; }

hipError_t launch_mx_quantize(const void* x, int in_bf16, int64_t rows, int64_t k, int64_t ldx, uint8_t* codes,
                              uint8_t* scales, hipStream_t st) {
  const int64_t blocks = mx_padded_rows(rows) * (k / kMxBlock);
  const int64_t grid = (blocks + 255) / 256;
  if (grid < 1 || grid > 0x7FFFFFFF || k % kMxTileK) return hipErrorInvalidValue;
  if (in_bf16)
    hipLaunchKernelGGL(k_mx_quantize<1>, dim3((unsigned)grid), dim3(256), 0, st, x, ldx, rows, k,
                       mx_padded_rows(rows), codes, scales);
  else
    hipLaunchKernelGGL(k_mx_quantize<0>, dim3((unsigned)grid), dim3(256), 0, st, x, ldx, rows, k,
                       mx_padded_rows(rows), codes, scales);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_codes,
                          const uint8_t* w_scales, int64_t n, int64_t k, void* c, int out_bf16, int64_t ldc,
                          hipStream_t st) {
  if (m < 1 || n < 1 || k < kMxTileK || k % kMxTileK) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128)), block(256);
  if (grid.y > 65535) return hipErrorInvalidValue;
  if (out_bf16)
    hipLaunchKernelGGL(k_gemm_mx<1>, grid, block, 0, st, a_codes, a_scales, m, w_codes, w_scales, n, k, c, ldc);
  else
    hipLaunchKernelGGL(k_gemm_mx<0>, grid, block, 0, st, a_codes, a_scales, m, w_codes, w_scales, n, k, c, ldc);
  return hipGetLastError();
}

}  // namespace fp4lib
