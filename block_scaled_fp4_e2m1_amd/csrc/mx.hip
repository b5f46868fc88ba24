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
#include <type_traits>

#include "fp4_device.h"
#include "fp4_kernels.h"

using namespace fp4dev;

namespace {

constexpr int kMxBlock = 32;
constexpr int kMxTileK = 128;
constexpr int kMxTileCode = 1024;
constexpr int kMxTileScale = 64;
constexpr int kMxRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format


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
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// 128 x 128 output tile per workgroup, 4 waves of 64 x 64 (4 x 4 MFMAs of 16 x 16), one
// 128-wide k tile per stage. Each stage's operands (8 A and 8 W tiles of 1 KB, their
// scale bytes) are copied once per workgroup into LDS by 16-byte LDS-DMA, three stages
// ahead into a four-slot ring, and each wave reads its fragments from there: the waves
// sharing rows or columns no longer fetch the same bytes through L1 twice. One barrier
// per stage publishes the next stage, whose fragments each wave then reads while its
// MFMAs work on the current one. One LDS object per slot and compile-time slot indices,
// so the compiler can tell the slot being filled from the ones being read.
struct MxStage {
  uint4 a[8][64];      // tile i (row block i of the workgroup), lane l's 16 bytes
  uint4 w[8][64];
  uint32_t as[8][16];  // tile i's 64 scale bytes
  uint32_t ws[8][16];
};
__shared__ MxStage g_mx0;
__shared__ MxStage g_mx1;
__shared__ MxStage g_mx2;
__shared__ MxStage g_mx3;
constexpr int kMxStages = 4;
constexpr int kMxCopies = 5;  // LDS-DMA instructions per wave and stage

template <int B>
__device__ __forceinline__ MxStage& mx_stage() {
  if constexpr (B == 0) return g_mx0;
  else if constexpr (B == 1) return g_mx1;
  else if constexpr (B == 2) return g_mx2;
  else return g_mx3;
}

// a wave's operands of one stage
struct MxFrags {
  u32x4_t af[4], wf[4];
  uint32_t as[4], ws[4];
};

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
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of tiles (n fastest), so its L2 keeps the same activation rows
  const int gx = gridDim.x, total = gx * gridDim.y;
  int bid = blockIdx.y * gx + blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int bx = bid % gx, by = bid / gx;
  const int64_t mb0 = (int64_t)by * 8, nb0 = (int64_t)bx * 8;  // first row block of A / W
  // copies of wave w: A tiles 2w, 2w + 1 and W tiles 2w, 2w + 1 (1 KB each), and one
  // scale copy (64 lanes x 4 bytes = the scale bytes of 4 tiles): A tiles 0-3 / 4-7 for
  // waves 0 / 1, W tiles 0-3 / 4-7 for waves 2 / 3
  int64_t a_tile[2], w_tile[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a_tile[i] = min(mb0 + 2 * wave + i, a_rb_count - 1) * kt_count;
    w_tile[i] = min(nb0 + 2 * wave + i, w_rb_count - 1) * kt_count;
  }
  const bool sc_a = wave < 2;
  const int sc_first = (wave & 1) * 4 + (lane >> 4);  // tile whose scale dword this lane moves
  const int64_t sc_tile = sc_a ? min(mb0 + sc_first, a_rb_count - 1) * kt_count
                               : min(nb0 + sc_first, w_rb_count - 1) * kt_count;
  const uint8_t* sc_src = (sc_a ? a_scales : w_scales) + sc_tile * kMxTileScale + (lane & 15) * 4;
  auto copy_stage = [&](MxStage& st, int64_t kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds((global_void_ptr)(a_codes + (a_tile[i] + kt) * kMxTileCode + lane * 16),
                                       (lds_void_ptr)&st.a[2 * wave + i][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((global_void_ptr)(w_codes + (w_tile[i] + kt) * kMxTileCode + lane * 16),
                                       (lds_void_ptr)&st.w[2 * wave + i][0], 16, 0, 0);
    }
    if (sc_a)  // wave-uniform
      __builtin_amdgcn_global_load_lds((global_void_ptr)(sc_src + kt * kMxTileScale),
                                       (lds_void_ptr)&st.as[(wave & 1) * 4][0], 4, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((global_void_ptr)(sc_src + kt * kMxTileScale),
                                       (lds_void_ptr)&st.ws[(wave & 1) * 4][0], 4, 0, 0);
  };

  const int wm = wave & 1, wn = wave >> 1;
  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto read_frags = [&](const MxStage& st, MxFrags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.af[i] = __builtin_bit_cast(u32x4_t, st.a[wm * 4 + i][lane]);
      f.wf[i] = __builtin_bit_cast(u32x4_t, st.w[wn * 4 + i][lane]);
      f.as[i] = reinterpret_cast<const uint8_t*>(st.as[wm * 4 + i])[lane];
      f.ws[i] = reinterpret_cast<const uint8_t*>(st.ws[wn * 4 + i])[lane];
    }
  };
  // The same reads as one inline-asm block that waits for its own results. Used by the
  // first stage of each pass of the stage loop: where the loop's back edge meets its
  // entry the compiler no longer knows which slots have copies in flight, and before a
  // plain LDS read there it waited for every copy, the ones issued three stages ahead
  // included.
  auto read_frags_waited = [&](const MxStage& st, MxFrags& f) {
    const uint32_t a_addr = (uint32_t)(uintptr_t)(lds_void_ptr)&st.a[wm * 4][lane];
    const uint32_t w_addr = (uint32_t)(uintptr_t)(lds_void_ptr)&st.w[wn * 4][lane];
    const uint32_t as_addr = (uint32_t)(uintptr_t)(lds_void_ptr)(reinterpret_cast<const uint8_t*>(st.as[wm * 4]) + lane);
    const uint32_t ws_addr = (uint32_t)(uintptr_t)(lds_void_ptr)(reinterpret_cast<const uint8_t*>(st.ws[wn * 4]) + lane);
    asm volatile(
        "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:1024\n\t"
        "ds_read_b128 %2, %16 offset:2048\n\tds_read_b128 %3, %16 offset:3072\n\t"
        "ds_read_b128 %4, %17\n\tds_read_b128 %5, %17 offset:1024\n\t"
        "ds_read_b128 %6, %17 offset:2048\n\tds_read_b128 %7, %17 offset:3072\n\t"
        "ds_read_u8 %8, %18\n\tds_read_u8 %9, %18 offset:64\n\t"
        "ds_read_u8 %10, %18 offset:128\n\tds_read_u8 %11, %18 offset:192\n\t"
        "ds_read_u8 %12, %19\n\tds_read_u8 %13, %19 offset:64\n\t"
        "ds_read_u8 %14, %19 offset:128\n\tds_read_u8 %15, %19 offset:192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.af[0]), "=&v"(f.af[1]), "=&v"(f.af[2]), "=&v"(f.af[3]), "=&v"(f.wf[0]), "=&v"(f.wf[1]),
          "=&v"(f.wf[2]), "=&v"(f.wf[3]), "=&v"(f.as[0]), "=&v"(f.as[1]), "=&v"(f.as[2]), "=&v"(f.as[3]),
          "=&v"(f.ws[0]), "=&v"(f.ws[1]), "=&v"(f.ws[2]), "=&v"(f.ws[3])
        : "v"(a_addr), "v"(w_addr), "v"(as_addr), "v"(ws_addr));
  };
  auto compute = [&](const MxFrags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v8i a = {(int)f.af[i][0], (int)f.af[i][1], (int)f.af[i][2], (int)f.af[i][3], 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8i b = {(int)f.wf[j][0], (int)f.wf[j][1], (int)f.wf[j][2], (int)f.wf[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i][j], 4, 4, 0, (int)f.as[i], 0,
                                                                       (int)f.ws[j]);
      }
    }
  };
  // Stage kt (slot B = kt % 4), its fragments already in registers (fr[kt & 1]): wait for this
  // wave's copies of kt + 1 (only the copies of kt + 2, issued one stage later, may stay in
  // flight), barrier (every wave's copies of kt + 1 have landed, and every wave is done
  // with kt - 1: its fragments were read a stage earlier and consumed by its MFMAs), copy
  // kt + 3 into kt - 1's slot, read kt + 1's fragments, then the MFMAs of kt. The barrier is
  // a bare s_barrier: a workgroup fence would also wait for the copies of kt + 2. LDS is
  // coherent inside the workgroup; the empty asm statements keep the compiler from moving
  // memory accesses across it. Every stage copies (past the end, the last tile again into
  // the slot of a finished stage), so exactly kMxCopies copies are younger than the awaited
  // ones on every path; past the end the fragments read are not used.
  MxFrags fr[2];  // stage kt's fragments in fr[kt & 1], the next stage's read into the other
  auto step = [&](auto b_const, int64_t kt) {
    constexpr int B = decltype(b_const)::value;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kVmcntWait<kMxCopies>::value);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    copy_stage(mx_stage<(B + 3) % kMxStages>(), min(kt + 3, kt_count - 1));
    MxFrags& nxt = fr[(B + 1) & 1];
    if constexpr (B == 0)
      read_frags_waited(mx_stage<1>(), nxt);
    else
      read_frags(mx_stage<(B + 1) % kMxStages>(), nxt);
    __builtin_amdgcn_sched_barrier(0);
    compute(fr[B & 1]);
    __builtin_amdgcn_sched_barrier(0);
    // (the next fragments are used here, after the MFMAs are issued: otherwise the
    // compiler sinks their reads to the next stage, right before the MFMAs that need them)
    asm volatile("" : : "v"(nxt.af[0]), "v"(nxt.af[1]), "v"(nxt.af[2]), "v"(nxt.af[3]), "v"(nxt.wf[0]),
                 "v"(nxt.wf[1]), "v"(nxt.wf[2]), "v"(nxt.wf[3]));
    asm volatile("" : : "v"(nxt.as[0]), "v"(nxt.as[1]), "v"(nxt.as[2]), "v"(nxt.as[3]), "v"(nxt.ws[0]),
                 "v"(nxt.ws[1]), "v"(nxt.ws[2]), "v"(nxt.ws[3]));
  };
  copy_stage(g_mx0, 0);
  copy_stage(g_mx1, min((int64_t)1, kt_count - 1));
  copy_stage(g_mx2, min((int64_t)2, kt_count - 1));
  // stage 0 published (this wave's copies of it done; those of 1 and 2 may be in flight)
  __builtin_amdgcn_s_waitcnt(kVmcntWait<2 * kMxCopies>::value);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_frags(g_mx0, fr[0]);
  // whole passes over the four slots (one exit), then the last 0-3 stages
  int64_t kt = 0;
  for (; kt + kMxStages <= kt_count; kt += kMxStages) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
    step(std::integral_constant<int, 2>{}, kt + 2);
    step(std::integral_constant<int, 3>{}, kt + 3);
  }
  if (kt < kt_count) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < kt_count) {
      step(std::integral_constant<int, 1>{}, kt + 1);
      if (kt + 2 < kt_count) step(std::integral_constant<int, 2>{}, kt + 2);
    }
  }
  // no copy may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(kVmcntWait<0>::value);
  // (an opaque copy of the lane index: the lane's store offset is formed here, not before
  // the loop, where it would hold a register; the resource below is built from wave-uniform
  // values only, so it stays in scalar registers)
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int64_t m0 = (int64_t)by * 128 + wm * 64;
  const int64_t n0 = (int64_t)bx * 128 + wn * 64;
  // The stores go through a raw buffer over the wave's valid rows: each store's row offset
  // is a scalar, and a row at or past m lies outside the buffer, where the hardware drops
  // the store (the boundary keeps 64 x ldc x 4 bytes below 2^31). Columns past n are
  // masked per lane: the buffer spans whole rows of ldc elements.
  constexpr int kES = OUT_BF16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char*>(c) + m0 * ldc * kES, (short)0,
      (int)(max((int64_t)0, min((int64_t)64, m - m0)) * ldc * kES), kMxRsrcWord3);
  const int64_t col0 = n0 + (lane_e & 15);
  const uint32_t c_voff = (uint32_t)(((int64_t)(4 * (lane_e >> 4)) * ldc + col0) * kES);
  // lane l holds rows 4 (l / 16) + t, column l % 16 of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (col0 + 16 * j >= n) continue;
#pragma unroll
      for (int t = 0; t < 4; t += 2) {  // rows t and t + 1: one bf16 conversion
        const uint32_t c_soff = (uint32_t)(((int64_t)(16 * i + t) * ldc + 16 * j) * kES);
        const uint32_t c_soff1 = c_soff + (uint32_t)(ldc * kES);
        if (OUT_BF16) {
          const uint32_t b = bf16x2_rne(acc[i][j][t], acc[i][j][t + 1]);
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)b, c_rsrc, c_voff, c_soff, 0);
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(b >> 16), c_rsrc, c_voff, c_soff1, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][t]), c_rsrc, c_voff, c_soff, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][t + 1]), c_rsrc, c_voff, c_soff1, 0);
        }
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
