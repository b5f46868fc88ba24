/*
 * fp4_probes.h -- measurement probes (libfp4_probes.so), not part of the product API: they
 * measure, on the device at hand, the ceilings the library's kernels are measured against.
 * Every pointer is caller-owned device memory; `stream` is a hipStream_t. Each call
 * enqueues one kernel and returns 0, 2 for invalid arguments (nothing enqueued) or 8 when
 * the launch fails.
 *
 * probe_read     -- reads `bytes` (a multiple of 16) from src with 16-byte nontemporal loads,
 *                   `blocks` workgroups of `threads` (a multiple of 64, <= 1024) in a grid-
 *                   stride loop with four loads in flight per thread; sink: 1024 uint32
 *                   words that receive an xor of what was read. The floor of a kernel that
 *                   reads the same bytes with the same launch shape.
 * probe_mfma     -- `blocks` workgroups of 4 waves, each wave issuing iters x chains MFMAs
 *                   (16384 flops each for 16x16x32, 32768 for 32x32x16) on `chains` (4, 8
 *                   or 16) independent register accumulators; kind 0: 16x16x32 f16, 1:
 *                   32x32x16 f16, 2: 16x16x32 bf16. The sustained dense 16-bit matrix rate.
 * probe_valu     -- `blocks` workgroups of 4 waves, each wave running iters x 8 independent
 *                   instructions of one kind (0: v_cvt_scalef32_pk_f16_fp4, 1: v_pk_mul_f16,
 *                   2: v_perm_b32, 3: v_mul_f32, 4: v_cvt_scalef32_pk_f16_fp8, 5: and-or
 *                   bit merge, 6: v_cvt_scalef32_pk_f32_fp4 plus an xor). VALU issue rates.
 * probe_mix      -- `blocks` workgroups of 4 waves, each wave running iters x (8 independent
 *                   v_mfma_f32_16x16x32_f16 interleaved with valu_per_8 (0, 8, 16, 24, 32
 *                   or 48) independent v_pk_mul_f16). Whether the SIMD overlaps MFMA and
 *                   VALU work, and at what cost.
 * probe_lds_read -- `blocks` workgroups of 4 waves, each wave issuing iters x 16 conflict-free
 *                   16-byte LDS reads per lane (1 KB per wave instruction) from a 64 KB LDS
 *                   buffer. The LDS read bandwidth per compute unit.
 *   For these: clocks (2 x blocks uint64) receives per workgroup the shader-clock cycles
 *   (s_memtime) and the 100 MHz real-time ticks (s_memrealtime) its wave 0 spent in the
 *   measured loop, from which the clock it ran at follows.
 */
#ifndef FP4_PROBES_H
#define FP4_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t probe_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t threads,
                   void* stream);
int32_t probe_mfma(int32_t kind, int32_t chains, int32_t blocks, int32_t iters, uint64_t* clocks, void* stream);
int32_t probe_valu(int32_t kind, int32_t blocks, int32_t iters, uint64_t* clocks, void* stream);
int32_t probe_mix(int32_t valu_per_8, int32_t blocks, int32_t iters, uint64_t* clocks, void* stream);
int32_t probe_lds_read(int32_t blocks, int32_t iters, uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4_PROBES_H */
