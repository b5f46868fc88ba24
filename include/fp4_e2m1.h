/*
 * fp4_e2m1.h -- C ABI of the MI355X (gfx950) two-level block-scaled FP4 library.
 *
 * The format ("NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell
 * B200", section "The Mathematical Breakthrough of Microscopic FP4 Scaling", items 1-3):
 *   - elements are E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no Inf/NaN;
 *   - each micro-vector of 16 consecutive elements (along K, inside one row) carries an
 *     FP8 E4M3 (OCP, max 448) micro-scale mu;
 *   - each run of 16 micro-vectors (256 elements) shares an FP16 macro-scale M;
 *   - value(x) = e2m1(code) * mu * M.
 * Scale selection (max-abs): M = RNE_fp16(amax_256 / (emax * 448)) clamped to
 * [2^-24, 65504] when amax_256 > 0 (else 0); mu = RNE_e4m3(amax_16 / (emax * M));
 * code = RNE_elem(|x| / (mu * M)) with the sign of x kept (a block whose mu*M is 0 gets
 * code 0). emax = 6 for E2M1 elements, 448 for E4M3 elements (8-bit activations of W4A8
 * layers, "llama.cpp Put Precision Policy Inside the Model", section "One model can need
 * more than one precision"). Every rounding is to nearest, ties to even, saturating.
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller (e.g. torch tensors);
 *     the library never allocates, frees or synchronizes.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it and the
 *     call returns; device faults surface at the caller's next synchronization.
 *   - Arguments are validated before anything is enqueued. On any error nothing is
 *     enqueued and a status code is returned. There is no fallback to another precision
 *     or another path (fail fast, as the AdaLLM page describes its decode path).
 *   - Inputs must be finite; non-finite inputs give unspecified codes.
 *   - The library runs only on gfx950 (FP4_E_ARCH elsewhere).
 *
 * Packed layouts of a quantized [rows x k] tensor (k % 256 == 0):
 *   CANONICAL  codes: row-major, E2M1 two per byte (element 2i in the low nibble of byte
 *              i) or E4M3 one per byte; micro[r*k/16 + b]; macro[r*k/256 + g].
 *   TILED      (E2M1 only, rows % 16 == 0) the same bytes permuted so that a 64-lane
 *              wave reads a 16-row x 256-column tile with two coalesced 16-byte loads
 *              per lane. Tile T = (r/16) * (k/256) + g. Inside a tile, with n = r % 16,
 *              column c = k_in_tile (0..255), t = c / 32, j = (c % 32) / 8:
 *                code byte  T*2048 + (t/4)*1024 + (16*j + n)*16 + (t%4)*4 + (c%8)/2
 *                           (nibble order inside the byte as canonical)
 *                micro byte T*256 + p*128 + n*8 + t   for block b = c/16 = 2t + p
 *                macro      T*16 + n                  (uint16 index)
 *              Total sizes equal the canonical ones.
 *              E4M3 elements (rows % 16 == 0): tiles of 4096 code bytes, T as above;
 *              with t, j, n as above,
 *                code byte  T*4096 + (t/4)*2048 + ((t%4)/2)*1024 + (16*j + n)*16
 *                           + (t%2)*8 + c%8
 *              micro and macro as for E2M1.
 */
#ifndef FP4_E2M1_H
#define FP4_E2M1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fp4_status;
enum {
  FP4_OK = 0,
  FP4_E_NULL = 1,       /* a required pointer is NULL                                  */
  FP4_E_SHAPE = 2,      /* bad size: k % 256, rows % 16 (tiled), m/n/rows < 1, ld < k  */
  FP4_E_ALIGN = 3,      /* a pointer or row stride is not 16-byte aligned              */
  FP4_E_DTYPE = 4,      /* unsupported dtype / precision combination                    */
  FP4_E_MODE = 5,       /* unknown act, elem, layout or policy value                    */
  FP4_E_NO_DEVICE = 6,  /* no HIP device is visible                                    */
  FP4_E_ARCH = 7,       /* the current device is not gfx950                             */
  FP4_E_HIP = 8,        /* a HIP runtime call or kernel launch failed                   */
  FP4_E_WORKSPACE = 9,  /* workspace NULL/too small for fp4_workspace_bytes()           */
  FP4_E_LAYOUT = 10     /* the operation needs the other packed layout                  */
};

enum { FP4_F32 = 0, FP4_BF16 = 1 };                         /* element types of x/y/a/c */
enum { FP4_A16 = 16, FP4_A8 = 8, FP4_A4 = 4 };              /* activation precision      */
/* further precision codes of the policy table: W4A4 / W4A8 with static activation
 * macro-scales (gemm_w4aX_static) and W8A8 (gemm_w8a8) */
enum { FP4_A4S = 40, FP4_A8S = 80, FP4_W8A8 = 88 };
enum { FP4_ELEM_E2M1 = 0, FP4_ELEM_E4M3 = 1 };              /* quantized element type    */
enum { FP4_LAYOUT_CANONICAL = 0, FP4_LAYOUT_TILED = 1 };
enum { FP4_POLICY_AUTO = 0, FP4_POLICY_SENSITIVE_W8 = 1, FP4_POLICY_STATIC = 2,
       FP4_POLICY_Q4 = 4, FP4_POLICY_Q8 = 8 };

/* A quantized tensor in device memory (see the layouts above). */
typedef struct fp4_tensor {
  const void* codes;       /* packed codes                                   */
  const uint8_t* micro;    /* rows * k / 16 E4M3 micro-scales                */
  const uint16_t* macro;   /* rows * k / 256 FP16 macro-scales (bit patterns) */
  int64_t rows;
  int64_t k;
  int32_t elem;            /* FP4_ELEM_*   */
  int32_t layout;          /* FP4_LAYOUT_* */
} fp4_tensor;

/*
 * quantize_fp4 -- two-level block-scaled quantization of x [rows x k].
 *   x        device, FP4_F32 or FP4_BF16 values, row r at x + r*ldx elements
 *   ldx      row stride in elements (>= k; ldx * sizeof(elem) % 16 == 0)
 *   elem     FP4_ELEM_E2M1 (4-bit codes) or FP4_ELEM_E4M3 (8-bit codes)
 *   layout   FP4_LAYOUT_CANONICAL or FP4_LAYOUT_TILED (rows % 16 == 0)
 *   codes    device out: rows*k/2 bytes (E2M1) or rows*k bytes (E4M3), 16-byte aligned
 *   micro    device out: rows*k/16 bytes
 *   macro    device out: rows*k/256 uint16
 * Source: TensorRT-LLM FP4 page, section on microscopic FP4 scaling, items 1-2.
 */
fp4_status quantize_fp4(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx,
                        int32_t elem, int32_t layout, void* codes, uint8_t* micro,
                        uint16_t* macro, void* stream);

/*
 * quantize_fp4_static -- quantize_fp4 with given macro-scales: macro_in (device, FP16 bit
 * patterns [k/256], finite and non-negative, e.g. from act_macro_calibrate) is the macro-
 * scale of every row's group g; mu = RNE_e4m3(amax_16 / (emax * M)) saturates at 448 and
 * elements at the element maximum for blocks beyond the calibrated range; M = 0 gives
 * zero codes. `macro` receives M for every row. Source: TensorRT-LLM FP4 page, section
 * "Step 2: Executing FP4 Calibration and Engine Compilation" (activation ranges are
 * calibrated ahead of deployment) and "Deployment Guidelines and Production Safeguards",
 * item 1 (calibration data matching production traffic).
 */
fp4_status quantize_fp4_static(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx,
                               int32_t elem, int32_t layout, const uint16_t* macro_in, void* codes,
                               uint8_t* micro, uint16_t* macro, void* stream);

/*
 * act_macro_calibrate -- static activation macro-scales from calibration data x [rows x k]
 * (device, FP4_BF16 or FP4_F32, stride ldx, 16-byte aligned rows):
 *   amax[g]  = max(amax[g], max |x[r, 256 g .. 256 g + 255]| over every row)   (running)
 *   macro[g] = FP16 bits of RNE_fp16(amax[g] / (emax * 448)) clamped to [2^-24, 65504],
 *              0 when amax[g] == 0 (the dynamic rule applied to the group's maximum)
 * amax: device float32 [k/256], zero it before the first batch; calling once per
 * calibration batch leaves the macro-scales of everything seen so far in `macro` (device
 * uint16 [k/256]). elem: the element type the activations will be quantized to. The
 * order of the rows and calls does not change the result.
 */
fp4_status act_macro_calibrate(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx,
                               int32_t elem, float* amax, uint16_t* macro, void* stream);

/*
 * repack_fp4 -- the same quantized tensor in the other packed layout: src (either layout,
 * E2M1 or E4M3 elements, rows % 16 == 0) is written to codes / micro / macro (device, the
 * sizes of src's arrays, codes and micro 16-byte aligned) in `layout`, which must differ
 * from src->layout (FP4_E_LAYOUT otherwise). A byte permutation of the codes, the micro-
 * scales and the macro-scales: nothing is decoded or re-rounded, so repacking is exact
 * and tiled -> canonical -> tiled returns the original bytes (re-quantizing dequantized
 * values is not exact in general: bf16 values are re-rounded, and with E4M3 elements a
 * block maximum that rounds down changes the block's micro-scale). This is
 * how weights stored in the canonical interchange layout reach the product kernels,
 * which read the tiled one. The source and destination must not overlap.
 * Source: TensorRT-LLM FP4 page, section on microscopic FP4 scaling, items 1-2 (the
 * format being moved); the tiled layout is this library's.
 */
fp4_status repack_fp4(const fp4_tensor* src, int32_t layout, void* codes, uint8_t* micro, uint16_t* macro,
                      void* stream);

/*
 * dequantize_fp4 -- y = value(code) * mu * M for every element of q (either layout).
 *   y        device out [q->rows x q->k], FP4_F32 (exact) or FP4_BF16 (round to nearest
 *            even of the exact value), row stride ldy elements (16-byte aligned rows)
 * Source: TensorRT-LLM FP4 page, section on microscopic FP4 scaling, item 3 (scales are
 * applied before the dot products).
 */
fp4_status dequantize_fp4(const fp4_tensor* q, void* y, int32_t y_dtype, int64_t ldy,
                          void* stream);

/*
 * Output row stride of the products below (gemm_w4aX and its _noalloc / _static forms,
 * gemm_w8a8, grouped_gemm_w4aX, grouped_gemm_w4aX_gated, gemm_mxfp4): n <= ldc <=
 * FP4_MAX_LDC elements, FP4_E_SHAPE otherwise, before anything is enqueued (the product
 * kernels address an output tile of up to 128 rows with 32-bit byte offsets).
 */
enum { FP4_MAX_LDC = 1 << 21 };

/*
 * gemm_w4aX -- C[m x n] = A_hat . W_hat^T with float32 accumulation.
 *   act      FP4_A16: A_hat = A;  FP4_A4: A_hat = dequant(quant_e2m1(A));
 *            FP4_A8: A_hat = dequant(quant_e4m3(A)); A is quantized on the device per
 *            call (dynamic activation quantization, no calibration).
 *   a        device [m x k] (FP4_BF16, or FP4_F32), row stride lda elements
 *   w        quantized weights [n x k], E2M1, TILED layout (FP4_E_LAYOUT otherwise)
 *   c        device out [m x n], FP4_BF16 (round to nearest even) or FP4_F32, stride ldc
 *   workspace device scratch of at least fp4_workspace_bytes(act, m, n, k) bytes
 *            (may be NULL when that is 0); contents are overwritten
 * Paths: FP4_A16 with FP4_F32 activations runs one thread per output (m * n <= 2^32 -
 * 256); FP4_A16 with bf16 activations and m <= 8, k <= 8192 runs the decode GEMV; every
 * other call runs the activation pass (FP4_A4 / FP4_A8) and the product kernel, which
 * needs k <= 21760 (its per-group tables fit LDS). Shapes outside these limits return
 * FP4_E_SHAPE before anything is enqueued. For FP4_A4 on the large-product form
 * (fp4_product_kernel names it) the activation pass writes A in the canonical E2M1
 * layout of quantize_fp4 into the workspace and the product kernel decodes it; other
 * paths write an FP16 operand and per-group factors there. Results are the same bits.
 * Source: "llama.cpp Put Precision Policy Inside the Model", intro and section "One model
 * can need more than one precision" (W4A4, W4A8 and W4A16 layers).
 */
fp4_status gemm_w4aX(int32_t act, const void* a, int32_t a_dtype, int64_t m, int64_t lda,
                     const fp4_tensor* w, void* c, int32_t c_dtype, int64_t ldc,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gemm_w4aX_noalloc -- gemm_w4aX for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, results and limits as gemm_w4aX, without the workspace: the FP4_A4 / FP4_A8
 * activation operand lives in the library's own device array of
 * FP4_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held from the library's first use of that
 * GPU until the process ends. A call whose workspace would exceed it
 * (fp4_workspace_bytes(act, m, n, k) > FP4_NOALLOC_SCRATCH_BYTES, e.g. m x k above
 * ~16.6 M activation elements at k = 4096) returns FP4_E_WORKSPACE before anything is
 * enqueued. No hipMalloc, hipFree or allocating library routine is called. Every call on
 * a GPU shares that GPU's array: calls enqueued on one stream are ordered, but calls that
 * overlap on one GPU (unordered streams, host threads) race and give wrong results. Each
 * call writes every scratch byte it reads, so nothing carries over between calls.
 */
enum { FP4_NOALLOC_SCRATCH_BYTES = 32 << 20 };
fp4_status gemm_w4aX_noalloc(int32_t act, const void* a, int32_t a_dtype, int64_t m, int64_t lda,
                             const fp4_tensor* w, void* c, int32_t c_dtype, int64_t ldc, void* stream);

/*
 * gemm_w4aX_static -- gemm_w4aX (FP4_A4 or FP4_A8 only) with static activation macro-
 * scales: A_hat = dequant(quantize_fp4_static(A, act_macro)), act_macro device uint16
 * [k/256] as for quantize_fp4_static. The micro-scales stay per row and per 16 elements.
 *   workspace >= fp4_workspace_bytes(act, m, n, k) (also for FP4_A4S / FP4_A8S)
 * k <= 21760 (FP4_E_SHAPE otherwise). Source: as for quantize_fp4_static; the policy
 * table's FP4_A4S / FP4_A8S.
 */
fp4_status gemm_w4aX_static(int32_t act, const void* a, int32_t a_dtype, int64_t m, int64_t lda,
                            const uint16_t* act_macro, const fp4_tensor* w, void* c, int32_t c_dtype,
                            int64_t ldc, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gemm_w8a8 -- the product for precision-sensitive layers: C[m x n] = A_hat . W_hat^T with
 * A_hat = dequant(quant_e4m3(A)) (the FP4_A8 activation quantization, dynamic) and W
 * quantized with E4M3 elements (elem FP4_ELEM_E4M3, TILED layout; FP4_E_DTYPE for E2M1
 * weights, FP4_E_LAYOUT for canonical ones). Every product of the two operands is exact;
 * accumulation in float32. c bf16 (round to nearest even) or f32, stride ldc.
 *   workspace >= fp4_workspace_bytes(FP4_W8A8, m, n, k); k <= 21760
 * Source: "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200",
 * section "Deployment Guidelines and Production Safeguards", item 2 (FP8 kept on the most
 * sensitive layers, such as the first layer and the output head).
 */
fp4_status gemm_w8a8(const void* a, int32_t a_dtype, int64_t m, int64_t lda, const fp4_tensor* w, void* c,
                     int32_t c_dtype, int64_t ldc, void* workspace, size_t workspace_bytes, void* stream);

/*
 * grouped_gemm_w4aX -- mixture-of-experts product: for expert e and every routed row r
 * in [expert_offsets[e], expert_offsets[e+1]):
 *     C[r, :] = A_hat[src(r), :] . W_hat_e^T,  src(r) = row_token ? row_token[r] : r
 *   a              device [a_rows x k], row stride lda (bf16 or f32)
 *   row_token      device int32 [total_rows] source row of each routed row, or NULL;
 *                  with a gather the product's operand (bf16 A for FP4_A16, else the
 *                  FP16 workspace copy, a_rows x k) must stay under 4 GiB (FP4_E_SHAPE)
 *   expert_offsets device int32 [n_experts + 1], non-decreasing, [0] = 0,
 *                  [n_experts] = total_rows (checked only in debug builds)
 *   w              quantized weights, experts stacked: rows = n_experts * n, TILED
 *   c              device out [total_rows x n] (bf16/f32), stride ldc
 *   workspace      >= fp4_workspace_bytes(act, a_rows, n, k)
 * k <= 21760 and n % 16 == 0 (FP4_E_SHAPE otherwise, before anything is enqueued).
 * Source: llama.cpp precision-policy page, section "One model can need more than one
 * precision" (the same routing for mixture-of-experts operations).
 */
fp4_status grouped_gemm_w4aX(int32_t act, const void* a, int32_t a_dtype, int64_t a_rows,
                             int64_t lda, const int32_t* row_token,
                             const int32_t* expert_offsets, int32_t n_experts,
                             int64_t total_rows, const fp4_tensor* w, void* c,
                             int32_t c_dtype, int64_t ldc, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * grouped_gemm_w4aX_gated -- the down product of a mixture-of-experts layer with the
 * SiLU-gated activation fused into its dynamic activation quantization: for expert e and
 * routed row r in [expert_offsets[e], expert_offsets[e+1]),
 *     C[r, :] = Q(h[r, :]) . W_hat_e^T,   h = bf16(silu(gate) * up),  silu(x) = x/(1+e^-x)
 * where gate = gate_up[r, 0:k] and up = gate_up[r, k:2k] (k = w->k), silu in float32 (the
 * exponential and reciprocal by the hardware approximations, a few ulp), and Q
 * is the FP4_A4 / FP4_A8 activation quantization of gemm_w4aX (FP4_A16: FP4_E_DTYPE).
 *   gate_up        device bf16 [rows x 2k], row stride ld >= 2k (the gate/up product's
 *                  output in routed-row order)
 *   expert_offsets device int32 [n_experts + 1] as for grouped_gemm_w4aX, [n_experts] = rows
 *   w              quantized down weights, experts stacked: rows = n_experts * n, TILED
 *   c              device out [rows x n] (bf16/f32), stride ldc
 *   workspace      >= fp4_workspace_bytes(act, rows, n, k)
 * k <= 21760 and n % 16 == 0 (FP4_E_SHAPE otherwise, before anything is enqueued).
 * Source: llama.cpp precision-policy page, section "One model can need more than one
 * precision" (W4A4 / W4A8 routing for mixture-of-experts operations). The pages fix no
 * activation function; SiLU gating is the usual reading for gate/up experts.
 */
fp4_status grouped_gemm_w4aX_gated(int32_t act, const void* gate_up, int64_t rows, int64_t ld,
                                   const int32_t* expert_offsets, int32_t n_experts,
                                   const fp4_tensor* w, void* c, int32_t c_dtype, int64_t ldc,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route -- float32 top-k routing of a mixture-of-experts layer (the router is never
 * quantized: ClusterBid FP4 cost guide, section "Where Does FP4 Hurt Accuracy?").
 *   logits         device float32 [tokens x n_experts]; -inf masks an expert out (it
 *                  ranks last, weight 0); NaN ranks with -inf, so the outputs always
 *                  stay a valid routing (the weights are then unspecified)
 *   topk_ids       device out int32 [tokens x top_k]: experts by decreasing logit, equal
 *                  logits in increasing expert id
 *   topk_weights   device out float32 [tokens x top_k]: softmax over the selected logits
 *   expert_offsets device out int32 [n_experts + 1]: routed rows of expert e are
 *                  [offsets[e], offsets[e+1]), tokens in increasing order
 *   row_token      device out int32 [tokens * top_k]: token of each routed row
 *   token_rows     device out int32 [tokens x top_k]: routed row of each choice
 *   workspace      >= moe_route_workspace_bytes(tokens, n_experts), 256-byte aligned
 *                  (expert counts, and five bits per (token, expert): chosen, rank)
 * 1 <= top_k <= min(16, n_experts), n_experts <= 1024, tokens * top_k < 2^31
 * (FP4_E_SHAPE otherwise). Deterministic (no atomics). Buffers are caller-owned.
 */
size_t moe_route_workspace_bytes(int64_t tokens, int32_t n_experts);
fp4_status moe_route(const float* logits, int64_t tokens, int32_t n_experts, int32_t top_k,
                     int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                     int32_t* row_token, int32_t* token_rows, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * moe_combine -- out[t, :] = sum_j topk_weights[t, j] * y[token_rows[t, j], :], float32
 * sums in rank order j = 0 .. top_k-1 (deterministic; a gather, no atomics).
 *   y    device [routed rows x hidden] (bf16/f32), stride ldy; out device [tokens x hidden]
 *   (bf16 round to nearest even / f32), stride ldo; hidden % 8 == 0, 16-byte aligned rows.
 */
fp4_status moe_combine(const void* y, int32_t y_dtype, int64_t ldy, const int32_t* token_rows,
                       const float* topk_weights, int64_t tokens, int32_t top_k, int64_t hidden,
                       void* out, int32_t out_dtype, int64_t ldo, void* stream);

/*
 * KV cache in the two-level FP4 format, and decode attention over it.
 * Sources: "NVIDIA Ships TensorRT-LLM 0.16: Native FP4 Quantization for Blackwell B200"
 * (the codec, section "The Mathematical Breakthrough of Microscopic FP4 Scaling"); "The
 * FP4 Inflection: Rethinking AI Inference Architecture", section "What does this mean for
 * model serving engines?" (a KV cache kept in FP4 cuts its memory footprint and
 * bandwidth, and needs attention kernels written for it); and "AdaLLM Breakthrough:
 * First NVFP4-Only Inference Engine for RTX 4090 Unveiled" (a quantized KV cache with
 * its own decode kernel, grouped-query models).
 *
 * Codec reading: each token's key (value) vector over all KV heads (kv_heads x head_dim
 * elements) is one codec row: E2M1 codes, an E4M3 micro-scale per 16 elements, an FP16
 * macro-scale per 256 (a pair of heads). head_dim must be 128, kv_heads even and <= 32,
 * max_tokens a multiple of 32 and at most 2^24 (FP4_E_SHAPE otherwise).
 *
 * Device layout (all arrays caller-owned device memory, T = max_tokens):
 *   k_codes [n_seq][kv_heads][T][64 B]: per token-head, dword 4g + s holds the codes of
 *           d = 32s + 8g .. 32s + 8g + 7 (low nibble first), g, s in 0..3;
 *   k_micro [n_seq][kv_heads][T][8]: micro-scale of block d / 16;
 *   k_macro [n_seq][kv_heads / 2][T]: FP16 bits of the head pair's macro-scale;
 *   v_codes [n_seq][kv_heads][T / 32][128][16 B]: tiles of 32 tokens, transposed: byte
 *           16 d + m of a tile holds slots 2m (low nibble) and 2m + 1 of column d;
 *   v_micro [n_seq][kv_heads][T / 32][8][32]: micro-scale of block b for each slot;
 *   v_macro [n_seq][kv_heads / 2][T].
 * Slot 8g + i (g in 0..3, i in 0..7) of a tile is its token 4g + i for i < 4 and
 * 16 + 4g + i - 4 for i >= 4. Alignment: codes 16 bytes, micro and macro 8 bytes.
 * fp4_kv_cache_bytes(.., part) gives each array's size (the K and V arrays of one part
 * have equal sizes); 0 for an unsupported shape.
 */
typedef struct {
  void* k_codes;
  uint8_t* k_micro;
  uint16_t* k_macro;
  void* v_codes;
  uint8_t* v_micro;
  uint16_t* v_macro;
  int32_t n_seq;
  int32_t max_tokens;
  int32_t kv_heads;
  int32_t head_dim;
} fp4_kv_cache;

enum { FP4_KV_CODES = 0, FP4_KV_MICRO = 1, FP4_KV_MACRO = 2 };

size_t fp4_kv_cache_bytes(int32_t n_seq, int32_t max_tokens, int32_t kv_heads, int32_t head_dim,
                          int32_t part);

/*
 * kv_cache_append -- quantize n_new new tokens per sequence into the cache: rows
 * b * n_new + i of k_new and v_new (device, FP4_BF16 or FP4_F32, row stride ld >=
 * kv_heads * head_dim elements, 16-byte aligned rows) become token positions[b] + i of
 * sequence b (positions: device int32 [n_seq]). Other tokens keep their contents. Tokens
 * at or past max_tokens, and sequences with a negative position, are skipped on the
 * device. 1 <= n_new <= 2^20.
 */
fp4_status kv_cache_append(const fp4_kv_cache* cache, const void* k_new, const void* v_new,
                           int32_t dtype, int64_t ld, const int32_t* positions, int32_t n_new,
                           void* stream);

/*
 * attention_decode_fp4kv -- one decode step of attention for every sequence:
 *   out[b, h, :] = sum_{t < L_b} softmax_t(scale * q[b, h, :] . K_hat[b, t, kv(h), :])
 *                  * V_hat[b, t, kv(h), :],   kv(h) = h / (q_heads / kv_heads),
 * K_hat, V_hat the dequantized cache and L_b = lengths[b] (device int32, clamped to
 * [0, max_tokens]; L_b = 0 gives zeros).
 *   q         device bf16 [n_seq][q_heads][128], 16-byte aligned; q_heads a multiple of
 *             kv_heads with at most 16 query heads per KV head
 *   out       device [n_seq][q_heads][128], FP4_BF16 (round to nearest even) or FP4_F32
 *   workspace >= attention_workspace_bytes(n_seq, q_heads, max_tokens), 256-byte aligned
 * Scores are exact products of the cache values and q (q is rescaled by a power of two
 * per head into FP16) accumulated in float32; softmax weights enter the value product as
 * a pair of FP16 values (about 2^-22 relative); the result is accumulated in float32.
 */
size_t attention_workspace_bytes(int32_t n_seq, int32_t q_heads, int32_t max_tokens);
fp4_status attention_decode_fp4kv(const void* q, int32_t q_heads, const fp4_kv_cache* cache,
                                  const int32_t* lengths, float scale, void* out, int32_t out_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * MX-native FP4 -- not the two-level format: E2M1 codes with one E8M0 power-of-two scale
 * per 32 consecutive elements of a row (OCP microscaling reading: e = floor(log2 max|x|)
 * - 2, clamped to [-127, 127], -127 for an all-zero block; codes = x / 2^e rounded to
 * nearest E2M1, ties to even, saturating at 6, sign kept). It is the format the block-
 * scaled FP4 matrix instruction of gfx950 consumes, kept beside the pages' format to
 * measure the FP4 matrix path and its accuracy against the two-level format; the pages'
 * E4M3-per-16 micro-scales and FP16 macro-scales have no exact E8M0-per-32 form (the
 * hardware applies powers of two only).
 * Tiled layout (rows padded to a multiple of 16; k % 128 == 0): tile T = (r/16)*(k/128)
 * + c/128 of 16 rows x 128 columns; codes at T*1024 + kb*256 + (r%16)*16 + (c%32)/2 with
 * kb = (c%128)/32 (low nibble = even c), scales (E8M0 bytes) at T*64 + kb*16 + r%16.
 * mxfp4_bytes(rows, k, FP4_MX_CODES / FP4_MX_SCALES) gives the sizes (0 when k % 128 or
 * rows < 1). All buffers are caller-owned device memory.
 *
 * quantize_mxfp4 -- x device [rows x k] (FP4_BF16 or FP4_F32, finite, stride ldx, 16-byte
 *   aligned rows) -> codes (16-byte aligned), scales; padding rows get zeros.
 * gemm_mxfp4 -- C[m x n] = A_hat . W_hat^T, A and W quantized by quantize_mxfp4 (m and n
 *   the real row counts), float32 accumulation by the matrix core; C FP4_BF16 (round to
 *   nearest even) or FP4_F32, row stride ldc.
 */
enum { FP4_MX_CODES = 0, FP4_MX_SCALES = 1 };
size_t mxfp4_bytes(int64_t rows, int64_t k, int32_t part);
fp4_status quantize_mxfp4(const void* x, int32_t x_dtype, int64_t rows, int64_t k, int64_t ldx, void* codes,
                          uint8_t* scales, void* stream);
fp4_status gemm_mxfp4(const void* a_codes, const uint8_t* a_scales, int64_t m, const void* w_codes,
                      const uint8_t* w_scales, int64_t n, int64_t k, void* c, int32_t c_dtype, int64_t ldc,
                      void* stream);

/* Bytes of device workspace gemm_w4aX / grouped_gemm_w4aX / gemm_w4aX_static / gemm_w8a8
 * need for a precision code (0 for FP4_A16; FP4_A4S as FP4_A4; FP4_A8S, FP4_W8A8 as FP4_A8). */
size_t fp4_workspace_bytes(int32_t act, int64_t m_or_rows, int64_t n, int64_t k);

/*
 * fp4_policy_select -- per-layer precision policy: FP4_POLICY_Q4 -> FP4_A4,
 * FP4_POLICY_Q8 -> FP4_A8, FP4_POLICY_AUTO -> (layer_flag ? FP4_A8 : FP4_A4),
 * FP4_POLICY_SENSITIVE_W8 -> (layer_flag ? FP4_W8A8 : FP4_A4) (FP8 kept on flagged
 * layers: TensorRT-LLM FP4 page, section "Deployment Guidelines and Production
 * Safeguards", item 2), FP4_POLICY_STATIC -> (layer_flag ? FP4_A8S : FP4_A4S)
 * (calibrated activation macro-scales).
 * Returns -FP4_E_MODE for an unknown mode. Source: llama.cpp precision-policy page,
 * section "Local inference is becoming a policy engine" (q4 / q8 / auto).
 */
int32_t fp4_policy_select(int32_t mode, int32_t layer_flag);

/* Static, human-readable name of a status code. */
const char* fp4_status_string(fp4_status status);

/* Device check without launching anything: FP4_OK on gfx950, else the error code. */
fp4_status fp4_device_check(void);

/*
 * fp4_product_kernel -- diagnostics: the kernel form a product call of this shape runs
 * on the current device (the choice depends on its compute-unit count), as a static
 * string, or NULL when the call would return FP4_E_SHAPE. Enqueues nothing.
 *   act, a_dtype  as for gemm_w4aX (the policy codes FP4_A4S / FP4_A8S / FP4_W8A8 map to
 *                 their activation precision)
 *   m, n, k       the product's rows (grouped: total routed rows), columns (grouped: per
 *                 expert) and reduction length
 *   grouped       nonzero for grouped_gemm_w4aX / grouped_gemm_w4aX_gated, n_experts
 *   w_e4m3        nonzero for gemm_w8a8 (E4M3 weights; act must be FP4_A8 or FP4_W8A8)
 */
const char* fp4_product_kernel(int32_t act, int32_t a_dtype, int64_t m, int64_t n, int64_t k,
                               int32_t grouped, int32_t n_experts, int32_t w_e4m3);

#ifdef __cplusplus
}
#endif
#endif /* FP4_E2M1_H */
