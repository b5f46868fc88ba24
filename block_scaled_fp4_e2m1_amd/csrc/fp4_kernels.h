// Kernel launchers of the gfx950 library (host side). Each returns the HIP error of the
// launch; all of them enqueue on the given stream and never synchronize.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4lib {

// Whether the quantize / activation-pass grid (one 256-thread block per 16 (row, group)
// pairs) and the dequantize grid fit one launch; the launchers refuse exactly these.
bool quantize_grid_ok(int64_t rows, int64_t k);
bool dequantize_grid_ok(int64_t rows, int64_t k);

// macro_in (optional): static macro-scales, FP16 bits per 256-column group shared by all
// rows (nullptr: each row's own groups, the dynamic rule).
hipError_t launch_quantize(const void* x, int in_bf16, int64_t rows, int64_t k, int64_t ldx,
                           int elem_e4m3, int tiled, uint8_t* codes, uint8_t* micro,
                           uint16_t* macro, const uint16_t* macro_in, hipStream_t st);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                             int64_t rows, int64_t k, int elem_e4m3, int tiled, void* y,
                             int out_bf16, int64_t ldy, hipStream_t st);

// Canonical <-> tiled repack of a quantized tensor (rows % 16 == 0, k % 256 == 0): a
// byte permutation of codes, micro- and macro-scales. hipErrorInvalidValue outside
// repack_supports().
bool repack_supports(int64_t rows, int64_t k, int elem_e4m3);
hipError_t launch_repack(const uint8_t* src_codes, const uint8_t* src_micro, const uint16_t* src_macro,
                         uint8_t* dst_codes, uint8_t* dst_micro, uint16_t* dst_macro, int64_t rows, int64_t k,
                         int elem_e4m3, int to_tiled, hipStream_t st);

// Activation pass for the matrix kernels: aq[r, c] * scale[r, c/256] == A_hat[r, c].
// macro_in as for launch_quantize.
hipError_t launch_act_prep(const void* a, int in_bf16, int64_t rows, int64_t k, int64_t lda,
                           int elem_e4m3, _Float16* aq, int64_t ldq, float* scale,
                           const uint16_t* macro_in, hipStream_t st);

// Static activation macro-scale calibration: amax[g] = max(amax[g], max |x[:, g]|), then
// macro[g] = the dynamic macro rule on amax[g] (0 for a zero maximum).
hipError_t launch_act_calibrate(const void* x, int in_bf16, int64_t rows, int64_t k, int64_t ldx,
                                int elem_e4m3, float* amax, uint16_t* macro, hipStream_t st);

// Gated form: a row holds gate in [0, k) and up in [k, 2k) (bf16, row stride lda >= 2k);
// the operand is h = bf16(silu(gate) * up).
hipError_t launch_act_prep_gated(const uint16_t* a, int64_t rows, int64_t k, int64_t lda, int elem_e4m3,
                                 _Float16* aq, int64_t ldq, float* scale, hipStream_t st);

// Decode product for m <= 8 bf16 activation rows against tiled E2M1 weights [n x k].
// Returns hipErrorInvalidValue when the shape is outside what the kernel covers.
// Compute units of the current device (cached per device).
int device_cus();
bool gemv_supports(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_bf16(const uint16_t* a, int64_t lda, int64_t m, int64_t k,
                            const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                            int64_t n, void* c, int out_bf16, int64_t ldc, hipStream_t st);

// Dense / grouped product on MFMA. The A operand is either the FP16 output of
// launch_act_prep (with its per-group factors) or raw bf16 activations (factor 1).
// For the grouped form, rows of expert e are expert_offsets[e] .. expert_offsets[e+1]
// of the routed list; row_token (optional) maps a routed row to its source row of A.
struct GemmArgs {
  const void* a;            // _Float16 (a_is_bf16 == 0) or bf16 bits
  int a_is_bf16;
  int64_t lda;              // elements
  const float* a_scale;     // [a_rows x k/256] or nullptr (== 1)
  int64_t m;                // rows of C (dense) / total routed rows (grouped)
  int64_t n, k;
  const uint8_t* codes;     // tiled E2M1 (or, w_e4m3, E4M3) weights; experts stacked along rows
  const uint8_t* micro;
  const uint16_t* macro;
  void* c;
  int c_is_bf16;
  int64_t ldc;
  const int32_t* row_token;       // grouped only, may be nullptr
  const int32_t* expert_offsets;  // grouped only; nullptr for a dense product
  int32_t n_experts;
  int w_e4m3;               // E4M3 weights (dense, FP16 activation operand only)
  // a_packed: the activations are E2M1 in the canonical layout (quantize_fp4's output):
  // a = codes (k/2 bytes per row), a_micro, a_macro; a_is_bf16, lda and a_scale unused.
  // Only the 128-row-wave form takes them (gemm_packed_a4 says when it runs).
  int a_packed;
  const uint8_t* a_micro;
  const uint16_t* a_macro;
};
// Reduction lengths the product kernel covers (its per-group tables fit in LDS).
bool gemm_supports(int64_t k);
// Whether launch_gemm covers a product of this shape (k within gemm_supports, a grid that
// fits one launch); grouped: m = total routed rows. launch_gemm refuses exactly these.
bool gemm_plan_ok(int64_t m, int64_t n, int64_t k, int grouped, int n_experts, int w_e4m3);
// Name of the kernel form launch_gemm selects for that shape (nullptr when refused).
const char* gemm_kernel_name(int64_t m, int64_t n, int64_t k, int grouped, int n_experts, int w_e4m3);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
// The 128-row-wave form for large dense E2M1 products (128 x 256 workgroup tiles, one per
// CU): the shapes it covers (its LDS holds three operand stages and the row-factor table:
// k <= 8192) and its launcher (hipErrorInvalidValue outside gemm_r8_supports()).
bool gemm_r8_supports(int64_t m, int64_t n, int64_t k);
// Whether a dense E2M1-weight product of this shape runs on the 128-row-wave form, which
// takes W4A4 activations packed (quantize_fp4's canonical output) and decodes them itself.
bool gemm_packed_a4(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_r8(const GemmArgs& g, hipStream_t st);

// Plain float32 product for float32 activations (small shapes): one thread per output.
hipError_t launch_gemm_f32act(const float* a, int64_t lda, int64_t m, int64_t k,
                              const uint8_t* codes, const uint8_t* micro, const uint16_t* macro,
                              int64_t n, void* c, int out_bf16, int64_t ldc, hipStream_t st);

// Mixture-of-experts routing: top_k experts per token (float32 logits [tokens x E]),
// softmax weights over the selected logits, routed rows ordered by (expert, token).
// workspace (256-byte aligned, route_workspace_bytes) holds the int32 expert counts and
// five 64-bit-word bit-planes per token and 64 experts (chosen, 4 rank bits). hipErrorInvalidValue outside route_supports().
bool route_supports(int n_experts, int top_k);
size_t route_workspace_bytes(int64_t tokens, int n_experts);
hipError_t launch_moe_route(const float* logits, int64_t tokens, int n_experts, int top_k,
                            int32_t* topk_ids, float* topk_w, int32_t* offsets, int32_t* row_token,
                            int32_t* token_rows, void* workspace, hipStream_t st);

// KV cache in the two-level FP4 format (layout: see attention.hip). max_tokens % 32 == 0,
// kv_heads even and <= 32, head_dim 128.
struct KvCacheArgs {
  uint8_t* k_codes;
  uint8_t* k_micro;
  uint16_t* k_macro;
  uint8_t* v_codes;
  uint8_t* v_micro;
  uint16_t* v_macro;
  int n_seq;
  int64_t max_tokens;
  int kv_heads;
};
bool kv_cache_supports(int max_tokens, int kv_heads, int head_dim);
size_t attention_partial_bytes(int64_t n_seq, int q_heads, int64_t max_tokens);
// n_new tokens per sequence b at positions[b] .. +n_new-1 (rows b * n_new + i of k_new /
// v_new, row stride ld elements); writes past max_tokens are skipped.
hipError_t launch_kv_append(const KvCacheArgs& c, const void* k_new, const void* v_new, int in_bf16,
                            int64_t ld, const int32_t* positions, int n_new, hipStream_t st);
// q bf16 [n_seq][q_heads][128]; out [n_seq][q_heads][128]; partial: attention_partial_bytes.
hipError_t launch_attention_decode(const KvCacheArgs& c, const uint16_t* q, int q_heads,
                                   const int32_t* lengths, float scale, float* partial, void* out,
                                   int out_bf16, hipStream_t st);

// MX-native FP4 (E2M1, E8M0 per 32; tiled layout: see mx.hip). rows padded to 16.
int64_t mx_padded_rows(int64_t rows);
hipError_t launch_mx_quantize(const void* x, int in_bf16, int64_t rows, int64_t k, int64_t ldx, uint8_t* codes,
                              uint8_t* scales, hipStream_t st);
hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, const uint8_t* w_codes,
                          const uint8_t* w_scales, int64_t n, int64_t k, void* c, int out_bf16, int64_t ldc,
                          hipStream_t st);

// out[t, :] = sum_j w[t, j] * y[token_rows[t, j], :] (float32, j in order); hidden % 8 == 0.
hipError_t launch_moe_combine(const void* y, int in_bf16, int64_t ldy, const int32_t* token_rows,
                              const float* topk_w, int64_t tokens, int top_k, int64_t hidden,
                              void* out, int out_bf16, int64_t ldo, hipStream_t st);

}  // namespace fp4lib
