"""CPU oracle for two-level block-scaled FP4 (E2M1 elements, E4M3 micro-scales per 16,
FP16 macro-scales per 256), the W4A16 / W4A8 / W4A4 products built on it, the
mixture-of-experts layer steps around the grouped product (routing, gated activation,
combine), decode attention over a KV cache kept in the same format, the MX-native FP4
variant (E8M0 power-of-two scale per 32) with its product, and the paths for sensitive
layers (W8A8) and calibrated (static) activation macro-scales.

TEST INFRASTRUCTURE ONLY. A plain, slow, float64 numpy restatement of the method that
the HIP library is checked against. It shares no code with the library. Only tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it.

Pins (tests that tie this oracle to something other than itself) live in
``tests/test_oracle_*.py``. No function here is "parity unpinned".
"""
from .formats import (E2M1, E4M3, FP16, BF16, round_to_grid, e2m1_decode, e4m3_decode,
                      e4m3_encode, fp16_bits, fp16_from_bits, bf16_round, bf16_bits)
from .quant import (quantize, dequantize, pack_e2m1, unpack_e2m1, element_values,
                    QuantizedTensor, BLOCK, GROUP)
from .gemm import (activation_values, gemm, gemm_bf16, grouped_gemm, policy_select,
                   A16, A8, A4, POLICY_AUTO, POLICY_Q4, POLICY_Q8)
from .moe import route, silu_gate, combine
from .attention import kv_quantize_rows, kv_dequantize_rows, attention_decode
from .mx import MX_BLOCK, e8m0_value, mx_quantize, mx_dequantize, mx_gemm
from .sensitive import (W8A8, A4S, A8S, POLICY_SENSITIVE_W8, POLICY_STATIC, calibrate_macro,
                        quantize_static, activation_values_static, gemm_w8a8, gemm_static,
                        policy_select_ext)
