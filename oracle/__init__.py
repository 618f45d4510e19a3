"""CPU oracle of the quantized attention path: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously checkable NumPy implementation of what the HIP path
computes, used to prove the GPU results.  Only the tests, the smoke check and
the CPU-baseline leg of the benchmark may import it; the library and its
Python binding never do, and it shares no code with them.

Pins (the checks that tie the oracle to something other than itself) live in
``tests/test_oracle_*.py``.  Parity against the pages is unpinned: the pages
print no worked value for any step of the method.
"""
from .formats import BF16, E2M1, E4M3, bf16_bits_to_f64, decode, encode, f64_to_bf16_bits, round_to
from .qsdpa import (E8M0_BIAS, FP4, FP4_GROUP, FP8, MX_BLOCK, MXFP4, P_SCALE, SOFTMAX_STEP, Quantized, attend,
                    channel_stats, dequantize_qk, exact_attention, forward, online_softmax_av, quantize,
                    quantize_fp4_groups, quantize_fp8_blocks, quantize_mxfp4_blocks, quantize_v, smooth_k,
                    unpack_fp4, VC_RHO, vc_count, vc_forward, vc_select, vc_token_error)

__all__ = [
    "BF16", "E2M1", "E4M3", "E8M0_BIAS", "FP4", "FP4_GROUP", "FP8", "MXFP4", "MX_BLOCK", "P_SCALE",
    "SOFTMAX_STEP", "Quantized", "quantize_mxfp4_blocks",
    "attend", "bf16_bits_to_f64", "channel_stats", "decode", "dequantize_qk", "encode",
    "exact_attention", "f64_to_bf16_bits", "forward", "online_softmax_av", "quantize",
    "quantize_fp4_groups", "quantize_fp8_blocks", "quantize_v", "round_to", "smooth_k", "unpack_fp4",
    "VC_RHO", "vc_count", "vc_forward", "vc_select", "vc_token_error",
]
