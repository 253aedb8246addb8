"""CPU oracle of the LM-head logits projection (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the library. See ``lmhead_oracle`` for the definitions it follows.
"""
from .lmhead_oracle import (bf16_to_f64, dot_f64, e2m1_to_f64, e4m3_to_f64, f16_to_f64,
                            f32_to_bf16_rne, f64_to_bf16_correct, f64_to_f16_correct,
                            f64_to_f32_round_to_odd, lmhead_logits, lmhead_logits_nvfp4,
                            lmhead_rowreduce, logits_bf16, quantize_nvfp4, e2m1_rne,
                            f32_to_e4m3_rne, logits_f16, logits_f32,
                            nvfp4_weight_f64, row_reduce, ulp_bf16, ulp_f16, unpack_e2m1)

__all__ = [
    "bf16_to_f64", "dot_f64", "e2m1_to_f64", "e4m3_to_f64", "f16_to_f64", "f32_to_bf16_rne",
    "f64_to_bf16_correct", "f64_to_f16_correct", "f64_to_f32_round_to_odd", "lmhead_logits",
    "lmhead_logits_nvfp4", "lmhead_rowreduce", "logits_bf16", "logits_f16", "logits_f32",
    "nvfp4_weight_f64", "row_reduce", "quantize_nvfp4", "e2m1_rne", "f32_to_e4m3_rne", "ulp_bf16", "ulp_f16", "unpack_e2m1",
]
