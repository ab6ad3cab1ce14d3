"""CPU oracle for the NF4 QLoRA linear layer. TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct reference of what the hot path computes, written from the pages'
statement of the method (chiefly "QLoRA, explained": the sections on blockwise absmax quantisation,
NormalFloat 4, double quantisation, the forward pass and gradients and the quality loss at merge
time and the training loop around the layer, plus its worked example and toy run). Floating point is float64 unless a step fixes a
narrower type (the fp32 codebook, fp32 scales, the bf16 dequantised weight), and the integer
decisions (nearest code, nearest 8-bit float) are taken in exact arithmetic.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package. It shares no code, header, table or constant with the HIP path
(``bit_nf4_quantised_amd``) and imports nothing from it.

Every function here has a pin in ``tests/test_oracle_*.py`` that checks it against something other
than itself: the pages' printed worked example, codes and toy statistics, exact rational brute force,
torch's own float8/bfloat16 casts, closed forms and finite differences. None is "parity unpinned".
"""
from .nf4 import (NF4_ZERO_INDEX, codebook, quantize_blocks, pack_nibbles, unpack_nibbles,
                  quantize, e4m3_value, e4m3_unit_values, double_quant, dequant_scales,
                  bf16_bits_from_f32, f32_from_bf16_bits, dequant, storage_bits, quantize_with,
                  dequant_blocks)
from .linear import linear_fwd, linear_bwd, linear_fwd_f64, linear_bwd_f64, linear_bwd_sampled
from .merge import bf16_bits_from_f64, merge
from .optim import AdamWConfig, global_grad_norm, clip_coefficient, adamw_step
from .toy import int4_codebook, fp4_codebook, relative_mse, residual_capture

__all__ = [
    "NF4_ZERO_INDEX", "codebook", "quantize_blocks", "pack_nibbles", "unpack_nibbles", "quantize",
    "e4m3_value", "e4m3_unit_values", "double_quant", "dequant_scales", "bf16_bits_from_f32",
    "f32_from_bf16_bits", "dequant", "storage_bits", "quantize_with", "dequant_blocks", "linear_fwd", "linear_bwd", "linear_fwd_f64",
    "linear_bwd_f64", "linear_bwd_sampled", "bf16_bits_from_f64", "merge", "AdamWConfig",
    "global_grad_norm", "clip_coefficient", "adamw_step", "int4_codebook",
    "fp4_codebook", "relative_mse", "residual_capture",
]
