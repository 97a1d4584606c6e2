"""CPU oracle for the continuous-batching decode step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the
HIP path; the two meet only in the seeded inputs drawn by ``synth``.

The oracle is the plain per-sequence definition of the step described on the
page "Continuous Decode Batching - the transformer capture" (section
"decode_step_batch - paint-by-numbers"): every row embeds its last token,
runs the decoder body with RoPE at its own position t_s, appends its K/V to
its own slab at t_s, attends to its own history [0..=t_s], and gets
lm_head logits; then its position advances by one. The segmented prefill of
the same page (section "REVISED ... forward_batch_segmented") is each
segment's causal forward with segment-local positions from 0, with no
attention across segments. Arithmetic is float64 throughout; storage
precision follows the model (bf16 weights, bf16 K/V slabs, or affine 8-bit K/V
slabs from ``kvquant``). ``sampling`` holds the seeded temperature / top-p
selection of a row's token.
"""
from .model import (OracleModel, SeqState, bf16_bits_to_f64, round_to_bf16, f64_to_bf16_bits,
                    rmsnorm, rope_angles, apply_rope, attend_one_head, silu, dequant_int4,
                    greedy)
from .sampling import philox4x64_10, uniform_draw, nucleus_order, sample_row, sample_rows
from .kvquant import quantize_affine8, quantize_affine4, dequantize_affine8

__all__ = ["OracleModel", "SeqState", "bf16_bits_to_f64", "round_to_bf16", "f64_to_bf16_bits",
           "rmsnorm", "rope_angles", "apply_rope", "attend_one_head", "silu", "dequant_int4",
           "greedy", "philox4x64_10", "uniform_draw", "nucleus_order", "sample_row", "sample_rows",
           "quantize_affine8", "quantize_affine4", "dequantize_affine8"]
