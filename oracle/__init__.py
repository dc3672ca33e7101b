"""CPU oracle for the batch-1 talker decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test suite, the smoke check and the CPU-baseline leg of the benchmark
call it.  It shares no code with the HIP library.

The decode step it computes is the plain forward pass of a Qwen3-style decoder
(embedding fetch, attention, MLP, norms, sampling; dev.to article "Porting a
1,200-line persistent CUDA megakernel to Qwen3-TTS", section "The idea: one
kernel that never exits"), with the talker's changes from the same article's
section "Porting it to Qwen3-TTS-1.7B" (untied LM head, multi-section rotary
embedding) and the theaicatchup article's section "Why Does a Single Kernel
Even Matter for TTS?" (inputs summed from 17 embeddings, read through a
negative sentinel id).  Every step is exact up to rounding order, so the oracle
is that definition written out, in float64 unless a caller asks otherwise.
"""
from .decoder import (  # noqa: F401
    Decoder,
    argmax_lowest,
    bf16_bits_to_float,
    bf16_round,
    embed_sum17,
    gqa_decode_attention,
    rms_norm,
    rope_angles,
    rotate_half_apply,
    silu,
    top2_margin,
)
