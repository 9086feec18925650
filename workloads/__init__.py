"""Seeded synthetic inputs for the verification step.

This module serves both the GPU path's tests/bench and the oracle.  It holds
none of the verification method's arithmetic: it only draws logits, Q/K/V,
lengths, uniforms and int8 cache codes with their scales, rounds fp32 to bfloat16 (round-to-nearest-even), and
samples draft tokens from the draft distribution with the Gumbel-max trick
(argmax of z/T plus Gumbel noise), which is the draft model's job, not the
verifier's, and uses none of the verifier's steps.

Shapes follow the pages' workloads (see ``configs.CONFIGS``); no page data or
trained weights exist here, so every tensor is synthetic.
"""

from .configs import CONFIGS, Config, get  # noqa: F401
from .gen import (  # noqa: F401
    attention_inputs,
    attention_inputs_device,
    attention_inputs_int8,
    attention_inputs_int8_device,
    bf16_bits,
    bf16_bits_to_f32,
    repeated_row_inputs,
    sampler_inputs,
    sampler_inputs_device,
)
