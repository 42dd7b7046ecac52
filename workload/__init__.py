"""Seeded synthetic workloads for the draft-correction pass.

This package holds the shapes of the benchmark configurations and a seeded
input generator.  It contains none of the corrector's arithmetic: it only
draws random inputs and weights, rounds them to bfloat16 where a tensor is
stored in bfloat16, and lays them out in memory.  Both the CPU oracle and the
GPU path consume exactly the arrays produced here.
"""

from .configs import CONFIGS, config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gen_inputs,
    gen_targets,
    gen_weights,
)
