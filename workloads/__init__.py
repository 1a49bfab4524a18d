"""Seeded synthetic workloads shared by the oracle, the tests and the benchmark.

This package holds data only: the five workload shapes, their block-mask
specifications (as plain segment descriptions) and the seeded input
generators.  It contains none of the attention arithmetic, none of the mask
evaluation and none of the block-index construction; the oracle and the HIP
library each implement those on their own.
"""

from .configs import (  # noqa: F401
    SEG_FULL, SEG_BLOCKWIN, SEG_IMAGE2D, SEG_VIDEO3D,
    Segment, MaskSpec, PrefillWorkload, DecodeWorkload,
    CONFIGS, get_config,
)
from .generate import (  # noqa: F401
    sinusoidal_position, gen_prefill_inputs, gen_prefill_grad_output, gen_decode_inputs,
    gen_decode_sequence,
)
