"""Seeded synthetic inputs for the GQA + RoPE attention path.

This package holds only the workload definitions and the seeded random draws
(tensors, document cuts, cache lengths). It contains none of the method's
arithmetic: no rotation, no scores, no softmax. Both the fp64 oracle and the
HIP path take their inputs from here, and nothing else is shared between them.
"""

from .configs import CONFIGS, Workload, get  # noqa: F401
from .gen import (  # noqa: F401
    draw_grad_output,
    draw_cu_docs,
    draw_decode_inputs,
    draw_prefill_inputs,
    draw_positions,
    draw_seq_lens,
    sample_rows,
    torch_dtype,
)
