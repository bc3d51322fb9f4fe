"""Seeded synthetic workloads for the DDTree tree-verify path.

This package draws random inputs and lays them out in the shapes the verify
step consumes.  It holds none of the method's own arithmetic (no log-softmax or
top-k selection, no tree search, no masking, no attention, no acceptance): both the CPU oracle and the HIP path
are fed from here, and neither imports the other.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_workload,
    draw_target_predict,
    draw_drafter_topk,
    draw_drafter_logits,
    draw_target_probs,
    draw_layer,
    sensitize_tree_columns,
)
