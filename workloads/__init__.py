"""Seeded synthetic workloads for the batched LoRA-delta apply.

This package only draws inputs: adapter ranks and scales, factors, token
adapter ids, activations.  It holds none of the apply's arithmetic, so the
CPU oracle and the HIP path can both consume it without sharing any code
that computes the result.
"""
from .configs import (  # noqa: F401
    CONFIG_KEYS,
    FLEET_INPUT_DIMS,
    FLEET_LAYERS,
    FLEET_PROJECTIONS,
    Module,
    Workload,
    base_weight,
    bf16_bits,
    fleet_base_weight,
    fleet_ids,
    fleet_module_shapes,
    fleet_ranks,
    fleet_x,
    make_config,
    make_fleet_module,
    make_integer_workload,
    make_random_workload,
    round_to_bf16,
    timing_y0,
    zipf_ids,
)
from .jd import JD_CONFIGS, JDWorkload, make_jd_config, make_jd_workload  # noqa: F401,E402
from .rsvd import RSVD_CONFIGS, RsvdWorkload, make_rsvd_config, make_rsvd_workload  # noqa: F401,E402
