"""Seeded synthetic workloads for the fused MoE expert FFN (see synth.moe_inputs)."""
from .moe_inputs import (CONFIGS, MoEInputs, config_inputs, draw_topk_ids,  # noqa: F401
                         fingerprint, make_inputs)
