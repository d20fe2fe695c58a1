"""Seeded synthetic workloads for the fused MoE expert FFN (see synth.moe_inputs)."""
from .moe_inputs import CONFIGS, MoEInputs, make_inputs, config_inputs, fingerprint  # noqa: F401
