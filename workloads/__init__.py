"""Seeded synthetic workloads for the tree-verification step.

Shared by the tests, the benchmark and the oracle's callers; holds input
generation only (shapes, random draws, tree topologies), none of the
verification arithmetic.
"""
from .configs import CONFIGS, VerifyConfig, get  # noqa: F401
from .generate import (StepInputs, default_seed, f32_to_bf16_bits, make_step,  # noqa: F401
                       normal_bf16_device, shrink)
from . import trees  # noqa: F401
