"""Seeded synthetic inputs for the sparse-linear attention forward pass.

This package only draws random tensors of the shapes and value structure of the
video-DiT attention workloads. It contains none of the attention method's
arithmetic, so both the HIP path and the float64 oracle can take their inputs
from it without sharing any computation.
"""

from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from .synth import Inputs, make_inputs, make_proj_o, sincos_posemb  # noqa: F401
