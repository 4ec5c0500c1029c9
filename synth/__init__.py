"""Seeded synthetic video-attention inputs and named workloads.

This module holds no step of the attention method: it only draws random
tensors and names the workload shapes.  Both the HIP path's tests/bench and
the CPU oracle's tests consume the tensors it produces.
"""
from .fields import smooth_field_qkv, smooth_field  # noqa: F401
from .configs import CONFIGS, Workload, get  # noqa: F401
