"""Seeded synthetic workloads for the sparse-decode path.

This package only draws numbers and names shapes. It holds none of the
methods' arithmetic (no scores, no softmax, no selection), so both the HIP
path and the CPU oracle can take their inputs from it without sharing any
computation.
"""
from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from . import generator  # noqa: F401
