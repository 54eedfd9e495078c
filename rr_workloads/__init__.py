"""Seeded synthetic workloads for the RRAttention sparse-prefill path.

This package holds the attention shapes of the five measured workloads and a
deterministic generator of bf16 Q/K/V tensors for them.  It contains none of
the method's arithmetic (no scoring, softmax, pooling, selection or
attention); it is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.
"""
from .configs import CONFIGS, Workload, get_config  # noqa: F401
from .gen import generate, bf16_bits_to_f32, f32_to_bf16_bits  # noqa: F401
