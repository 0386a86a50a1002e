"""Seeded synthetic inputs for split-KV paged decode attention.

This module only *creates* inputs: random values, their storage encodings
(bf16 bits, int8 codes, fp8 e4m3 codes plus fp32 scales), page pools with a
random page table, NaN poisoning of unused storage, and the five workload
shapes. It holds none of the attention arithmetic, so both the fp64 oracle and
the HIP path can consume what it produces without sharing any of the method.
"""

from .configs import CONFIGS, ProblemSpec, config_spec, small_spec
from .problem import Problem, make_problem, extract_request, to_contiguous

__all__ = [
    "CONFIGS",
    "ProblemSpec",
    "config_spec",
    "small_spec",
    "Problem",
    "make_problem",
    "extract_request",
    "to_contiguous",
]
