"""Seeded synthetic inputs for tree-masked verification.

This module only draws random inputs (trees, draft tokens, logits, Q/K/V,
prefix lengths, cache bit patterns).  It contains none of the verification
arithmetic, so that the GPU library and the CPU oracle can both be fed from it
without sharing any computation.
"""
from .gen import *  # noqa: F401,F403
from .workloads import WORKLOADS, Workload, workload  # noqa: F401
