"""Seeded synthetic workloads for the recurrent-state decode step.

This module only draws random inputs of the shapes and distributions of the
decode workloads; it holds none of the decode method's arithmetic and is the
one piece of code that both the GPU path's callers and the CPU oracle's
callers use.
"""
from .gen import SWEEP_B, WORKLOADS, Workload, generate, generate_workload, seed_for  # noqa: F401
