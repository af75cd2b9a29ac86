"""Seeded synthetic inputs shaped like SparSTAR's late 720p refinement scales.

This package only draws random numbers and lays them out; it holds none of
the method's arithmetic (no means, scores, selection or attention).  Both the
CPU oracle and the HIP path read their inputs from here.
"""
from .configs import CONFIGS, Workload, workload, sweep_workloads
from .generate import make_inputs, bf16_bits_from_f32

__all__ = ["CONFIGS", "Workload", "workload", "sweep_workloads",
           "make_inputs", "bf16_bits_from_f32"]
