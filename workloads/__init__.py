"""Seeded synthetic decode workloads for the LoReS quantized recurrent-state step.

This module only draws inputs (q, k, v, alpha, beta) with the shapes and value
distributions of the decode workloads the LoReS pages name (Gated DeltaNet,
Mamba-2 / SSD, KDA-style layers).  It holds none of the method's arithmetic:
no state, no quantizer, no rounding noise.  Both the CPU oracle and the HIP
path take their inputs from here; neither imports the other.
"""
from .configs import WORKLOADS, Workload, get_workload, PREC_FP32, PREC_BF16, PREC_INT8, PREC_INT4
from .gen import make_inputs, make_random_int_state

__all__ = [
    "WORKLOADS", "Workload", "get_workload", "make_inputs", "make_random_int_state",
    "PREC_FP32", "PREC_BF16", "PREC_INT8", "PREC_INT4",
]
