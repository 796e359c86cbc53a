"""Seeded synthetic inputs for EAGLE tree verification.

This package only *draws* inputs: random weights, KV prefixes, node hidden
states, token ids and tree topologies, plus the bf16 storage format they are
kept in.  It contains none of the method's arithmetic (no attention, no
projection, no argmax, no acceptance), so both the fp64 CPU oracle and the HIP
path can consume the same inputs without sharing any of the method's code.
"""
from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32, bf16_bits_to_f64
from .configs import (LayerDims, DraftParams, CONFIGS, Workload, make_workload, mini_dims, StackWorkload,
                      stack_workload)
from . import trees

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_bits_to_f64",
    "LayerDims", "DraftParams", "CONFIGS", "Workload", "make_workload", "mini_dims", "trees",
    "StackWorkload", "stack_workload",
]
