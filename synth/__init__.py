"""Seeded synthetic inputs for the draft-block verification path.

This package only draws inputs (weights, hidden states, draft tokens,
draft logits, confidences, uniforms) and rounds them to the storage types
the path consumes. It holds none of the verification arithmetic, so both
the CPU oracle and the HIP path can be fed from it.
"""
from .inputs import (WORKLOADS, Workload, StepInputs, bf16_round, bf16_to_f32,
                     make_weights, make_step, workload)

__all__ = ["WORKLOADS", "Workload", "StepInputs", "bf16_round", "bf16_to_f32",
           "make_weights", "make_step", "workload"]
