"""Seeded synthetic inputs for the MoE expert layer.

This module is shared by the oracle's tests and by the GPU path's tests and
benchmark. It holds no arithmetic of the layer itself: it only draws the
tensors the layer consumes (activations, weights, upstream gradient and, for
the random-routing workloads, the expert choices and gates), rounds them to
the storage precision, and describes the workload shapes.

Value recipe (same for every workload): activations and the upstream gradient
are N(0, 1); every weight is N(0, 0.02). bf16 workloads round the fp32 draws
to bf16 with round-to-nearest-even, and both sides consume those exact values.

Streams: numpy ``SeedSequence(seed, spawn_key=(i,))`` for
i = 0..7 in the order x, W_router, W_gate, W_up, W_down, dY, route-choice,
route-gate. Expert weights use one child stream per expert,
``spawn_key=(i, e)``, so a single expert can be regenerated on its own.
"""
from .generators import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_round,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    expert_weight,
    zipf_routing,
    balanced_routing,
)
