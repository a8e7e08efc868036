"""Seeded synthetic workloads for the activation-sparse gated FFN.

This package draws inputs only. It is shared by the test suite (which feeds
the same arrays to the CPU oracle and to the HIP library) and by the
benchmark. Nothing in here evaluates the FFN's output; see
:mod:`synth.workloads` for the recipes.
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    make_workload,
    round_bf16,
    round_f32,
    bf16_bits,
    draw_dy,
)
