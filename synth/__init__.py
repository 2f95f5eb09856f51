"""Seeded synthetic workloads shared by the oracle, the tests and the bench.

This package draws random numbers and rounds them to bf16 storage; it holds none
of the compression method's arithmetic (no scales, codes, pruning or encoding),
so that the oracle and the HIP path can both consume its output without sharing
any of the computation they are compared on.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    f32_to_bf16_bits,
    gen_weight_rows,
    gen_weights,
    gen_x,
    gen_x_outlier_channels,
    gen_act_norms,
    gen_routes,
    gen_down_inputs,
    gen_expert,
    stream,
    gen_zero_blocks,
    zero_out_blocks,
    ZERO_BLOCK_FRAC,
)
