"""Seeded synthetic inputs for causal attention, shared by the tests and the benchmark.

This module holds no attention arithmetic: it draws tensors, rounds them to the
input dtype and lays out packed-document boundaries.  Both the fp64 oracle and
the HIP path receive the arrays it returns.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    DECODE_CONFIGS,
    AttnConfig,
    DecodeConfig,
    round_to,
    round_to_bf16,
    round_to_f16,
    make_cu_seqlens,
    make_inputs,
    make_inputs_device,
    make_decode_inputs,
    allowed_pair_count,
)
