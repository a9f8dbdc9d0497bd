"""Seeded synthetic inputs for the paged decode path.

This package serves both the oracle side and the HIP side of every test and
of the benchmark.  It only draws random numbers and lays them out: context
lengths, where each sequence's blocks sit in the pool (popped from a seeded,
shuffled free list), Q, the resident K/V contents and the new tokens' K/V.
It computes no slot, no translation and no attention; those live in the
oracle and in the kernels, independently.
"""

from .configs import (  # noqa: F401
    CONFIG_NAMES,
    PREFILL_NAMES,
    PrefillWorkload,
    TokenModel,
    config_lengths,
    make_block_size_sweep,
    make_prefill,
    make_prefill_custom,
    make_token_model,
    Step,
    Workload,
    make_config,
    make_custom,
    make_tp_share,
    to_bf16_bits,
)
