"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This package holds no quantization, packing or attention arithmetic: only
random draws, bf16 rounding of the draws, context lengths and page tables.
Both the GPU library's callers and the CPU oracle take their inputs from here.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    context_lengths,
    outlier_channels,
    host_sequence,
    host_prompt,
    host_queries,
    PageAllocator,
)
