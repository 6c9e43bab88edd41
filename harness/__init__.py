"""Assembles the synthetic workloads on the GPU through libkv4.

Used by the GPU tests and by bench.py.  It draws inputs from ``workloads``,
allocates device memory with torch and fills the caches by calling the
library's append -- it implements none of the method's arithmetic itself.
"""
from .device import (  # noqa: F401
    GpuWorkload,
    build_from_host,
    build_config,
    build_layers,
    MultiLayerWorkload,
    ORACLE_FMT,
)
