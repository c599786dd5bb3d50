"""Seeded synthetic inputs for paged decode attention.

This package is the only code shared by the CPU oracle's tests and the HIP
path's tests and bench.  It draws random numbers, builds block tables with a
host block pool, and lays the drawn values into the paged cache.  It holds
none of the attention arithmetic: no dot products, no softmax, no gather.

Shapes follow the decode workloads the pages motivate (a tiny fp32 case, a
Llama-3-8B-shaped bf16 layer, a 70B-shaped 80-layer fp16 step, a 13B MHA
batch that shares a 1200-token system prompt, a 131072-token FP8 case, and
two 131072-token 8-bit variants: K fp8 with V int8, and int8 K and V with
outlier K channels and per-channel K factors).
"""

from .specs import DecodeWorkload, WORKLOADS, workload, scaled
from .pool import BlockPool, PoolExhausted
from .build import (
    DecodeLayout,
    build_layout,
    share_prefixes,
    make_host_inputs,
    make_device_inputs,
    fp8_quantize_blocks,
    quantize_blocks,
    outlier_factors,
    POISON_FP8_CODE,
    POISON_INT8_CODE,
)

__all__ = [
    "DecodeWorkload",
    "WORKLOADS",
    "workload",
    "scaled",
    "BlockPool",
    "PoolExhausted",
    "DecodeLayout",
    "build_layout",
    "share_prefixes",
    "make_host_inputs",
    "make_device_inputs",
    "fp8_quantize_blocks",
    "quantize_blocks",
    "outlier_factors",
    "POISON_FP8_CODE",
    "POISON_INT8_CODE",
]
