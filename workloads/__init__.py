"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package only draws random numbers and stores them in the byte formats the
indexer consumes (bf16, OCP FP8 E4M3 with one fp32 scale per token, fp32).  It
holds none of the indexer's arithmetic: no dot products, no ReLU, no head
reduction and no selection.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    e4m3_quantize_rows,
    make_decode,
    make_group_bank,
    make_mtp,
    make_prefill,
    make_workload,
    to_bf16,
)
