"""Seeded synthetic inputs for the hybrid compressed-attention workloads.

This package is shared by the test oracle and the HIP path. It holds no arithmetic
of the attention method: only random draws, fp32 -> bf16 rounding (torch's
round-to-nearest-even cast) and the fp8 e4m3 encoding of indexer keys, which is an
input-format step done with torch's own cast.
"""
from .workloads import (  # noqa: F401
    CONFIG_ORDER,
    WORKLOADS,
    Lane,
    Workload,
    draw_lengths,
    generate,
    random_scores,
    random_selection,
)
