"""CPU oracle for hybrid compressed attention -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it. It shares no code with the HIP library (``compressed_sparse_long_amd``)
and never imports it; the two meet only through the seeded inputs of ``synth``.

Every function is plain fp64 numpy with explicit loops over batch, query row and head.
"""
from .csa import (  # noqa: F401
    attend,
    compress,
    compress_entry,
    decode_e4m3,
    hca_attn,
    indexer,
    n_visible,
    sparse_attn,
    to_bf16_f64,
    topk,
    window_rows,
)
from . import pipeline  # noqa: F401
