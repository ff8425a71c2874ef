"""Seeded synthetic workloads for the paged KV-cache hot path.

See :mod:`workloads.cases`.  This package builds inputs only; it holds none of
the hot path's arithmetic and imports neither the oracle nor the HIP binding.
"""
from .cases import (  # noqa: F401
    Geometry,
    Region,
    Case,
    tiny_decode,
    qwen3_decode,
    gqa_prefix_share,
    mla_decode,
    encdec_extend,
    mixed_spans,
    shared_prefix_batch,
    make_values,
    to_numpy_bits,
    CONFIG_BUILDERS,
)
