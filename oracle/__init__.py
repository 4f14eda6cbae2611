"""CPU oracle for HGA routed attention — test infrastructure, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library under
``hierarchical_sparse_attention_build_amd/``; the product path never calls it.
"""
from .hga_oracle import (  # noqa: F401
    HGAConfig, rope_thetas, high_freq_pairs, rotate_pairs, apply_rope,
    span_summary_literal, span_summary_relative, build_summaries,
    select_top, boundary_gap, chunk_candidates, route_unit, route,
    forced_chunks, visible_tokens, softmax_attend, attend, attend_unit_block,
    prefill, decode, dense_causal, warm_lru_step, attend_backward,
)
