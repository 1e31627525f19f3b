"""fp64 CPU oracle for hybrid prefill/decode paged attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg; never by the library.  Every function is pinned by the ``-m "not gpu"``
tests in tests/test_oracle_*.py (no function here is "parity unpinned").
"""
from .attention import (  # noqa: F401
    PAGE, HybridProblem, append_tokens, attend, attend_blockwise, attend_online,
    bf16_bits_to_f64, combine_partials, e4m3_to_f64, gather_kv, gather_kv_token, masked_scores,
    row_positions, softmax_rows, split_partials, to_f64,
)
