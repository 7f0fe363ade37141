"""CPU oracle for absorbed Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg, never by the library.  It is a plain,
slow fp64 NumPy implementation of the direct form (explicit K = U_K c and
V = U_V c per head, RoPE at true positions, ordinary softmax) and shares no
code with the HIP path.  Every function is pinned by ``tests/test_oracle.py``
against the pages' worked examples, closed forms, library routines and brute
force; none is "parity unpinned".
"""
from .mla_direct import (  # noqa: F401
    NEG_INF,
    OracleSegment,
    absorb_query,
    attend_direct,
    cache_bytes,
    direct_mla_decode,
    expand,
    merge_lse,
    mha_cache_bytes,
    output_expand,
    rope_frequencies,
    rope_relocate,
    rope_rotate,
    softmax_lse,
)
