"""Plain CPU oracle for the Memory Sparse Attention (MSA) routed-layer hot path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
reference that the HIP path is checked against.  Only the test suite
(``tests/``), ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``routed_sparse_attention_msa_amd``)
never imports, calls or links anything here, and nothing here imports the
product path: the two share no code.

All arithmetic is NumPy float64.  Stored (rounded) results are produced with
the round-to-nearest-even helper in :mod:`oracle.bf16`.

Every function cites the passage of the source pages it follows; the readings
taken where the pages are silent are listed in each docstring.

Parity status
-------------
Every function here is pinned by ``tests/test_oracle_*.py`` (brute force on
tiny shapes, closed forms, invariants, and independent library routines).
The *semantic readings* (head-mean of per-head cosines, max over chunks,
tie-break to the lower id, bottom-right causal alignment, scale 1/sqrt(d))
cannot be confirmed by any value the pages print; those readings are fixed
here and the GPU must match them.
"""

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, round_bf16, round_f32
from .msa_oracle import (
    pool_chunks_mean,
    pool_chunks_stored,
    chunk_norms,
    rope_rotate_half,
    chunk_offsets,
    encode_docs,
    route_scores,
    topk_docs,
    topk_docs_excluding,
    route_rounds,
    gather_kv,
    sparse_attention,
    sparse_attention_rows,
    merge_attention,
    sparse_attention_backward,
    gated_delta_rule,
    inject_states,
)

__all__ = [
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "round_bf16",
    "round_f32",
    "pool_chunks_mean",
    "pool_chunks_stored",
    "chunk_norms",
    "rope_rotate_half",
    "chunk_offsets",
    "encode_docs",
    "route_scores",
    "topk_docs",
    "topk_docs_excluding",
    "route_rounds",
    "gather_kv",
    "sparse_attention",
    "sparse_attention_rows",
    "merge_attention",
    "sparse_attention_backward",
    "gated_delta_rule",
    "inject_states",
]
