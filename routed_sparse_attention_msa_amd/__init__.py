"""MI355X (gfx950) hot path of Memory Sparse Attention (MSA), one routed layer.

The work runs in hand-written HIP kernels in ``libmsa.so`` behind the C ABI
of ``include/msa.h``; this package is its thin Python binding:

    msa_pool_chunks          S1  chunk-mean pooling of K / V / K_r into the bank
    msa_chunk_offsets        offline encoder over variable-length documents:
    msa_encode_docs            document-wise RoPE + chunk means (+ norms)
    msa_route_scores         S2  cosine routing scores per document
    msa_topk_docs            S3  top-k documents
    msa_topk_docs_excluding  top-k among the documents not yet selected
    msa_route_rounds         multi-round routing (Memory Interleave)
    msa_gather_kv            S4  gather (or host-tier fetch) of the selected pooled K/V
    msa_sparse_attn          S5/S6 sparse GQA attention (prefill and decode)
    msa_attn_merge           log-sum-exp merge of two partial attentions (disjoint key sets)
    msa_sparse_attn_backward its gradients (training through the routed layer)
    msa_gdn_state_sum        linear-layer variant: sum of the selected documents' states
    msa_gated_delta_rule       and the gated delta rule from that initial state (token by token)
    msa_gated_delta_rule_chunked  the same rule in its chunked form (MFMA, 32 tokens per chunk)
    msa_workspace_size       scratch bytes of any of these calls, by operation code
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MsaError,
    lib,
    msa_attn_merge,
    msa_chunk_offsets,
    msa_encode_docs,
    msa_gated_delta_rule,
    msa_gated_delta_rule_chunked,
    msa_gather_kv,
    msa_gdn_state_sum,
    msa_pool_chunks,
    msa_route_rounds,
    msa_route_rounds_workspace,
    msa_route_scores,
    msa_route_scores_workspace,
    msa_sparse_attn,
    msa_sparse_attn_backward,
    msa_sparse_attn_backward_workspace,
    msa_sparse_attn_workspace,
    msa_topk_docs,
    msa_topk_docs_excluding,
    msa_topk_docs_workspace,
    msa_workspace_size,
    SIGNATURES,
)
