"""The C-ABI library loads, exports every entry point include/msa.h declares,
and rejects invalid arguments on the host (no GPU work is enqueued by any of
these calls)."""

import ctypes
import os
import re
import subprocess

import pytest

import routed_sparse_attention_msa_amd as msa
from routed_sparse_attention_msa_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(L.SIGNATURES)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (msa_\w+)", out))
    missing = [s for s in _declared() if s not in exported]
    assert not missing, missing


def test_loads_and_reports_version():
    lib = msa.lib()
    assert lib.msa_abi_version() == 1
    for name in _declared():
        assert hasattr(lib, name)


def _err():
    return msa.lib().msa_last_error().decode()


def test_pool_validation():
    lib = msa.lib()
    p = ctypes.c_void_p(16)
    # doc_len not a multiple of chunk
    assert lib.msa_pool_chunks(p, p, None, 4, 100, 64, 8, 128, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    assert "multiple of chunk" in _err()
    # unknown dtype
    assert lib.msa_pool_chunks(p, p, None, 4, 512, 64, 8, 128, 7, None) == L.MSA_ERR_INVALID
    # misaligned pointer
    q = ctypes.c_void_p(18)
    assert lib.msa_pool_chunks(q, p, None, 4, 512, 64, 8, 128, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    assert "aligned" in _err()
    # norms need a power-of-two head size in bytes
    assert lib.msa_pool_chunks(p, p, p, 4, 512, 64, 1, 24, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    # zero documents is a no-op
    assert lib.msa_pool_chunks(None, None, None, 0, 512, 64, 8, 128, L.MSA_BF16, None) == L.MSA_OK


def test_encode_validation():
    lib = msa.lib()
    p = ctypes.c_void_p(16)
    # chunk must be positive
    assert lib.msa_chunk_offsets(p, 4, 0, p, None) == L.MSA_ERR_INVALID
    assert lib.msa_encode_docs(p, p, None, p, p, 4, 100, 10, 0, 8, 128, 0.0, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    # RoPE needs a power-of-two head of at least 32 bytes
    assert lib.msa_encode_docs(p, p, None, p, p, 4, 100, 10, 8, 2, 8, 1e4, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    assert "power of two" in _err()
    assert lib.msa_encode_docs(p, p, None, p, p, 4, 100, 10, 8, 1, 24, 1e4, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    # negative rope base, unknown dtype, misaligned rows
    assert lib.msa_encode_docs(p, p, None, p, p, 4, 100, 10, 8, 8, 128, -1.0, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    assert lib.msa_encode_docs(p, p, None, p, p, 4, 100, 10, 8, 8, 128, 0.0, 9, None) == L.MSA_ERR_INVALID
    q = ctypes.c_void_p(18)
    assert lib.msa_encode_docs(q, p, None, p, p, 4, 100, 10, 8, 8, 128, 0.0, L.MSA_BF16, None) == L.MSA_ERR_INVALID
    # no chunks is a no-op
    assert lib.msa_encode_docs(None, None, None, None, None, 0, 0, 0, 8, 8, 128, 0.0, L.MSA_BF16, None) == L.MSA_OK


def test_topk_validation_and_workspace():
    lib = msa.lib()
    n = ctypes.c_size_t(123)
    assert lib.msa_topk_docs_workspace(1, 100, 0, ctypes.byref(n)) == L.MSA_ERR_INVALID
    assert lib.msa_topk_docs_workspace(1, 100, 101, ctypes.byref(n)) == L.MSA_ERR_INVALID
    assert lib.msa_topk_docs_workspace(1, 5000, 1025, ctypes.byref(n)) == L.MSA_ERR_INVALID
    assert lib.msa_topk_docs_workspace(1, 4096, 16, ctypes.byref(n)) == L.MSA_OK and n.value == 0
    assert lib.msa_topk_docs_workspace(4, 195313, 16, ctypes.byref(n)) == L.MSA_OK
    assert n.value == 2 * 4 * 48 * 16 * 8
    p = ctypes.c_void_p(256)
    assert lib.msa_topk_docs(p, 4, 195313, 16, p, None, None, 0, None) == L.MSA_ERR_INVALID
    assert "workspace" in _err()


def test_rounds_validation():
    lib = msa.lib()
    p = ctypes.c_void_p(256)
    n = ctypes.c_size_t(0)
    # k + n_excl must leave k documents; strides must hold the rows
    assert lib.msa_topk_docs_excluding(p, 2, 100, 10, p, 91, 91, p, None, 10, None, 0, None) == L.MSA_ERR_INVALID
    assert "k + n_excl" in _err()
    assert lib.msa_topk_docs_excluding(p, 2, 100, 10, p, 5, 4, p, None, 10, None, 0, None) == L.MSA_ERR_INVALID
    assert lib.msa_topk_docs_excluding(p, 2, 100, 10, None, 5, 5, p, None, 10, None, 0, None) == L.MSA_ERR_INVALID
    assert lib.msa_topk_docs_excluding(p, 2, 100, 10, None, 0, 0, p, None, 9, None, 0, None) == L.MSA_ERR_INVALID
    # exclusion entries inside the outputs: only the multi-round layout is accepted
    ids = 4096
    ok = (ctypes.c_void_p(ids), ctypes.c_void_p(ids + 4 * 8))          # excl = ids, out = ids + 8 (n_excl 8)
    bad = (ctypes.c_void_p(ids), ctypes.c_void_p(ids + 4 * 4))         # out starts inside the exclusion
    assert lib.msa_topk_docs_excluding(p, 2, 100, 4, ok[0], 8, 12, bad[1], None, 12, None, 0, None) == L.MSA_ERR_INVALID
    assert "overlap" in _err()
    assert lib.msa_topk_docs_excluding(p, 2, 100, 4, ok[0], 8, 12, ok[1], None, 16, None, 0, None) == L.MSA_ERR_INVALID
    # rounds * k may not exceed the documents
    assert lib.msa_route_rounds_workspace(3, 1, 8, 8, 128, 40, 8, 16, L.MSA_BF16, ctypes.byref(n)) == L.MSA_ERR_INVALID
    assert lib.msa_route_rounds_workspace(0, 1, 8, 8, 128, 40, 8, 4, L.MSA_BF16, ctypes.byref(n)) == L.MSA_ERR_INVALID
    assert lib.msa_route_rounds_workspace(3, 2, 8, 8, 128, 48, 8, 16, L.MSA_BF16, ctypes.byref(n)) == L.MSA_OK
    assert n.value >= 2 * 48 * 4
    assert lib.msa_route_rounds(p, p, p, 3, 2, 8, 8, 128, 48, 8, 16, L.MSA_BF16, p, None, None, 0,
                                None) == L.MSA_ERR_INVALID
    assert "workspace" in _err()


def test_route_validation():
    lib = msa.lib()
    p = ctypes.c_void_p(256)
    assert lib.msa_route_scores(p, p, None, 1, 8, 8, 128, 16, 8, L.MSA_BF16, p, None, 0, None) == L.MSA_ERR_INVALID
    assert lib.msa_route_scores(p, p, p, 1, 8, 8, 12, 16, 8, L.MSA_BF16, p, None, 0, None) == L.MSA_ERR_INVALID
    n = ctypes.c_size_t(0)
    assert lib.msa_route_scores_workspace(1, 2048, 8, 128, 2048, 8, L.MSA_BF16, ctypes.byref(n)) == L.MSA_OK


def test_attn_validation():
    lib = msa.lib()
    p = ctypes.c_void_p(256)
    # heads_q not a multiple of heads_kv
    assert lib.msa_sparse_attn(p, p, p, 8, p, p, 16, 1, 16, 6, 4, 128, 0.1, L.MSA_BF16, p, None, None, 0,
                               None) == L.MSA_ERR_INVALID
    # local KV shorter than the query
    assert lib.msa_sparse_attn(p, p, p, 8, p, p, 8, 1, 16, 8, 4, 128, 0.1, L.MSA_BF16, p, None, None, 0,
                               None) == L.MSA_ERR_INVALID
    # non-positive scale
    assert lib.msa_sparse_attn(p, p, p, 8, p, p, 16, 1, 16, 8, 4, 128, 0.0, L.MSA_BF16, p, None, None, 0,
                               None) == L.MSA_ERR_INVALID
    # memory rows without tensors
    assert lib.msa_sparse_attn(p, None, None, 8, p, p, 16, 1, 16, 8, 4, 128, 0.1, L.MSA_BF16, p, None, None,
                               0, None) == L.MSA_ERR_INVALID


def test_attn_merge_validation():
    lib = msa.lib()
    p, f = ctypes.c_void_p(256), ctypes.c_void_p(260)
    ok = (p, f, p, f, 2, 1, 32, 128, L.MSA_BF16, p, f, None)
    def call(*args):
        return lib.msa_attn_merge(*args)
    bad = list(ok); bad[8] = 7                        # unknown dtype
    assert call(*bad) == L.MSA_ERR_INVALID
    bad = list(ok); bad[7] = 512                      # dim above 256
    assert call(*bad) == L.MSA_ERR_INVALID
    bad = list(ok); bad[7] = 100                      # 200 bytes per row: not whole 16-byte pieces
    assert call(*bad) == L.MSA_ERR_INVALID
    bad = list(ok); bad[4] = 0                        # empty batch
    assert call(*bad) == L.MSA_ERR_INVALID
    bad = list(ok); bad[2] = None                     # missing input
    assert call(*bad) == L.MSA_ERR_INVALID
    bad = list(ok); bad[9] = ctypes.c_void_p(264)     # output not 16-byte aligned
    assert call(*bad) == L.MSA_ERR_INVALID
    bad = list(ok); bad[1] = ctypes.c_void_p(258)     # lse not 4-byte aligned
    assert call(*bad) == L.MSA_ERR_INVALID
    assert "aligned" in _err()


def test_attn_rejects_spans_of_4gib():
    """One sequence's memory or local rows must span less than 4 GiB (the
    kernels' buffer offsets are 32-bit)."""
    lib = msa.lib()
    p = ctypes.c_void_p(256)
    n = ctypes.c_size_t(0)
    big = 1 << 21                       # 2^21 rows x 8 heads x 128 x 2 B = 4 GiB
    assert lib.msa_sparse_attn_workspace(1, 16, 32, 8, 128, big, 16, L.MSA_BF16, ctypes.byref(n)) == L.MSA_ERR_INVALID
    assert "4 GiB" in _err()
    assert lib.msa_sparse_attn(p, p, p, 0, p, p, big, 1, 16, 32, 8, 128, 0.1, L.MSA_BF16, p, None, None, 0,
                               None) == L.MSA_ERR_INVALID
    assert lib.msa_sparse_attn_backward_workspace(1, 16, 32, 8, 128, 16, big, L.MSA_BF16,
                                                  ctypes.byref(n)) == L.MSA_ERR_INVALID
    assert lib.msa_sparse_attn_workspace(1, 16, 32, 8, 128, big - 1, 16, L.MSA_BF16, ctypes.byref(n)) == L.MSA_OK


def _ws(op, dims):
    arr = (ctypes.c_int64 * max(1, len(dims)))(*dims)
    n = ctypes.c_size_t(12345)
    st = msa.lib().msa_workspace_size(op, arr, len(dims), ctypes.byref(n))
    return st, n.value


def test_workspace_size_by_operation_matches_the_per_operation_calls():
    lib = msa.lib()
    n = ctypes.c_size_t(0)
    bf = L.MSA_BF16
    cases = [
        (L.MSA_OP_ROUTE_SCORES, [1, 2048, 8, 128, 2048, 8, bf], lambda: lib.msa_route_scores_workspace(
            1, 2048, 8, 128, 2048, 8, bf, ctypes.byref(n))),
        (L.MSA_OP_ROUTE_SCORES, [4, 512, 8, 128, 195313, 8, bf], lambda: lib.msa_route_scores_workspace(
            4, 512, 8, 128, 195313, 8, bf, ctypes.byref(n))),
        (L.MSA_OP_TOPK_DOCS, [4, 195313, 16], lambda: lib.msa_topk_docs_workspace(4, 195313, 16, ctypes.byref(n))),
        (L.MSA_OP_TOPK_DOCS_EXCLUDING, [2, 9000, 32], lambda: lib.msa_topk_docs_workspace(2, 9000, 32,
                                                                                         ctypes.byref(n))),
        (L.MSA_OP_ROUTE_ROUNDS, [3, 1, 2048, 8, 128, 2048, 8, 16, bf], lambda: lib.msa_route_rounds_workspace(
            3, 1, 2048, 8, 128, 2048, 8, 16, bf, ctypes.byref(n))),
        (L.MSA_OP_SPARSE_ATTN, [32, 1, 32, 8, 128, 128, 4096, bf], lambda: lib.msa_sparse_attn_workspace(
            32, 1, 32, 8, 128, 128, 4096, bf, ctypes.byref(n))),
        (L.MSA_OP_SPARSE_ATTN, [1, 2048, 32, 8, 128, 128, 2048, bf], lambda: lib.msa_sparse_attn_workspace(
            1, 2048, 32, 8, 128, 128, 2048, bf, ctypes.byref(n))),
        (L.MSA_OP_SPARSE_ATTN_BACKWARD, [1, 2048, 32, 8, 128, 128, 2048, bf],
         lambda: lib.msa_sparse_attn_backward_workspace(1, 2048, 32, 8, 128, 128, 2048, bf, ctypes.byref(n))),
    ]
    for op, dims, per_op in cases:
        assert per_op() == L.MSA_OK
        st, got = _ws(op, dims)
        assert st == L.MSA_OK and got == n.value, (op, dims, got, n.value)
    # the tiled routing and the backward need scratch at these sizes
    assert _ws(L.MSA_OP_ROUTE_SCORES, [1, 2048, 8, 128, 2048, 8, bf])[1] > 0
    assert _ws(L.MSA_OP_SPARSE_ATTN_BACKWARD, [1, 2048, 32, 8, 128, 128, 2048, bf])[1] > 0
    # operations without scratch
    for op in (L.MSA_OP_POOL_CHUNKS, L.MSA_OP_GATHER_KV, L.MSA_OP_ENCODE_DOCS, L.MSA_OP_GDN_STATE_SUM,
               L.MSA_OP_GATED_DELTA_RULE):
        assert _ws(op, []) == (L.MSA_OK, 0)
    # a wrong count of dims, an unknown op, an argument the operation rejects, an int32 overflow
    assert _ws(L.MSA_OP_TOPK_DOCS, [4, 100])[0] == L.MSA_ERR_INVALID
    assert "3 dims" in _err()
    assert _ws(99, [1])[0] == L.MSA_ERR_INVALID
    assert "unknown operation" in _err()
    assert _ws(L.MSA_OP_TOPK_DOCS, [1, 100, 101])[0] == L.MSA_ERR_INVALID
    assert _ws(L.MSA_OP_SPARSE_ATTN, [1 << 31, 1, 32, 8, 128, 0, 1, bf])[0] == L.MSA_ERR_INVALID
    assert "int32" in _err()
    # n_docs is a 64-bit argument and may exceed the int32 range on the way in (then rejected by the op)
    assert _ws(L.MSA_OP_TOPK_DOCS, [1, 1 << 31, 16])[0] == L.MSA_ERR_INVALID
    assert "2^31" in _err()
    assert msa.msa_workspace_size(L.MSA_OP_TOPK_DOCS, [4, 195313, 16]) == 2 * 4 * 48 * 16 * 8


def test_gather_validation():
    lib = msa.lib()
    p = ctypes.c_void_p(256)
    assert lib.msa_gather_kv(p, p, 0, p, 1, 4, 16, 8, 8, 128, L.MSA_BF16, p, p, 0x10, None) == L.MSA_ERR_INVALID
    assert lib.msa_gather_kv(p, p, 0, p, 1, 4, 16, 8, 1, 4, L.MSA_BF16, p, p, 0, None) == L.MSA_ERR_INVALID


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((2, 64, 1, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        msa.msa_pool_chunks(x, 64)


def test_gated_delta_rule_chunked_validation():
    """The chunked form takes bf16 with dk = dv = 128 and rejects the rest on the host."""
    lib = L.lib()
    p = ctypes.c_void_p(4096)
    args = lambda dt, dk, dv, q=p: (q, p, p, p, p, 0.1, None, 2, 64, 8, dk, dv, dt, p, p, None)
    assert lib.msa_gated_delta_rule_chunked(*args(L.MSA_F32, 128, 128)) == L.MSA_ERR_INVALID
    assert lib.msa_gated_delta_rule_chunked(*args(L.MSA_BF16, 64, 128)) == L.MSA_ERR_INVALID
    assert lib.msa_gated_delta_rule_chunked(*args(L.MSA_BF16, 128, 64)) == L.MSA_ERR_INVALID
    assert lib.msa_gated_delta_rule_chunked(*args(L.MSA_BF16, 128, 128, q=None)) == L.MSA_ERR_INVALID
    assert lib.msa_gated_delta_rule_chunked(*args(L.MSA_BF16, 128, 128, q=ctypes.c_void_p(4098))) == L.MSA_ERR_INVALID
    # a sequence spanning 4 GiB of rows (2^21 tokens x 8 heads x 256 B) would wrap the 32-bit buffer offsets
    big = (p, p, p, p, p, 0.1, None, 1, 1 << 21, 8, 128, 128, L.MSA_BF16, p, p, None)
    assert lib.msa_gated_delta_rule_chunked(*big) == L.MSA_ERR_INVALID
    assert "4 GiB" in lib.msa_last_error().decode()
    n = ctypes.c_size_t(7)
    dims = (ctypes.c_int64 * 1)(0)
    assert lib.msa_workspace_size(L.MSA_OP_GATED_DELTA_RULE_CHUNKED, dims, 0, ctypes.byref(n)) == L.MSA_OK
    assert n.value == 0
