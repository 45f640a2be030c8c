"""msa_route_scores_noalloc (the routing entry point that allocates nothing:
its scratch is a library-resident device array) against msa_route_scores,
called through the C ABI: two calls in a row, the second with a smaller input,
each equal bit for bit to the entry point with a caller workspace."""

import ctypes

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from routed_sparse_attention_msa_amd import _lib as L
from tests.parity import case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(batch, q_len, n_docs, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q_r = torch.randn((batch, q_len, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    kbar = torch.randn((n_docs * 8, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    norm = torch.linalg.vector_norm(kbar.float(), dim=-1).contiguous()
    return q_r, kbar, norm


def _noalloc(q_r, kbar, norm, n_docs):
    batch, q_len = q_r.shape[:2]
    out = torch.full((batch, n_docs), float("nan"), device=DEV)
    st = msa.lib().msa_route_scores_noalloc(
        ctypes.c_void_p(q_r.data_ptr()), ctypes.c_void_p(kbar.data_ptr()), ctypes.c_void_p(norm.data_ptr()),
        batch, q_len, 8, 128, n_docs, 8, L.MSA_BF16, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out


def _with_ws(q_r, kbar, norm, n_docs):
    batch, q_len = q_r.shape[:2]
    nbytes = msa.msa_route_scores_workspace(batch, q_len, 8, 128, n_docs, 8, torch.bfloat16)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((batch, n_docs), device=DEV)
    st = msa.lib().msa_route_scores(
        ctypes.c_void_p(q_r.data_ptr()), ctypes.c_void_p(kbar.data_ptr()), ctypes.c_void_p(norm.data_ptr()),
        batch, q_len, 8, 128, n_docs, 8, L.MSA_BF16, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(ws.data_ptr()), nbytes, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out, nbytes


@pytest.mark.parametrize("shapes", [
    # (batch, q_len, n_docs): tiled over several row tiles per sequence, then a smaller tiled call
    [(2, 512, 3000), (1, 320, 1000)],
    # the 1M-token prefill shape, then a decode-sized scan (no scratch at all)
    [(1, 2048, 2048), (32, 1, 2048)],
])
def test_noalloc_equals_route_scores(shapes):
    for batch, q_len, n_docs in shapes:
        case(f"route noalloc B={batch} T={q_len} N={n_docs}")
        q_r, kbar, norm = _inputs(batch, q_len, n_docs, batch * 1000 + q_len + n_docs)
        st0, ref, nbytes = _with_ws(q_r, kbar, norm, n_docs)
        st1, got = _noalloc(q_r, kbar, norm, n_docs)
        torch.cuda.synchronize()
        assert st0 == L.MSA_OK and st1 == L.MSA_OK, msa.lib().msa_last_error()
        print(f"  scratch {nbytes} bytes; max |diff| {float((got - ref).abs().max()):.3e}")
        assert torch.equal(got, ref)


def test_noalloc_rejects_scratch_above_its_limit():
    case("route noalloc above the limit")
    n_docs = 2048
    batch, q_len = 1, (1 << 20) + 32              # 32 B of inverse norms per token: just over 32 MiB
    need = msa.msa_route_scores_workspace(batch, q_len, 8, 128, n_docs, 8, torch.bfloat16)
    assert need > 32 << 20
    p = ctypes.c_void_p(256)
    st = msa.lib().msa_route_scores_noalloc(p, p, p, batch, q_len, 8, 128, n_docs, 8, L.MSA_BF16, p, None)
    assert st == L.MSA_ERR_INVALID
    assert b"scratch" in msa.lib().msa_last_error()
