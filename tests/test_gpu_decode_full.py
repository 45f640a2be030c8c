"""The decode step at full size, in the launch configuration the decode bench
times: the 1M-token bank (2048 documents x 512 tokens, pooled on the GPU),
32 sequences x 1 new token, 32 query / 8 KV heads, head dim 128, 4096 cached
local tokens; routing over all 16,384 pooled chunks, top-k, gather, split-KV
attention.  Every output is compared with the oracle: all 32 x 2048 routing
scores, the top-k by the band rule, the gather bit for bit, and all 1,024
(sequence, head) attention rows.  k = 16 gives 128 memory rows; k = 32 gives
the 256 rows the workload's text also names."""

import math

import numpy as np
import pytest
import torch

import msa_inputs as mi
import routed_sparse_attention_msa_amd as msa
from oracle import gather_kv, route_scores, sparse_attention
from tests.parity import ATTN_RTOL_BF16, ROUTE_ATOL, case, row_rel_l2, to_f64, topk_band_check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def decode_inputs():
    """The bank drawn and pooled as the decode bench does (the prefill draw of
    seed 0), and the decode-side tensors from seed 1."""
    case("decode full: drawing the 1M-token bank and the 32-sequence decode inputs")
    cfg = mi.DECODE
    t = mi.draw_layer(mi.PREFILL, seed=0, device=DEV)
    kbar, _ = msa.msa_pool_chunks(t["k"], cfg.chunk)
    vbar, _ = msa.msa_pool_chunks(t["v"], cfg.chunk)
    kbar_r, knorm = msa.msa_pool_chunks(t["k_r"], cfg.chunk, with_norm=True)
    del t
    d = mi.draw_layer(cfg, seed=1, device=DEV, with_raw=False)
    torch.cuda.synchronize()
    return dict(kbar=kbar, vbar=vbar, kbar_r=kbar_r, knorm=knorm, q=d["q"], k_loc=d["k_loc"],
                v_loc=d["v_loc"], q_r=d["q_r"])


@pytest.mark.parametrize("topk", [16, 32])
def test_decode_step_full_size(decode_inputs, topk):
    cfg = mi.DECODE
    x = decode_inputs
    cpd = cfg.chunks_per_doc
    case(f"decode full: 32 sequences x (M={topk * cpd} + 4096) keys, top-{topk}")
    scores = msa.msa_route_scores(x["q_r"], x["kbar_r"], x["knorm"], cpd)
    ids, _ = msa.msa_topk_docs(scores, topk)
    k_sel, v_sel = msa.msa_gather_kv(x["kbar"], x["vbar"], ids, cpd)
    out, lse = msa.msa_sparse_attn(x["q"], k_sel, v_sel, x["k_loc"], x["v_loc"])
    torch.cuda.synchronize()
    # S2: every score
    ref_scores = route_scores(to_f64(x["q_r"]), to_f64(x["kbar_r"]), cpd)
    err = np.abs(to_f64(scores) - ref_scores).max()
    assert err <= ROUTE_ATOL and err <= 2e-5, err
    # S3: band rule against the oracle's scores
    ok, exact = topk_band_check(ids.cpu().numpy(), ref_scores, topk)
    print(f"  route err {err:.2e}; top-{topk} band rule {ok}, exact {exact}")
    assert ok
    # S4: bit for bit on the GPU's ids
    id64 = ids.cpu().numpy().astype(np.int64)
    raw = lambda t: t.cpu().view(torch.int16).numpy()
    rk, rv = gather_kv(raw(x["kbar"]), raw(x["vbar"]), id64, cpd)
    assert np.array_equal(raw(k_sel), rk) and np.array_equal(raw(v_sel), rv)
    # S6: all 1,024 (sequence, head) rows against the oracle on the gathered memory
    ro, rlse = sparse_attention(to_f64(x["q"]), to_f64(k_sel), to_f64(v_sel), to_f64(x["k_loc"]),
                                to_f64(x["v_loc"]), scale=1.0 / math.sqrt(cfg.dim))
    rel = row_rel_l2(to_f64(out), ro)
    lerr = np.abs(to_f64(lse) - rlse)
    print(f"  attention: max row rel-L2 {rel.max():.2e} over {rel.size} rows, max |lse err| {lerr.max():.2e}")
    assert rel.shape == (32, 1, 32) and rel.max() <= ATTN_RTOL_BF16
    assert lerr.max() <= 2e-3


def test_decode_step_full_size_overlapped(decode_inputs):
    """The overlapped form the decode bench times: attention over the 4096
    local rows on a second stream beside route -> top-k -> gather, then the
    128 memory rows' attention (passed as the local rows of a call without
    memory: the one token sees them all) and the log-sum-exp merge.  All 1,024
    (sequence, head) rows against the oracle's attention over [memory ; local]."""
    cfg = mi.DECODE
    x = decode_inputs
    cpd, topk = cfg.chunks_per_doc, cfg.topk
    case("decode full, overlapped: local attention on a second stream, memory attention + merge after the gather")
    cur, side = torch.cuda.current_stream(), torch.cuda.Stream()
    o_loc = torch.empty_like(x["q"])
    l_loc = torch.empty((cfg.batch, cfg.heads_q, 1), dtype=torch.float32, device=DEV)
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        msa.msa_sparse_attn(x["q"], None, None, x["k_loc"], x["v_loc"], out=o_loc, lse=l_loc)
    scores = msa.msa_route_scores(x["q_r"], x["kbar_r"], x["knorm"], cpd)
    ids, _ = msa.msa_topk_docs(scores, topk)
    k_sel, v_sel = msa.msa_gather_kv(x["kbar"], x["vbar"], ids, cpd)
    o_mem, l_mem = msa.msa_sparse_attn(x["q"], None, None, k_sel, v_sel)
    cur.wait_stream(side)
    out, lse = msa.msa_attn_merge(o_loc, l_loc, o_mem, l_mem)
    torch.cuda.synchronize()
    ro, rlse = sparse_attention(to_f64(x["q"]), to_f64(k_sel), to_f64(v_sel), to_f64(x["k_loc"]),
                                to_f64(x["v_loc"]), scale=1.0 / math.sqrt(cfg.dim))
    rel = row_rel_l2(to_f64(out), ro)
    lerr = np.abs(to_f64(lse) - rlse)
    print(f"  overlapped attention: max row rel-L2 {rel.max():.2e} over {rel.size} rows, max |lse err| {lerr.max():.2e}")
    assert rel.shape == (32, 1, 32) and rel.max() <= ATTN_RTOL_BF16
    assert lerr.max() <= 2e-3
