"""GPU parity of S1 (pool) and S2 (route) against the oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import msa_inputs as mi
import routed_sparse_attention_msa_amd as msa
from oracle import chunk_norms, pool_chunks_mean, route_scores
from oracle.bf16 import round_f32
from tests.parity import ROUTE_ATOL, bf16_ulp_distance, case, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _norms_supported(x):
    head_bytes = x.shape[-1] * x.element_size()
    return 16 <= head_bytes <= 1024 and head_bytes & (head_bytes - 1) == 0


def _check_pool(x, chunk):
    """GPU pooling of x (on the GPU) vs the oracle, element by element."""
    xbar, norm = msa.msa_pool_chunks(x, chunk, with_norm=_norms_supported(x))
    torch.cuda.synchronize()
    xf = to_f64(x)
    exact = pool_chunks_mean(xf, chunk)
    if x.dtype == torch.bfloat16:
        ulps = bf16_ulp_distance(xbar, exact)
        assert ulps.max() <= 1, f"pool differs by {ulps.max()} bf16 ulp"
    else:
        # float32 accumulation of `chunk` terms: |err| <= (chunk-1) u sum|x| / chunk + u |mean|
        u = 2.0 ** -24
        bound = (chunk - 1) * u * pool_chunks_mean(np.abs(xf), chunk) * 1.01 + u * np.abs(exact) + 1e-45
        err = np.abs(to_f64(xbar) - exact)
        assert np.all(err <= bound), f"max err {err.max()}"
    if norm is not None:
        ref = chunk_norms(to_f64(xbar))                       # norm of the stored rows
        np.testing.assert_allclose(to_f64(norm), ref, rtol=2e-6, atol=1e-30)
    return xbar, norm


@pytest.mark.parametrize("shape,chunk,dtype", [
    ((64, 512, 2, 64), 64, torch.float32),       # tiny workload shapes
    ((16, 512, 8, 128), 64, torch.bfloat16),     # production head layout
    ((5, 128, 32, 128), 64, torch.bfloat16),     # 8 KiB rows: two column segments
    ((7, 96, 3, 64), 32, torch.bfloat16),        # 3 heads: row of 24 lanes
    ((4, 64, 2, 64), 64, torch.bfloat16),        # one chunk per document
    ((3, 40, 1, 16), 1, torch.float32),          # chunk of one row (copy)
    ((3, 60, 2, 40), 20, torch.float32),         # head of 160 B: no norms
])
def test_pool_parity(shape, chunk, dtype):
    case(f"pool {shape} chunk={chunk} {dtype}")
    g = torch.Generator(device=DEV)
    g.manual_seed(sum(shape) + chunk)
    x = torch.randn(shape, generator=g, device=DEV).to(dtype)
    _check_pool(x, chunk)


def test_pool_many_chunks_per_workgroup():
    """Enough chunks that a workgroup pools several (rows staged in LDS), with
    a last workgroup that holds fewer than the others."""
    case("pool 1031 chunks, several per workgroup")
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    x = torch.randn((1031, 64, 2, 64), generator=g, device=DEV).to(torch.bfloat16)
    _check_pool(x, 64)


@pytest.mark.parametrize("n_docs", [2048, 2047])
def test_pool_full_bank_sampled(n_docs):
    """The 1M-token bank (512 rows x 8 heads x 128 per document, bf16) in the
    launch configuration of the benchmark; sampled chunks against the oracle."""
    case(f"pool full bank n_docs={n_docs} (sampled)")
    g = torch.Generator(device=DEV)
    g.manual_seed(n_docs)
    x = (torch.randn((n_docs, 512, 8, 128), generator=g, device=DEV) / 11.3).to(torch.bfloat16)
    xbar, norm = msa.msa_pool_chunks(x, 64, with_norm=True)
    torch.cuda.synchronize()
    n_ch = n_docs * 8
    rng = np.random.default_rng(n_docs)
    picks = np.unique(np.concatenate([[0, 31, 32, n_ch - 1], rng.integers(0, n_ch, 60)]))
    rows = x.view(n_ch, 64, 8, 128)[torch.as_tensor(picks, device=DEV)]
    exact = pool_chunks_mean(to_f64(rows), 64)
    got = xbar[torch.as_tensor(picks, device=DEV)]
    assert bf16_ulp_distance(got, exact).max() <= 1
    np.testing.assert_allclose(to_f64(norm[torch.as_tensor(picks, device=DEV)]), chunk_norms(to_f64(got)),
                               rtol=2e-6, atol=1e-30)
    del x


def test_pool_is_deterministic():
    case("pool determinism")
    x = torch.randn((32, 512, 8, 128), device=DEV).to(torch.bfloat16)
    a, na = msa.msa_pool_chunks(x, 64, with_norm=True)
    b, nb = msa.msa_pool_chunks(x, 64, with_norm=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(na, nb)


def _route_case(batch, q_len, heads, dim, n_docs, cpd, dtype, seed, planted=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    kbar = (torch.randn((n_docs * cpd, heads, dim), generator=g, device=DEV) / 8).to(dtype)
    norm = torch.linalg.vector_norm(kbar.float(), dim=-1).contiguous()   # recomputed below by pool parity
    q_r = torch.randn((batch, q_len, heads, dim), generator=g, device=DEV).to(dtype)
    if planted is not None:
        # copy doc `planted`'s chunks into some tokens of every sequence
        for t in range(0, q_len, 3):
            q_r[:, t] = (kbar[planted * cpd + t % cpd].float() + 0.02 * torch.randn_like(q_r[:, t].float())).to(dtype)
    return q_r, kbar, norm


@pytest.mark.parametrize("batch,q_len,heads,dim,n_docs,cpd,dtype", [
    (1, 32, 2, 64, 64, 8, torch.float32),         # tiny workload shapes
    (1, 256, 8, 128, 96, 8, torch.bfloat16),      # prefill-like, ragged column tile
    (4, 1, 8, 128, 300, 8, torch.bfloat16),       # decode-like
    (3, 4, 8, 128, 77, 8, torch.bfloat16),        # short queries, several sequences
    (2, 64, 8, 128, 129, 8, torch.bfloat16),
    (1, 33, 8, 128, 40, 8, torch.bfloat16),       # odd query length
    (2, 16, 4, 64, 50, 4, torch.bfloat16),        # other head count / dim / chunks
    (1, 8, 3, 96, 20, 5, torch.bfloat16),         # shape-general path
    # MFMA tiled path: direct, and sequences over several row tiles (atomic maxima), ragged column tiles
    (1, 512, 8, 128, 100, 8, torch.bfloat16),     # 2 row tiles per sequence
    (3, 96, 8, 128, 70, 8, torch.bfloat16),       # sequences straddle 256-row tiles
    (5, 64, 8, 128, 33, 8, torch.bfloat16),       # several sequences per tile, direct
    (1, 2048, 8, 128, 300, 8, torch.bfloat16),    # prefill query length
    (1, 512, 8, 128, 64, 16, torch.bfloat16),     # 16 chunks per document
    (1, 256, 4, 128, 90, 8, torch.bfloat16),      # 4 heads
    (1, 256, 1, 128, 64, 2, torch.bfloat16),      # 1 head
    # tiled workgroup order with several row groups (uneven where the row tiles
    # do not divide): 10 row tiles in 4 groups, 12 in 4, 17 (the last ragged) in 8
    (5, 512, 8, 128, 40, 8, torch.bfloat16),
    (3, 1024, 8, 128, 36, 8, torch.bfloat16),
    (1, 4288, 8, 128, 35, 8, torch.bfloat16),
    # MFMA stream path: odd head counts, 16 heads, one chunk per document
    (2, 32, 5, 128, 50, 8, torch.bfloat16),
    (1, 8, 16, 128, 40, 8, torch.bfloat16),
    (2, 2, 8, 128, 200, 1, torch.bfloat16),
    (32, 1, 8, 128, 2048, 8, torch.bfloat16),     # decode: 32 sequences x 1 token
    (2, 16, 8, 128, 100, 32, torch.bfloat16),     # 32 chunks per document
    # HBM scan path with 2 and 4 query blocks of 32 rows (8 heads)
    (4, 16, 8, 128, 150, 8, torch.bfloat16),      # 64 rows, 16-token sequences
    (1, 64, 8, 128, 150, 8, torch.bfloat16),      # one sequence over both wave groups
    (1, 128, 8, 128, 170, 8, torch.bfloat16),     # one sequence over four query blocks
    (3, 32, 8, 128, 90, 8, torch.bfloat16),       # 96 rows: the fourth block is empty
    (128, 1, 8, 128, 60, 8, torch.bfloat16),      # 128 single-token sequences
    (20, 4, 8, 128, 61, 4, torch.bfloat16),       # 80 rows, 4 chunks per document
    (9, 8, 8, 128, 45, 16, torch.bfloat16),       # 72 rows, 16 chunks per document
    (5, 16, 8, 128, 33, 32, torch.bfloat16),      # 80 rows, 32 chunks per document
    (33, 2, 8, 128, 70, 2, torch.bfloat16),       # 66 rows, 2 chunks per document
])
def test_route_parity(batch, q_len, heads, dim, n_docs, cpd, dtype):
    case(f"route B={batch} T={q_len} H={heads} d={dim} N={n_docs} C={cpd} {dtype}")
    q_r, kbar, _ = _route_case(batch, q_len, heads, dim, n_docs, cpd, dtype, seed=q_len * 7 + n_docs,
                               planted=min(3, n_docs - 1))
    xbar_norm = torch.linalg.vector_norm(kbar.double(), dim=-1).float().contiguous()
    scores = msa.msa_route_scores(q_r, kbar, xbar_norm, cpd)
    torch.cuda.synchronize()
    ref = route_scores(to_f64(q_r), to_f64(kbar), cpd)
    err = np.abs(to_f64(scores) - ref)
    print(f"  max |route err| = {err.max():.3e}")
    assert err.max() <= ROUTE_ATOL
    # the design target is far tighter than the tolerance: products are exact in fp32
    assert err.max() <= 2e-5


@pytest.mark.parametrize("batch,q_len", [(1, 1), (4, 32), (4, 512)])
def test_route_scan_large_bank_sampled(batch, q_len):
    """The 100M-token shard's bank (195,313 documents x 8 chunks x 8 heads x 128,
    3.2 GB bf16); the scores of sampled documents against the oracle on those
    documents' chunks.  Up to 128 query tokens this is the streaming scan; the
    shard's own query batch, 4 sequences x 512 tokens, runs the tiled MFMA path
    over the whole bank (about 6.5 TFLOP, some 9 ms)."""
    case(f"route scan large bank B={batch} T={q_len} (sampled)")
    n_docs, cpd = 195313, 8
    g = torch.Generator(device=DEV)
    g.manual_seed(11 + batch)
    kbar = torch.empty((n_docs * cpd, 8, 128), device=DEV, dtype=torch.bfloat16)
    for lo in range(0, n_docs * cpd, 1 << 18):                 # slabs: bounded fp32 temporaries
        hi = min(n_docs * cpd, lo + (1 << 18))
        kbar[lo:hi] = torch.randn((hi - lo, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    norm = torch.linalg.vector_norm(kbar.float(), dim=-1).contiguous()
    q_r = torch.randn((batch, q_len, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    scores = msa.msa_route_scores(q_r, kbar, norm, cpd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(batch)
    docs = np.unique(np.concatenate([[0, 1, n_docs // 2, n_docs - 1], rng.integers(0, n_docs, 60)]))
    rows = torch.as_tensor((docs[:, None] * cpd + np.arange(cpd)).ravel(), device=DEV)
    ref = route_scores(to_f64(q_r), to_f64(kbar[rows]), cpd)
    got = to_f64(scores)[:, docs]
    assert np.abs(got - ref).max() <= 2e-5
    del kbar


def test_route_zero_rows():
    case("route zero rows")
    q_r = torch.zeros((1, 32, 8, 128), device=DEV, dtype=torch.bfloat16)
    q_r[0, 5] = 1.0
    kbar = torch.randn((64 * 8, 8, 128), device=DEV).to(torch.bfloat16)
    kbar[8:16] = 0                                   # doc 1 all zero
    norm = torch.linalg.vector_norm(kbar.double(), dim=-1).float().contiguous()
    scores = msa.msa_route_scores(q_r, kbar, norm, 8)
    torch.cuda.synchronize()
    ref = route_scores(to_f64(q_r), to_f64(kbar), 8)
    assert np.abs(to_f64(scores) - ref).max() <= 2e-5
    assert float(scores[0, 1]) == 0.0


def test_pool_then_route_tiny_planted():
    case("tiny pool+route planted")
    cfg = mi.TINY
    for seed in range(3):
        t = mi.draw_tiny(seed)
        k_r = t["k_r"].to(DEV)
        kbar_r, knorm = msa.msa_pool_chunks(k_r, cfg.chunk, with_norm=True)
        q_r = mi.plant_router_queries(kbar_r, t["planted"].to(DEV), t["q_r_noise"].to(DEV), cfg)
        scores = msa.msa_route_scores(q_r, kbar_r, knorm, cfg.chunks_per_doc)
        torch.cuda.synchronize()
        ref = route_scores(to_f64(q_r), to_f64(kbar_r), cfg.chunks_per_doc)
        assert np.abs(to_f64(scores) - ref).max() <= 1e-5
        assert int(torch.argmax(scores[0])) == 7
        # the stored fp32 bank equals the oracle's rounded mean within the fp32 bound
        exact = pool_chunks_mean(to_f64(k_r), cfg.chunk)
        assert np.abs(to_f64(kbar_r) - round_f32(exact)).max() <= 4 * 2.0 ** -24 * np.abs(exact).max()
