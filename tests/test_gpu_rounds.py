"""GPU parity of multi-round routing (Memory Interleave at kernel level): the
top-k with an exclusion set, and the rounds of routing, against the oracle."""

import math

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from oracle import route_scores, topk_docs, topk_docs_excluding
from tests.parity import case, to_f64, topk_band_check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("batch,n,k,n_excl", [
    (1, 100, 10, 0),          # no exclusion: plain top-k
    (2, 100, 10, 90),         # k + n_excl = n: exactly the remaining documents
    (3, 4096, 16, 48),        # one tile
    (2, 4097, 16, 200),       # two tiles, the second holding one document
    (4, 195313, 16, 64),      # many tiles, rounds of reduction
    (1, 12289, 300, 1000),    # large k
    (2, 5000, 1024, 3000),
])
def test_topk_excluding_exact(batch, n, k, n_excl):
    case(f"topk excluding B={batch} N={n} k={k} n_excl={n_excl}")
    g = torch.Generator(device=DEV)
    g.manual_seed(n + k + n_excl)
    # rounded scores: many ties, broken by the lower id
    scores = torch.round(torch.randn((batch, n), generator=g, device=DEV) * 8) / 8
    rng = np.random.default_rng(n_excl)
    excl = np.empty((batch, n_excl), dtype=np.int32)
    for b in range(batch):
        if n_excl and k + n_excl == n:
            excl[b] = rng.permutation(n)[:n_excl]               # distinct: exactly k remain
        elif n_excl:
            # the best documents first (so the exclusion matters), then random ids,
            # repeats, padding and out-of-range entries
            best = np.argsort(-to_f64(scores[b]), kind="stable")[: n_excl // 2]
            rest = rng.integers(-2, n + 2, n_excl - len(best))
            excl[b] = np.concatenate([best, rest])
    ex_t = torch.as_tensor(excl, device=DEV)
    ids, vals = msa.msa_topk_docs_excluding(scores, k, ex_t)
    torch.cuda.synchronize()
    ref_ids, ref_vals = topk_docs_excluding(to_f64(scores), k, excl)
    # the same float32 scores on both sides: the selection is exact
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.array_equal(vals.cpu().numpy().astype(np.float64), ref_vals)


def test_topk_excluding_everything_in_one_tile():
    case("topk excluding a whole tile")
    n, k = 3 * 4096, 8
    s = torch.zeros((1, n), device=DEV)
    s[0, 4096:8192] = torch.linspace(1.0, 2.0, 4096, device=DEV)
    excl = torch.arange(4096, 8192, dtype=torch.int32, device=DEV)[None]
    ids, _ = msa.msa_topk_docs_excluding(s, k, excl)
    torch.cuda.synchronize()
    assert ids[0].tolist() == list(range(k))                    # ties at 0.0 go to the lower ids


def _bank(n_docs, cpd, heads, dim, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    raw = (torch.randn((n_docs, cpd * 64, heads, dim), generator=g, device=DEV) / math.sqrt(dim)).to(torch.bfloat16)
    kbar, norm = msa.msa_pool_chunks(raw, 64, with_norm=True)
    del raw
    return kbar, norm


def _planted_queries(kbar, cpd, rounds, batch, q_len, seed, docs_per_round):
    """Round r's queries copy pooled rows of its own documents plus noise."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    n_docs = kbar.shape[0] // cpd
    heads, dim = kbar.shape[1:]
    rng = np.random.default_rng(seed)
    q = torch.empty((rounds, batch, q_len, heads, dim), dtype=torch.bfloat16, device=DEV)
    for r in range(rounds):
        for b in range(batch):
            docs = rng.choice(n_docs, docs_per_round, replace=False)
            t = np.arange(q_len)
            rows = torch.as_tensor(docs[t % docs_per_round] * cpd + t % cpd, device=DEV)
            noise = torch.randn((q_len, heads, dim), generator=g, device=DEV) * (0.1 / math.sqrt(dim))
            q[r, b] = (kbar[rows].float() + noise).to(torch.bfloat16)
    return q


def _check_rounds(q, kbar, norm, cpd, k, ids, vals):
    """Stage-wise: round r against the oracle's scores of its own query, with
    the GPU's earlier picks as the exclusion set."""
    rounds, batch = q.shape[:2]
    ids = ids.cpu().numpy()
    vals = vals.cpu().numpy()
    kb = to_f64(kbar)
    exact_rounds = 0
    for r in range(rounds):
        s = route_scores(to_f64(q[r]), kb, cpd)
        got = ids[:, r * k:(r + 1) * k]
        prev = ids[:, :r * k]
        for b in range(batch):
            assert not set(got[b].tolist()) & set(prev[b].tolist()), "a round re-selected a document"
        # the band rule over the documents left after the exclusion
        masked = s.copy()
        for b in range(batch):
            masked[b, prev[b]] = -np.inf
        ok, exact = topk_band_check(got, masked, k)
        assert ok
        exact_rounds += exact
        sel = np.take_along_axis(s, got.astype(np.int64), axis=1)
        assert np.abs(vals[:, r * k:(r + 1) * k] - sel).max() <= 1e-3
    return exact_rounds


@pytest.mark.parametrize("n_docs,cpd,heads,dim,rounds,batch,q_len,k", [
    (64, 8, 2, 64, 3, 1, 32, 4),            # small bank, f32-sized shapes in bf16
    (300, 8, 8, 128, 4, 2, 16, 16),         # scan routing, several rounds
    (2048, 8, 8, 128, 3, 1, 256, 16),       # tiled routing (T > 128)
    (5000, 8, 8, 128, 2, 4, 1, 16),         # many top-k tiles, decode-sized queries
])
def test_route_rounds_parity(n_docs, cpd, heads, dim, rounds, batch, q_len, k):
    case(f"route rounds N={n_docs} R={rounds} B={batch} T={q_len} k={k}")
    kbar, norm = _bank(n_docs, cpd, heads, dim, seed=n_docs)
    q = _planted_queries(kbar, cpd, rounds, batch, q_len, seed=rounds + q_len, docs_per_round=k // 2)
    ids, vals = msa.msa_route_rounds(q, kbar, norm, cpd, k)
    torch.cuda.synchronize()
    exact = _check_rounds(q, kbar, norm, cpd, k, ids, vals)
    print(f"  rounds with the exact oracle order: {exact} of {rounds}")


def test_route_rounds_fixed_query_is_one_larger_topk():
    """The same query in every round selects, in order, the top rounds*k of
    one round: a property that holds exactly on the GPU at the 1M-token size."""
    case("route rounds fixed query, 1M-token bank")
    cpd, k, rounds = 8, 16, 3
    kbar, norm = _bank(2048, cpd, 8, 128, seed=5)
    q1 = _planted_queries(kbar, cpd, 1, 1, 2048, seed=6, docs_per_round=16)
    q = q1.expand(rounds, *q1.shape[1:]).contiguous()
    ids, vals = msa.msa_route_rounds(q, kbar, norm, cpd, k)
    s = msa.msa_route_scores(q1[0], kbar, norm, cpd)
    one_ids, one_vals = msa.msa_topk_docs(s, rounds * k)
    torch.cuda.synchronize()
    assert torch.equal(ids, one_ids) and torch.equal(vals, one_vals)


@pytest.mark.parametrize("batch,q_len", [(2, 256), (1, 512)])
def test_route_rounds_fused_launch_matches_separate_calls(batch, q_len):
    """Shapes the tiled kernel routes both per round and for all rounds together: the rounds' routing
    runs as one launch, and its picks and scores equal round-by-round calls bit for bit (one 256-row
    tile per sequence, and sequences over two tiles merged by atomic maxima)."""
    case(f"route rounds, one routing launch: B={batch} T={q_len}")
    cpd, k, rounds = 8, 16, 3
    kbar, norm = _bank(1000, cpd, 8, 128, seed=10)
    q = _planted_queries(kbar, cpd, rounds, batch, q_len, seed=11, docs_per_round=8)
    ids, vals = msa.msa_route_rounds(q, kbar, norm, cpd, k)
    prev = torch.full((batch, 1), -1, dtype=torch.int32, device=DEV)
    for r in range(rounds):
        s = msa.msa_route_scores(q[r], kbar, norm, cpd)
        i_r, v_r = msa.msa_topk_docs_excluding(s, k, prev)
        assert torch.equal(i_r, ids[:, r * k:(r + 1) * k]) and torch.equal(v_r, vals[:, r * k:(r + 1) * k])
        prev = ids[:, :(r + 1) * k].contiguous()
    torch.cuda.synchronize()


def test_route_rounds_matches_separate_calls():
    """msa_route_rounds equals route + top-k-excluding called round by round."""
    case("route rounds vs separate calls")
    cpd, k, rounds = 8, 16, 3
    kbar, norm = _bank(1000, cpd, 8, 128, seed=8)
    q = _planted_queries(kbar, cpd, rounds, 2, 64, seed=9, docs_per_round=8)
    ids, vals = msa.msa_route_rounds(q, kbar, norm, cpd, k)
    prev = torch.full((2, 1), -1, dtype=torch.int32, device=DEV)
    for r in range(rounds):
        s = msa.msa_route_scores(q[r], kbar, norm, cpd)
        i_r, v_r = msa.msa_topk_docs_excluding(s, k, prev)
        assert torch.equal(i_r, ids[:, r * k:(r + 1) * k]) and torch.equal(v_r, vals[:, r * k:(r + 1) * k])
        prev = ids[:, :(r + 1) * k].contiguous()
    torch.cuda.synchronize()
    # the gathered memory of all rounds is the rounds' documents in order
    vbar = kbar.clone()
    k_sel, _ = msa.msa_gather_kv(kbar, vbar, ids, cpd)
    torch.cuda.synchronize()
    rows = (ids.long()[:, :, None] * cpd + torch.arange(cpd, device=DEV)).reshape(2, -1)
    assert torch.equal(k_sel, kbar[rows])
