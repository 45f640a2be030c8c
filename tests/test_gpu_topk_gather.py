"""GPU parity of S3 (top-k) and S4 (gather, device and host tier), through the C ABI."""

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from oracle import gather_kv, topk_docs
from tests.parity import case, to_f64, topk_band_check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_topk(scores, k):
    ids, vals = msa.msa_topk_docs(scores, k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), vals.cpu().numpy()


@pytest.mark.parametrize("batch,n,k", [
    (1, 64, 4), (1, 2048, 16), (32, 2048, 16), (1, 4096, 16), (2, 4097, 16), (4, 195313, 16),
    (1, 19532, 32), (1, 5000, 1024), (3, 1024, 1024), (2, 100, 1), (1, 12289, 300), (2, 1, 1),
])
def test_topk_exact(batch, n, k):
    case(f"topk B={batch} N={n} k={k}")
    g = torch.Generator(device=DEV)
    g.manual_seed(n + k)
    scores = torch.randn((batch, n), generator=g, device=DEV)
    ids, vals = _gpu_topk(scores, k)
    ref_ids, ref_vals = topk_docs(to_f64(scores), k)
    # same input scores on both sides: the selection is exact (integer work)
    assert np.array_equal(ids, ref_ids)
    assert np.array_equal(vals.astype(np.float64), ref_vals)


def test_topk_ties_and_signed_zero():
    case("topk ties")
    s = torch.zeros((2, 5000), device=DEV)
    s[0, ::7] = -0.0                     # -0.0 ties with +0.0: lower ids first
    s[0, 1000:1010] = 1.0
    s[1] = torch.tensor([0.5, -0.0, 0.0, 0.5] * 1250, device=DEV)
    ids, vals = _gpu_topk(s, 20)
    ref_ids, ref_vals = topk_docs(to_f64(s), 20)
    assert np.array_equal(ids, ref_ids)
    assert ids[0, :10].tolist() == list(range(1000, 1010))
    assert ids[0, 10:].tolist() == list(range(10))
    assert ids[1, :4].tolist() == [0, 3, 4, 7]


@pytest.mark.parametrize("n", [2048, 4096])
@pytest.mark.parametrize("k", [1, 5, 12, 16, 40, 64])
def test_topk_small_path_ties(n, k):
    """Rows of one tile (the routing and decode sizes): all-equal rows, signed zeros, -inf and
    repeated values, against the oracle (ties to the lower id)."""
    case(f"topk small path ties N={n} k={k}")
    s = torch.full((4, n), 0.5, device=DEV)                                  # row 0: all equal
    s[1] = torch.tensor([0.0, -0.0] * (n // 2), device=DEV)
    s[1, 3::97] = 1.0                                                        # row 1: +-0 and a few ones
    s[2] = float("-inf")
    s[2, n - 1] = 2.0
    s[2, 7] = 2.0                                                            # row 2: two equal maxima, rest -inf
    g = torch.Generator(device=DEV)
    g.manual_seed(n + k)
    s[3] = torch.randint(0, 8, (n,), generator=g, device=DEV).float()        # row 3: eight values, many ties
    ids, vals = _gpu_topk(s, k)
    ref_ids, ref_vals = topk_docs(to_f64(s), k)
    assert np.array_equal(ids, ref_ids)
    assert np.array_equal(vals.astype(np.float64), ref_vals)


def test_topk_infinities_and_all_equal():
    case("topk inf")
    s = torch.full((1, 9000), 0.25, device=DEV)
    s[0, 17] = float("inf")
    s[0, 8999] = float("-inf")
    s[0, 4096] = 0.75
    ids, _ = _gpu_topk(s, 5)
    assert ids[0].tolist() == [17, 4096, 0, 1, 2]
    s2 = torch.full((1, 9000), float("-inf"), device=DEV)
    ids, _ = _gpu_topk(s2, 3)
    assert ids[0].tolist() == [0, 1, 2]


def test_topk_band_comparator_on_route_like_scores():
    case("topk band")
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    s = (0.3 + 0.03 * torch.randn((8, 2048), generator=g, device=DEV))
    ids, _ = _gpu_topk(s, 16)
    ok, exact = topk_band_check(ids, to_f64(s), 16)
    assert ok and exact


def test_topk_deterministic():
    case("topk determinism")
    s = torch.randn((4, 50000), device=DEV)
    a, _ = _gpu_topk(s, 64)
    b, _ = _gpu_topk(s, 64)
    assert np.array_equal(a, b)


def _bank(n_docs, cpd, heads, dim, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    kb = torch.randn((n_docs * cpd, heads, dim), generator=g, device=DEV).to(dtype)
    vb = torch.randn((n_docs * cpd, heads, dim), generator=g, device=DEV).to(dtype)
    return kb, vb


@pytest.mark.parametrize("n_docs,cpd,heads,dim,batch,k,dtype", [
    (2048, 8, 8, 128, 1, 16, torch.bfloat16),
    (2048, 8, 8, 128, 32, 32, torch.bfloat16),
    (64, 8, 2, 64, 1, 4, torch.float32),
    (10, 3, 1, 8, 2, 10, torch.bfloat16),
])
def test_gather_bit_exact(n_docs, cpd, heads, dim, batch, k, dtype):
    case(f"gather N={n_docs} C={cpd} B={batch} k={k}")
    kb, vb = _bank(n_docs, cpd, heads, dim, dtype, n_docs + k)
    ids = torch.stack([torch.randperm(n_docs, device=DEV)[:k] for _ in range(batch)]).to(torch.int32)
    ks, vs = msa.msa_gather_kv(kb, vb, ids, cpd)
    torch.cuda.synchronize()
    raw = torch.int16 if dtype == torch.bfloat16 else torch.int32     # compare bit patterns
    rk, rv = gather_kv(kb.cpu().view(raw).numpy(), vb.cpu().view(raw).numpy(),
                       ids.cpu().numpy().astype(np.int64), cpd)
    assert np.array_equal(ks.cpu().view(raw).numpy(), rk)
    assert np.array_equal(vs.cpu().view(raw).numpy(), rv)


def test_gather_out_of_range_is_zero_and_checked_raises():
    case("gather out of range")
    kb, vb = _bank(16, 8, 8, 128, torch.bfloat16, 3)
    ids = torch.tensor([[3, 16, -1, 15]], dtype=torch.int32, device=DEV)
    ks, vs = msa.msa_gather_kv(kb, vb, ids, 8)
    torch.cuda.synchronize()
    assert torch.equal(ks[0, :8], kb[24:32]) and torch.equal(ks[0, 24:32], kb[120:128])
    assert not ks[0, 8:24].any() and not vs[0, 8:24].any()
    with pytest.raises(msa.MsaError, match="outside"):
        msa.msa_gather_kv(kb, vb, ids, 8, checked=True)
    ok_ids = torch.tensor([[3, 1]], dtype=torch.int32, device=DEV)
    msa.msa_gather_kv(kb, vb, ok_ids, 8, checked=True)


@pytest.mark.parametrize("host_memcpy", [False, True])
def test_host_tier_equals_device_gather(host_memcpy):
    case(f"gather host tier memcpy={host_memcpy}")
    kb, vb = _bank(512, 8, 8, 128, torch.bfloat16, 11)
    hk = kb.cpu().pin_memory()
    hv = vb.cpu().pin_memory()
    ids = torch.stack([torch.randperm(512, device=DEV)[:16] for _ in range(4)]).to(torch.int32)
    dk, dv = msa.msa_gather_kv(kb, vb, ids, 8)
    tk, tv = msa.msa_gather_kv(hk, hv, ids, 8, host_memcpy=host_memcpy)
    torch.cuda.synchronize()
    assert torch.equal(dk, tk) and torch.equal(dv, tv)


def test_host_tier_rejects_pageable_memory():
    case("gather pageable")
    kb = torch.zeros((64, 8, 128), dtype=torch.bfloat16)      # not pinned
    ids = torch.zeros((1, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="pinned"):
        msa.msa_gather_kv(kb, kb, ids, 8)


def test_host_tier_memcpy_waits_only_for_its_own_stream():
    """The per-document copies of the host tier while a routing launch runs on
    another stream (queued before the call, so the host's wait for the ids
    overlaps it) and another is queued on the same stream behind the copies:
    the fetched rows equal the device gather, and both routings are intact."""
    case("gather host tier memcpy overlapped with routing")
    n_docs, cpd = 4096, 8
    kb, vb = _bank(n_docs, cpd, 8, 128, torch.bfloat16, 21)
    hk, hv = kb.cpu().pin_memory(), vb.cpu().pin_memory()
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    kr = torch.randn((n_docs * cpd, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    norm = torch.linalg.vector_norm(kr.float(), dim=-1).contiguous()
    q_small = torch.randn((4, 1, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    q_big = torch.randn((4, 512, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    ref_big = msa.msa_route_scores(q_big, kr, norm, cpd)
    torch.cuda.synchronize()
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(a):
        sc = msa.msa_route_scores(q_small, kr, norm, cpd)
        ids, _ = msa.msa_topk_docs(sc, 16)
    with torch.cuda.stream(b):                       # queued before the host-tier call
        big = msa.msa_route_scores(q_big, kr, norm, cpd)
        done_b = torch.cuda.Event()
        done_b.record(b)
    with torch.cuda.stream(a):
        tk, tv = msa.msa_gather_kv(hk, hv, ids, cpd, host_memcpy=True)
        b_running = not done_b.query()               # reported, not asserted: timing dependent
        after = msa.msa_route_scores(q_big, kr, norm, cpd)     # queued behind the copies
    torch.cuda.synchronize()
    print(f"  the other stream's routing was {'still running' if b_running else 'done'} when the call returned")
    dk, dv = msa.msa_gather_kv(kb, vb, ids, cpd)
    torch.cuda.synchronize()
    assert torch.equal(dk, tk) and torch.equal(dv, tv)
    assert torch.equal(big, ref_big) and torch.equal(after, ref_big)


def test_checked_gathers_in_threads_report_their_own_ids():
    """Checked gathers from several threads at once, each on its own stream,
    some with an out-of-range id: each call reports exactly its own result."""
    import threading
    case("checked gathers from 8 threads")
    kb, vb = _bank(64, 8, 8, 128, torch.bfloat16, 4)
    results = {}

    def worker(i):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            bad = i % 2 == 1
            ids = torch.tensor([[1, 64 if bad else 2, 3]], dtype=torch.int32, device=DEV)
            out = []
            for _ in range(20):
                try:
                    msa.msa_gather_kv(kb, vb, ids, 8, checked=True)
                    out.append(False)
                except msa.MsaError:
                    out.append(True)
            results[i] = (bad, out)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, (bad, out) in results.items():
        assert out == [bad] * 20, (i, out)


def test_binding_checks_output_shapes():
    """Caller-supplied outputs of the wrong shape are refused before any launch."""
    case("binding output shape checks")
    kb, vb = _bank(16, 8, 8, 128, torch.bfloat16, 1)
    ids = torch.tensor([[1, 2]], dtype=torch.int32, device=DEV)
    small = torch.empty((1, 8, 8, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="k_sel"):
        msa.msa_gather_kv(kb, vb, ids, 8, k_sel=small)
    with pytest.raises(ValueError, match="whole number"):
        msa.msa_gather_kv(kb[:100], vb[:100], ids, 8)
    scores = torch.randn((2, 16), device=DEV)
    with pytest.raises(ValueError, match="topk_ids"):
        msa.msa_topk_docs(scores, 4, topk_ids=torch.empty((2, 3), dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError, match="topk_scores"):
        msa.msa_topk_docs(scores, 4, topk_scores=torch.empty((1, 4), device=DEV))
    q_r = torch.randn((2, 4, 8, 128), device=DEV).to(torch.bfloat16)
    norm = torch.linalg.vector_norm(kb.float(), dim=-1).contiguous()
    with pytest.raises(ValueError, match="doc_scores"):
        msa.msa_route_scores(q_r, kb, norm, 8, doc_scores=torch.empty((2, 15), device=DEV))
    q = torch.randn((1, 4, 8, 128), device=DEV).to(torch.bfloat16)
    kl = torch.randn((1, 4, 2, 128), device=DEV).to(torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        msa.msa_sparse_attn(q, None, None, kl, kl, out=torch.empty((1, 3, 8, 128), dtype=torch.bfloat16,
                                                                   device=DEV))
    with pytest.raises(ValueError, match="lse"):
        msa.msa_sparse_attn(q, None, None, kl, kl, lse=torch.empty((1, 8, 3), device=DEV))
