"""Pins for the oracle's cosine routing.

Cosine similarity, averaged over heads, then the max over query tokens: MSA
README, "Overall Design"; the per-layer cosine router over the chunk-pooled
bank: william-0g/MSA-Qwen3.5 model card, opening paragraph.  The max over a
document's chunks is the reading used throughout this implementation.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.spatial.distance import cdist

import msa_inputs as mi
from oracle import pool_chunks_stored, route_scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_route(q, k, c, eps=1e-12):
    b_, t_, h_, d_ = q.shape
    n_ch = k.shape[0]
    out = np.full((b_, n_ch // c), -np.inf)
    for b in range(b_):
        for n in range(n_ch):
            for t in range(t_):
                acc = 0.0
                for h in range(h_):
                    dot = sum(float(q[b, t, h, e]) * float(k[n, h, e]) for e in range(d_))
                    nq = math.sqrt(sum(float(q[b, t, h, e]) ** 2 for e in range(d_)))
                    nk = math.sqrt(sum(float(k[n, h, e]) ** 2 for e in range(d_)))
                    acc += dot / (max(nq, eps) * max(nk, eps))
                s = acc / h_
                out[b, n // c] = max(out[b, n // c], s)
    return out


def test_bruteforce_tiny():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 3, 2, 5))
    k = rng.standard_normal((12, 2, 5))
    for c in (1, 3, 4):
        np.testing.assert_allclose(route_scores(q, k, c), _brute_route(q, k, c), atol=1e-13)


def test_range_and_scale_invariance():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 5, 3, 8))
    k = rng.standard_normal((20, 3, 8))
    s = route_scores(q, k, 4)
    assert np.all(s <= 1 + 1e-12) and np.all(s >= -1 - 1e-12)
    qs = q * rng.uniform(0.1, 10, (2, 5, 3, 1))
    ks = k * rng.uniform(0.1, 10, (20, 3, 1))
    np.testing.assert_allclose(route_scores(qs, ks, 4), s, atol=1e-13)


def test_doc_permutation_equivariance():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 2, 6))
    k = rng.standard_normal((6 * 4, 2, 6))
    perm = rng.permutation(6)
    kp = k.reshape(6, 4, 2, 6)[perm].reshape(24, 2, 6)
    np.testing.assert_allclose(route_scores(q, kp, 4), route_scores(q, k, 4)[:, perm], atol=1e-14)


def test_single_head_token_chunk_is_cosine_similarity():
    # H = T = C = 1: the score is the plain cosine similarity (SciPy cdist).
    rng = np.random.default_rng(3)
    q = rng.standard_normal((7, 1, 1, 16))
    k = rng.standard_normal((30, 1, 16))
    ref = 1.0 - cdist(q[:, 0, 0], k[:, 0], metric="cosine")
    np.testing.assert_allclose(route_scores(q, k, 1), ref, atol=1e-13)


def test_head_mean_of_cosines_not_cosine_of_concatenation():
    # Head 0 aligned (+1), head 1 opposite (-1) with 10x the norm: the head
    # mean is exactly 0; the cosine of the concatenated vectors would be
    # (1 - 10) / (sqrt(101) * sqrt(2)).
    q = np.array([[[[1.0, 0.0], [10.0, 0.0]]]])          # [B=1, T=1, H=2, d=2]
    k = np.array([[[1.0, 0.0], [-1.0, 0.0]]])            # [N_ch=1, H=2, d=2]
    assert route_scores(q, k, 1)[0, 0] == 0.0


def test_max_over_tokens_and_chunks():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((5 * 8, 2, 4))
    q = rng.standard_normal((1, 6, 2, 4))
    q[0, 4] = k[3 * 8 + 5] * 2.5            # token 4 copies chunk 5 of doc 3 (scaled)
    s = route_scores(q, k, 8)
    assert s[0, 3] == pytest.approx(1.0, abs=1e-14)
    assert np.argmax(s[0]) == 3


def test_zero_rows_score_zero():
    q = np.zeros((1, 1, 2, 3))
    k = np.ones((2, 2, 3))
    np.testing.assert_array_equal(route_scores(q, k, 1), [[0.0, 0.0]])


def test_golden_hand_worked():
    with open(os.path.join(GOLDEN, "route_hand.json")) as f:
        g = json.load(f)
    q = np.array(g["q_r"], dtype=np.float64)
    k = np.array(g["kbar_r"], dtype=np.float64)
    got = route_scores(q, k, g["chunks_per_doc"])
    np.testing.assert_allclose(got, np.array(g["expected"]), atol=1e-15)


@pytest.mark.parametrize("seed", range(5))
def test_planted_doc_ranks_first_tiny(seed):
    cfg = mi.TINY
    t = mi.draw_tiny(seed)
    kbar_r = pool_chunks_stored(t["k_r"].double().numpy(), cfg.chunk, "f32")
    q_r = mi.plant_router_queries(torch.from_numpy(kbar_r).float(), t["planted"], t["q_r_noise"], cfg)
    s = route_scores(q_r.double().numpy(), kbar_r, cfg.chunks_per_doc)
    assert int(np.argmax(s[0])) == 7
    # the margin is large (copied pooled rows give cos ~ 0.8 against ~ 0.35)
    assert s[0, 7] - np.sort(s[0])[-2] > 0.2
