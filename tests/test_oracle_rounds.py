"""Pins for the oracle's multi-round routing (Memory Interleave, kernel level).

Routing may run for several rounds, each jumping to further memory segments:
MSA README, "Inference Pipeline", Figure 3, and the page's FAQ entry on Memory
Interleave.  The readings (a later round never re-selects an earlier pick; the
rounds' picks are concatenated in round order) are this implementation's.
"""

import numpy as np
import pytest

from oracle import pool_chunks_stored, route_rounds, route_scores, topk_docs, topk_docs_excluding


def _brute(scores_row, k, banned):
    """Python's sort over the allowed ids with the key (-score, id)."""
    allowed = [d for d in range(len(scores_row)) if d not in banned]
    best = sorted(allowed, key=lambda d: (-scores_row[d], d))[:k]
    return best, [scores_row[d] for d in best]


def test_hand_worked_exclusion():
    s = np.array([[0.3, 0.9, 0.5, 0.9, 0.1]])
    # without exclusion: 0.9 (doc 1, lower id first), 0.9 (doc 3)
    ids, vals = topk_docs_excluding(s, 2, [[]])
    assert ids.tolist() == [[1, 3]] and vals.tolist() == [[0.9, 0.9]]
    # doc 1 excluded: doc 3, then 0.5 (doc 2)
    ids, vals = topk_docs_excluding(s, 2, [[1]])
    assert ids.tolist() == [[3, 2]] and vals.tolist() == [[0.9, 0.5]]
    # out-of-range ids and padding are ignored, repeats count once
    ids, _ = topk_docs_excluding(s, 3, [[3, 7, -1, 3]])
    assert ids.tolist() == [[1, 2, 0]]


def test_matches_brute_force():
    rng = np.random.default_rng(0)
    for trial in range(30):
        b_, n = 3, int(rng.integers(5, 60))
        s = np.round(rng.standard_normal((b_, n)), 1)          # many ties
        n_ex = int(rng.integers(0, n // 2))
        excl = rng.integers(-3, n + 3, (b_, n_ex))
        k = int(rng.integers(1, n - n_ex + 1))
        ids, vals = topk_docs_excluding(s, k, excl)
        for b in range(b_):
            banned = {int(i) for i in excl[b] if 0 <= i < n}
            bi, bv = _brute(list(s[b]), k, banned)
            assert ids[b].tolist() == bi and vals[b].tolist() == bv


def test_empty_exclusion_is_plain_topk():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((4, 100))
    a = topk_docs_excluding(s, 10, np.full((4, 5), -1))
    b = topk_docs(s, 10)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_too_few_remaining_raises():
    s = np.zeros((1, 4))
    topk_docs_excluding(s, 2, [[0, 1]])
    with pytest.raises(ValueError):
        topk_docs_excluding(s, 3, [[0, 1]])


def _bank(rng, n_doc, cpd, h, d):
    x = rng.standard_normal((n_doc, cpd * 4, h, d))
    return pool_chunks_stored(x, 4, "f32").reshape(n_doc * cpd, h, d)


def test_same_query_every_round_is_one_larger_topk():
    """R rounds of k with a fixed router query select exactly the top R*k of a
    single round, in the same order (closed form of the exclusion)."""
    rng = np.random.default_rng(2)
    kbar = _bank(rng, 40, 3, 2, 8)
    q = rng.standard_normal((2, 5, 2, 8))
    ids, vals = route_rounds([q, q, q], kbar, 3, 4)
    ref_ids, ref_vals = topk_docs(route_scores(q, kbar, 3), 12)
    assert np.array_equal(ids, ref_ids) and np.allclose(vals, ref_vals, rtol=0, atol=0)


def test_rounds_are_disjoint_and_follow_their_queries():
    """Each round's query is planted on pooled rows of its own documents; a
    round whose planted documents were taken earlier moves on to others."""
    rng = np.random.default_rng(3)
    n_doc, cpd, h, d = 64, 2, 2, 16
    kbar = _bank(rng, n_doc, cpd, h, d)

    def planted(doc):
        rows = kbar.reshape(n_doc, cpd, h, d)[doc]                      # [cpd, h, d]
        return (rows + 0.05 * rng.standard_normal(rows.shape))[None]    # [1, T=cpd, h, d]

    q0, q1, q2 = planted(5), planted(9), planted(5)
    ids, vals = route_rounds([q0, q1, q2], kbar, cpd, 1)
    assert ids[0, 0] == 5 and ids[0, 1] == 9
    assert ids[0, 2] not in (5, 9)
    # round 3 is round 1's query with doc 5 and 9 excluded: its second choice
    s2 = route_scores(q2, kbar, cpd)
    assert ids[0, 2] == topk_docs_excluding(s2, 1, [[5, 9]])[0][0, 0]
    assert len(set(ids[0].tolist())) == 3
    assert np.isclose(vals[0, 2], s2[0, ids[0, 2]], rtol=0, atol=0)
