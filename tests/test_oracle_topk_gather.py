"""Pins for the oracle's top-k selection and gather.

Top-k documents by routing score, then loading only the selected pooled K/V:
MSA README, "Overall Design" and "Inference Pipeline" stage 2.  Range checks
on gather ids follow the failure recorded on the dormouse ADR-0014 page
(out-of-range block indices made every gather fault).
"""

import numpy as np
import pytest

from oracle import gather_kv, topk_docs


def _brute_topk(s, k):
    ids, vals = [], []
    for row in s:
        order = sorted(range(len(row)), key=lambda d: (-row[d], d))[:k]
        ids.append(order)
        vals.append([row[d] for d in order])
    return np.array(ids), np.array(vals)


@pytest.mark.parametrize("n,k", [(10, 1), (10, 3), (37, 37), (100, 16)])
def test_bruteforce(n, k):
    rng = np.random.default_rng(n + k)
    s = rng.standard_normal((3, n))
    ids, vals = topk_docs(s, k)
    bid, bval = _brute_topk(s, k)
    assert np.array_equal(ids, bid)
    assert np.array_equal(vals, bval)


def test_ties_go_to_lower_id():
    s = np.array([[0.5, 0.9, 0.5, 0.9, 0.1, 0.5]])
    ids, vals = topk_docs(s, 4)
    assert ids.tolist() == [[1, 3, 0, 2]]
    assert vals.tolist() == [[0.9, 0.9, 0.5, 0.5]]
    ids, _ = topk_docs(np.zeros((1, 9)), 5)
    assert ids.tolist() == [[0, 1, 2, 3, 4]]


def test_closed_forms():
    n = 50
    ids, _ = topk_docs(-np.arange(n, dtype=np.float64)[None], 7)
    assert ids.tolist() == [list(range(7))]
    ids, _ = topk_docs(np.arange(n, dtype=np.float64)[None], 7)
    assert ids.tolist() == [list(range(n - 1, n - 8, -1))]


def test_k_bounds():
    with pytest.raises(ValueError):
        topk_docs(np.zeros((1, 4)), 0)
    with pytest.raises(ValueError):
        topk_docs(np.zeros((1, 4)), 5)


def test_gather_bruteforce_and_order():
    rng = np.random.default_rng(0)
    n_doc, c, h, d = 9, 3, 2, 4
    kb = rng.standard_normal((n_doc * c, h, d))
    vb = rng.standard_normal((n_doc * c, h, d))
    ids = np.array([[4, 0, 8], [2, 2, 7]])
    ks, vs = gather_kv(kb, vb, ids, c)
    assert ks.shape == (2, 3 * c, h, d)
    for b in range(2):
        for i in range(3):
            for j in range(c):
                assert np.array_equal(ks[b, i * c + j], kb[ids[b, i] * c + j])
                assert np.array_equal(vs[b, i * c + j], vb[ids[b, i] * c + j])


def test_gather_rejects_out_of_range():
    kb = np.zeros((6, 1, 1))
    with pytest.raises(IndexError):
        gather_kv(kb, kb, np.array([[3]]), 2)
    with pytest.raises(IndexError):
        gather_kv(kb, kb, np.array([[-1]]), 2)
