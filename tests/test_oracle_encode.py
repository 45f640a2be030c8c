"""Pins of the oracle's offline encoder (rotary embedding, variable-length chunk means).

Each check ties the oracle to something other than itself: a hand-worked
fixture, closed forms, invariants of a rotation, an independent formulation
(complex multiplication), and library routines (reshape-mean, add.reduceat).
"""

import json
import os

import numpy as np
import pytest

from oracle import chunk_offsets, encode_docs, pool_chunks_mean, rope_rotate_half

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "encode_hand.json")


def test_hand_worked_fixture():
    g = json.load(open(GOLDEN))
    out, c_off = encode_docs(np.array(g["x"], dtype=np.float64), g["doc_off"], g["chunk"], g["rope_base"])
    assert c_off.tolist() == g["expected_chunk_off"]
    np.testing.assert_allclose(out, np.array(g["expected"]), rtol=0, atol=1e-15)


def test_rope_closed_form_second_pair():
    # d = 4, base b: pair (1, 3) turns by p * b^(-1/2); e_1 -> (cos, sin) on dims (1, 3)
    b, p = 500.0, 7.0
    x = np.zeros((1, 1, 4))
    x[0, 0, 1] = 1.0
    y = rope_rotate_half(x, np.array([p]), b)[0, 0]
    ang = p * b ** -0.5
    np.testing.assert_allclose(y, [0.0, np.cos(ang), 0.0, np.sin(ang)], atol=1e-15)


def test_rope_matches_complex_multiplication():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 3, 16))
    pos = rng.integers(0, 5000, 9)
    base = 1e6
    y = rope_rotate_half(x, pos, base)
    z = x[..., :8] + 1j * x[..., 8:]
    theta = base ** (-np.arange(8) * 2.0 / 16)
    w = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    np.testing.assert_allclose(y, np.concatenate([w.real, w.imag], axis=-1), atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 32))
    k = rng.standard_normal((1, 2, 32))
    base = 1e4
    # position 0 is the identity, and a rotation keeps each head's norm
    np.testing.assert_allclose(rope_rotate_half(q, np.array([0]), base), q, atol=0)
    r = rope_rotate_half(q, np.array([123]), base)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    # scores depend only on the relative position
    for p, pp in [(3, 10), (100, 37), (0, 5)]:
        lhs = (rope_rotate_half(q, np.array([p]), base) * rope_rotate_half(k, np.array([pp]), base)).sum(-1)
        rhs = (q * rope_rotate_half(k, np.array([pp - p]), base)).sum(-1)
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_uniform_lengths_without_rope_is_pooling():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 128, 2, 8))
    out, c_off = encode_docs(x.reshape(5 * 128, 2, 8), np.arange(6) * 128, 32)
    assert c_off.tolist() == [0, 4, 8, 12, 16, 20]
    np.testing.assert_allclose(out, pool_chunks_mean(x, 32), rtol=1e-15, atol=1e-15)
    # and the plain reshape-mean library routine
    np.testing.assert_allclose(out, x.reshape(5, 4, 32, 2, 8).mean(axis=2).reshape(20, 2, 8), atol=1e-14)


@pytest.mark.parametrize("chunk", [1, 3, 8])
def test_variable_lengths_match_reduceat(chunk):
    rng = np.random.default_rng(chunk)
    lens = np.array([0, 1, chunk - 1, chunk, chunk + 1, 5 * chunk + 2, 0, 7])
    lens = np.maximum(lens, 0)
    doc_off = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((int(doc_off[-1]), 2, 4))
    out, c_off = encode_docs(x, doc_off, chunk)
    # chunk starts and sizes, then NumPy's segmented sum
    starts, sizes = [], []
    for n, ln in enumerate(lens):
        for j in range(0, ln, chunk):
            starts.append(doc_off[n] + j)
            sizes.append(min(chunk, ln - j))
    assert len(starts) == c_off[-1]
    sums = np.add.reduceat(x, starts, axis=0) if starts else np.zeros((0, 2, 4))
    np.testing.assert_allclose(out, sums / np.array(sizes)[:, None, None], atol=1e-14)


def test_chunk_offsets():
    assert chunk_offsets([0, 0, 5, 5, 6, 70], 4).tolist() == [0, 0, 2, 2, 3, 19]
    with pytest.raises(ValueError):
        chunk_offsets([0, 3, 2], 4)
    with pytest.raises(ValueError):
        chunk_offsets([1, 3], 4)
