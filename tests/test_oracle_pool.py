"""Pins for the oracle's chunk-mean pooling and chunk norms.

Chunk-mean pooling of K, V and K_r: MSA README, "Overall Design" and
"Inference Pipeline" stage 1.  Pins: element-by-element brute force, a closed
form for rows linear in the position, and mean-of-means invariants.
"""

import math

import numpy as np
import pytest

from oracle import chunk_norms, pool_chunks_mean, pool_chunks_stored
from oracle.bf16 import round_bf16


def _brute_pool(x, chunk):
    n_doc, l_doc, h, d = x.shape
    c = l_doc // chunk
    out = np.zeros((n_doc * c, h, d))
    for n in range(n_doc):
        for j in range(c):
            for hh in range(h):
                for e in range(d):
                    acc = 0.0
                    for i in range(chunk):
                        acc += float(x[n, j * chunk + i, hh, e])
                    out[n * c + j, hh, e] = acc / chunk
    return out


def test_bruteforce_tiny():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 12, 2, 5))
    np.testing.assert_allclose(pool_chunks_mean(x, 4), _brute_pool(x, 4), rtol=0, atol=1e-15)
    np.testing.assert_allclose(pool_chunks_mean(x, 3), _brute_pool(x, 3), rtol=0, atol=1e-15)


def test_closed_form_linear_rows():
    # x[n, i] = a + b * i  =>  mean over chunk j = a + b * (j*c + (c-1)/2), exactly.
    rng = np.random.default_rng(1)
    n_doc, l_doc, h, d, c = 2, 32, 3, 4, 8
    a = rng.integers(-8, 8, (n_doc, 1, h, d)).astype(np.float64)
    b = rng.integers(-8, 8, (n_doc, 1, h, d)).astype(np.float64)
    i = np.arange(l_doc, dtype=np.float64)[None, :, None, None]
    x = a + b * i
    got = pool_chunks_mean(x, c).reshape(n_doc, l_doc // c, h, d)
    for j in range(l_doc // c):
        np.testing.assert_array_equal(got[:, j], (a + b * (j * c + (c - 1) / 2))[:, 0])


def test_constant_chunks_and_mean_of_means():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 64, 2, 3))
    pooled = pool_chunks_mean(x, 16).reshape(4, 4, 2, 3)
    # equal-size chunks: the mean of the chunk means is the mean of all rows
    np.testing.assert_allclose(pooled.mean(axis=1), x.mean(axis=1), atol=1e-14)
    const = np.broadcast_to(rng.standard_normal((4, 1, 2, 3)), (4, 64, 2, 3))
    np.testing.assert_allclose(pool_chunks_mean(const, 16).reshape(4, 4, 2, 3),
                               np.broadcast_to(const[:, :1], (4, 4, 2, 3)), rtol=1e-15, atol=0)


def test_rejects_partial_chunk():
    with pytest.raises(ValueError):
        pool_chunks_mean(np.zeros((1, 10, 1, 1)), 4)


def test_stored_rounding():
    rng = np.random.default_rng(3)
    x = round_bf16(rng.standard_normal((2, 128, 2, 8)))
    stored = pool_chunks_stored(x, 64, "bf16")
    exact = pool_chunks_mean(x, 64)
    assert np.array_equal(stored, round_bf16(exact))
    # within half an ulp of bf16 (8 significant bits)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    assert np.all(np.abs(stored - exact) <= ulp / 2)


def test_norms():
    row = np.zeros((1, 2, 4))
    row[0, 0, :2] = [3.0, 4.0]          # 3-4-5 triangle
    row[0, 1, :] = [1.0, 1.0, 1.0, 1.0]
    np.testing.assert_array_equal(chunk_norms(row), [[5.0, 2.0]])
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 3, 7))
    brute = np.array([[math.sqrt(sum(float(v) ** 2 for v in x[n, h])) for h in range(3)] for n in range(5)])
    np.testing.assert_allclose(chunk_norms(x), brute, rtol=1e-15)
