"""Pins for the oracle's sparse-attention backward.

The method's sparse attention is trained end to end (MSA README, "Abstract"
and the Figure 1 caption; model card "Training (CPT)").  The gradients are
pinned by central finite differences of the forward oracle, by torch autograd
through scaled_dot_product_attention in float64 on the CPU, and by the
softmax identities (the rows of P sum to 1, those of dS to 0).
"""

import numpy as np
import pytest
import torch

from oracle import sparse_attention, sparse_attention_backward


def _inputs(seed, b_, t_, hq, hkv, d, m, l_):
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s)
    return r(b_, t_, hq, d), r(b_, m, hkv, d), r(b_, m, hkv, d), r(b_, l_, hkv, d), r(b_, l_, hkv, d), r(b_, t_, hq, d)


SHAPES = [
    (1, 3, 4, 2, 4, 2, 5),     # T < L: a causal band, GQA group 2
    (2, 1, 2, 1, 3, 3, 4),     # decode-like: one token sees everything
    (1, 4, 2, 2, 3, 0, 4),     # no memory rows, T = L
]


@pytest.mark.parametrize("shape", SHAPES)
def test_central_finite_differences(shape):
    q, ks, vs, kl, vl, do = _inputs(0, *shape)
    scale = 0.7
    grads = sparse_attention_backward(q, ks, vs, kl, vl, do, scale=scale)
    args = [q, ks, vs, kl, vl]

    def loss(a):
        o, _ = sparse_attention(*a, scale=scale)
        return float((o * do).sum())

    h = 1e-6
    for i, x in enumerate(args):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[i][idx] += h
            minus[i][idx] -= h
            fd[idx] = (loss(plus) - loss(minus)) / (2 * h)
        np.testing.assert_allclose(grads[i], fd, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("shape", SHAPES + [(2, 6, 8, 2, 16, 5, 9)])
def test_matches_torch_autograd(shape):
    q, ks, vs, kl, vl, do = _inputs(1, *shape)
    b_, t_, hq, hkv, d, m, l_ = shape
    group = hq // hkv
    tq, tks, tvs, tkl, tvl = (torch.tensor(a, requires_grad=True) for a in (q, ks, vs, kl, vl))
    keys = torch.cat([tks, tkl], dim=1).transpose(1, 2).repeat_interleave(group, dim=1)   # [B, Hq, M+L, d]
    vals = torch.cat([tvs, tvl], dim=1).transpose(1, 2).repeat_interleave(group, dim=1)
    j = torch.arange(m + l_)
    t = torch.arange(t_)
    mask = (j[None, :] < m) | ((j[None, :] - m) <= (l_ - t_ + t)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(tq.transpose(1, 2), keys, vals, attn_mask=mask)
    (o.transpose(1, 2) * torch.tensor(do)).sum().backward()
    grads = sparse_attention_backward(q, ks, vs, kl, vl, do)
    for g, t_in in zip(grads, (tq, tks, tvs, tkl, tvl)):
        np.testing.assert_allclose(g, t_in.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_softmax_identities():
    b_, t_, hq, hkv, d, m, l_ = 2, 5, 6, 3, 8, 4, 7
    q, ks, vs, kl, vl, do = _inputs(2, b_, t_, hq, hkv, d, m, l_)
    dq, dks, dvs, dkl, dvl = sparse_attention_backward(q, ks, vs, kl, vl, do)
    # each row of dS sums to 0, so the key gradients of a KV head sum to 0
    np.testing.assert_allclose(dks.sum(axis=1) + dkl.sum(axis=1), 0.0, atol=1e-12)
    # each row of P sums to 1, so the value gradients of a KV head sum to the
    # output gradients of its query heads over all tokens
    want = do.reshape(b_, t_, hkv, hq // hkv, d).sum(axis=(1, 3))
    np.testing.assert_allclose(dvs.sum(axis=1) + dvl.sum(axis=1), want, rtol=1e-12, atol=1e-12)


def test_single_visible_key():
    """One key per row: the softmax is constant, so dq = dk = 0 and dv = dO."""
    q, ks, vs, kl, vl, do = _inputs(3, 1, 1, 2, 2, 4, 0, 1)
    dq, dks, dvs, dkl, dvl = sparse_attention_backward(q, ks, vs, kl, vl, do)
    assert np.all(dq == 0) and np.all(dkl == 0)
    np.testing.assert_allclose(dvl[0, 0], do[0, 0], rtol=0, atol=0)
    assert dks.shape == (1, 0, 2, 4) and dvs.shape == (1, 0, 2, 4)
