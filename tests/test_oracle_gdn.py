"""Pins for the oracle's linear-layer variant: the gated delta rule over a
sequence and the injection of the selected documents' states.

The model card (william-0g/MSA-Qwen3.5, "Architecture summary") encodes each
document through the linear layer's recurrence, sums the top-k documents'
states into S_ext, and runs the query path from S_ext as its initial state.
The rule's equations are the published gated delta rule (a reading); these
tests pin the oracle's arithmetic to closed forms and to an independent
formulation with explicit transition matrices.
"""

import numpy as np
import pytest

from oracle import gated_delta_rule, inject_states


def _seq(seed, b_=2, t_=7, h_=3, dk=5, dv=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b_, t_, h_, dk))
    k = rng.standard_normal((b_, t_, h_, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((b_, t_, h_, dv))
    g = -rng.uniform(0.0, 0.5, (b_, t_, h_))
    beta = rng.uniform(0.1, 1.0, (b_, t_, h_))
    h0 = rng.standard_normal((b_, h_, dk, dv))
    return q, k, v, g, beta, h0


def test_transition_matrix_form():
    """h_t = A_t h_{t-1} + B_t with A_t = alpha_t (I - beta_t k_t k_t^T) and
    B_t = beta_t k_t v_t^T, built as explicit matrices."""
    q, k, v, g, beta, h0 = _seq(0)
    scale = 0.37
    o, hT = gated_delta_rule(q, k, v, g, beta, scale=scale, initial_state=h0)
    b_, t_, h_, dk = q.shape
    for b in range(b_):
        for hh in range(h_):
            h = h0[b, hh].copy()
            for t in range(t_):
                kt = k[b, t, hh][:, None]
                a_t = np.exp(g[b, t, hh]) * (np.eye(dk) - beta[b, t, hh] * (kt @ kt.T))
                h = a_t @ h + beta[b, t, hh] * (kt @ v[b, t, hh][None, :])
                np.testing.assert_allclose(o[b, t, hh], scale * (h.T @ q[b, t, hh]), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(hT[b, hh], h, rtol=1e-12, atol=1e-12)


def test_no_writes_only_decays():
    q, k, v, g, beta, h0 = _seq(1)
    beta[:] = 0.0
    o, hT = gated_delta_rule(q, k, v, g, beta, scale=1.0, initial_state=h0)
    decay = np.exp(np.cumsum(g, axis=1))                                      # [B, T, H]
    want_o = decay[..., None] * np.einsum("bhkv,bthk->bthv", h0, q)
    np.testing.assert_allclose(o, want_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hT, decay[:, -1][..., None, None] * h0, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_store_and_replace_values():
    """alpha = beta = 1 and basis-vector keys: writing (e_j, v) makes row j of
    the state equal v exactly (a second write to the same key replaces it), so
    querying e_j returns the last value written there."""
    dk, dv = 6, 3
    keys = [2, 0, 5, 2]
    rng = np.random.default_rng(2)
    vals = rng.standard_normal((len(keys), dv))
    h0 = rng.standard_normal((1, 1, dk, dv))
    k = np.zeros((1, len(keys), 1, dk))
    for t, j in enumerate(keys):
        k[0, t, 0, j] = 1.0
    q = k.copy()
    g = np.zeros((1, len(keys), 1))
    beta = np.ones((1, len(keys), 1))
    o, hT = gated_delta_rule(q, k, vals[None, :, None, :], g, beta, scale=1.0, initial_state=h0)
    for t in range(len(keys)):
        np.testing.assert_allclose(o[0, t, 0], vals[t], rtol=0, atol=1e-15)
    np.testing.assert_allclose(hT[0, 0, 2], vals[3], atol=1e-15)    # rewritten key keeps the last value
    np.testing.assert_allclose(hT[0, 0, 0], vals[1], atol=1e-15)
    np.testing.assert_allclose(hT[0, 0, 5], vals[2], atol=1e-15)
    for j in (1, 3, 4):
        np.testing.assert_allclose(hT[0, 0, j], h0[0, 0, j], atol=0)


def test_split_sequence_carries_the_state():
    q, k, v, g, beta, h0 = _seq(3, t_=9)
    o, hT = gated_delta_rule(q, k, v, g, beta, initial_state=h0)
    o1, h1 = gated_delta_rule(q[:, :4], k[:, :4], v[:, :4], g[:, :4], beta[:, :4], initial_state=h0)
    o2, h2 = gated_delta_rule(q[:, 4:], k[:, 4:], v[:, 4:], g[:, 4:], beta[:, 4:], initial_state=h1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h2, hT, rtol=1e-13, atol=1e-13)


def test_initial_state_enters_linearly():
    """With v = 0 the outputs and final state are linear in the initial state,
    so a sum of injected document states acts as the sum of their effects."""
    q, k, v, g, beta, h0 = _seq(4)
    rng = np.random.default_rng(5)
    h1 = rng.standard_normal(h0.shape)
    z = np.zeros_like(v)
    oa, ha = gated_delta_rule(q, k, z, g, beta, initial_state=h0)
    ob, hb = gated_delta_rule(q, k, z, g, beta, initial_state=h1)
    oc, hc = gated_delta_rule(q, k, z, g, beta, initial_state=h0 + h1)
    np.testing.assert_allclose(oc, oa + ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hc, ha + hb, rtol=1e-12, atol=1e-12)


def test_inject_states_sum_and_range():
    rng = np.random.default_rng(6)
    states = rng.standard_normal((10, 2, 3, 4))
    ids = np.array([[3, 7, 0], [9, 9, 1]])
    s = inject_states(states, ids)
    for b in range(2):
        want = np.zeros((2, 3, 4))
        for i in ids[b]:
            want += states[i]
        np.testing.assert_allclose(s[b], want, rtol=1e-15, atol=0)
    with pytest.raises(IndexError):
        inject_states(states, np.array([[10]]))
