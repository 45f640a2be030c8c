"""Pins for the oracle's sparse GQA attention.

Softmax attention over the concatenation of the selected documents' pooled
K/V and the local K/V: william-0g/MSA-Qwen3.5 model card, "Architecture
summary"; MSA README, "Overall Design" and "Inference Pipeline" stage 3.
Pins: brute force with math.exp, closed forms (constant V, one-hot V, zero
query), a hand-worked fixture, the GQA head map, and equality with PyTorch's
scaled_dot_product_attention (float64, CPU) when every document is selected.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax

import msa_inputs as mi
from oracle import (gather_kv, merge_attention, pool_chunks_stored, route_scores, sparse_attention,
                    sparse_attention_rows, topk_docs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(q, ks, vs, kl, vl, scale):
    b_, t_, hq, d = q.shape
    m, l_len, hkv = ks.shape[1], kl.shape[1], ks.shape[2]
    g = hq // hkv
    o = np.zeros_like(q)
    lse = np.zeros((b_, hq, t_))
    for b in range(b_):
        for h in range(hq):
            kvh = h // g
            for t in range(t_):
                keys = [ks[b, i, kvh] for i in range(m)] + [kl[b, j, kvh] for j in range(l_len - t_ + t + 1)]
                vals = [vs[b, i, kvh] for i in range(m)] + [vl[b, j, kvh] for j in range(l_len - t_ + t + 1)]
                logits = [scale * sum(float(q[b, t, h, e]) * float(kk[e]) for e in range(d)) for kk in keys]
                mx = max(logits)
                w = [math.exp(x - mx) for x in logits]
                z = sum(w)
                for e in range(d):
                    o[b, t, h, e] = sum(w[i] * float(vals[i][e]) for i in range(len(w))) / z
                lse[b, h, t] = mx + math.log(z)
    return o, lse


@pytest.mark.parametrize("t_len,l_len", [(3, 3), (2, 5), (1, 4)])
def test_bruteforce(t_len, l_len):
    rng = np.random.default_rng(t_len * 10 + l_len)
    q = rng.standard_normal((2, t_len, 4, 3))
    ks = rng.standard_normal((2, 2, 2, 3))
    vs = rng.standard_normal((2, 2, 2, 3))
    kl = rng.standard_normal((2, l_len, 2, 3))
    vl = rng.standard_normal((2, l_len, 2, 3))
    o, lse = sparse_attention(q, ks, vs, kl, vl, scale=0.7)
    bo, blse = _brute(q, ks, vs, kl, vl, 0.7)
    np.testing.assert_allclose(o, bo, atol=1e-13)
    np.testing.assert_allclose(lse, blse, atol=1e-13)


def test_golden_hand_worked():
    with open(os.path.join(GOLDEN, "attention_hand.json")) as f:
        g = json.load(f)
    arr = {k: np.array(g[k], dtype=np.float64) for k in ("q", "k_sel", "v_sel", "k_loc", "v_loc")}
    o, lse = sparse_attention(arr["q"], arr["k_sel"], arr["v_sel"], arr["k_loc"], arr["v_loc"], scale=g["scale"])
    np.testing.assert_allclose(o, np.array(g["expected_o"]), atol=1e-14)
    np.testing.assert_allclose(lse, np.array(g["expected_lse"]), atol=1e-14)


def test_constant_values_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 6, 4, 8)) * 3
    ks = rng.standard_normal((1, 5, 2, 8))
    kl = rng.standard_normal((1, 9, 2, 8))
    o, _ = sparse_attention(q, ks, np.ones((1, 5, 2, 8)), kl, np.ones((1, 9, 2, 8)))
    np.testing.assert_allclose(o, 1.0, atol=1e-14)


def test_zero_query_pins_causal_count():
    # q = 0: every visible key has weight 1/n_t, so lse = log n_t with
    # n_t = M + L_loc - T + t + 1, and o is the mean of the visible values.
    rng = np.random.default_rng(2)
    b_, t_, l_len, m = 1, 4, 7, 3
    ks = rng.standard_normal((b_, m, 1, 2))
    kl = rng.standard_normal((b_, l_len, 1, 2))
    vs = rng.standard_normal((b_, m, 1, 2))
    vl = rng.standard_normal((b_, l_len, 1, 2))
    o, lse = sparse_attention(np.zeros((b_, t_, 1, 2)), ks, vs, kl, vl)
    for t in range(t_):
        n_t = m + l_len - t_ + t + 1
        assert lse[0, 0, t] == pytest.approx(math.log(n_t), abs=1e-14)
        vis = np.concatenate([vs[0, :, 0], vl[0, : l_len - t_ + t + 1, 0]])
        np.testing.assert_allclose(o[0, t, 0], vis.mean(axis=0), atol=1e-14)


def test_one_hot_values_read_off_probabilities():
    # Tiny workload shapes: M + L_loc = 32 + 32 = 64 = d, so V = identity
    # rows return each row's softmax weights (SciPy softmax of the logits).
    cfg = mi.TINY
    rng = np.random.default_rng(3)
    m, l_len, t_, d = cfg.mem_len, cfg.loc_len, cfg.q_len, cfg.dim
    q = rng.standard_normal((1, t_, 2, d))
    ks = rng.standard_normal((1, m, 1, d))
    kl = rng.standard_normal((1, l_len, 1, d))
    eye = np.eye(m + l_len)
    o, _ = sparse_attention(q, ks, eye[None, :m, None, :], kl, eye[None, m:, None, :])
    keys = np.concatenate([ks[0, :, 0], kl[0, :, 0]])
    for h in range(2):
        for t in range(t_):
            n_t = m + l_len - t_ + t + 1
            p = softmax(keys[:n_t] @ q[0, t, h] / math.sqrt(d))
            np.testing.assert_allclose(o[0, t, h, :n_t], p, atol=1e-14)
            np.testing.assert_array_equal(o[0, t, h, n_t:], 0.0)


def test_gqa_head_map():
    # KV head g carries the constant value g: query head h must return h // (H_q / H_kv).
    rng = np.random.default_rng(4)
    hq, hkv = 8, 2
    q = rng.standard_normal((1, 3, hq, 4))
    ks = rng.standard_normal((1, 2, hkv, 4))
    kl = rng.standard_normal((1, 3, hkv, 4))
    val = np.broadcast_to(np.arange(hkv, dtype=np.float64)[None, None, :, None], (1, 2, hkv, 4)).copy()
    vall = np.broadcast_to(np.arange(hkv, dtype=np.float64)[None, None, :, None], (1, 3, hkv, 4)).copy()
    o, _ = sparse_attention(q, ks, val, kl, vall)
    for h in range(hq):
        np.testing.assert_allclose(o[0, :, h], h // (hq // hkv), atol=1e-14)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, 1, 1, 6))
    o, lse = sparse_attention(rng.standard_normal((1, 1, 1, 6)), np.zeros((1, 0, 1, 6)), np.zeros((1, 0, 1, 6)),
                              rng.standard_normal((1, 1, 1, 6)), v)
    np.testing.assert_array_equal(o, v)


def test_all_documents_selected_equals_dense_sdpa():
    # With k = N_doc the sparse context is the whole pooled memory; the result
    # must equal dense attention over [all pooled K/V ; local causal] computed by
    # torch.nn.functional.scaled_dot_product_attention in float64 on the CPU.
    cfg = mi.TINY
    t = mi.draw_tiny(11)
    x = {k: v.double().numpy() for k, v in t.items() if k in ("k", "v", "k_r", "q", "k_loc", "v_loc")}
    kbar = pool_chunks_stored(x["k"], cfg.chunk, "f32")
    vbar = pool_chunks_stored(x["v"], cfg.chunk, "f32")
    kbar_r = pool_chunks_stored(x["k_r"], cfg.chunk, "f32")
    q_r = mi.plant_router_queries(torch.from_numpy(kbar_r).float(), t["planted"], t["q_r_noise"], cfg).double().numpy()
    scores = route_scores(q_r, kbar_r, cfg.chunks_per_doc)
    ids, _ = topk_docs(scores, cfg.n_doc)
    ks, vs = gather_kv(kbar, vbar, ids, cfg.chunks_per_doc)
    o, _ = sparse_attention(x["q"], ks, vs, x["k_loc"], x["v_loc"])

    # dense reference in document order (attention is invariant to key order)
    m = kbar.shape[0]
    g = cfg.heads_q // cfg.heads_kv
    keys = torch.from_numpy(np.concatenate([kbar[None], x["k_loc"]], axis=1))       # [1, m+L, Hkv, d]
    vals = torch.from_numpy(np.concatenate([vbar[None], x["v_loc"]], axis=1))
    keys = keys.repeat_interleave(g, dim=2).permute(0, 2, 1, 3).contiguous()          # [1, Hq, m+L, d]
    vals = vals.repeat_interleave(g, dim=2).permute(0, 2, 1, 3).contiguous()
    qq = torch.from_numpy(x["q"]).permute(0, 2, 1, 3).contiguous()
    t_len, l_len = cfg.q_len, cfg.loc_len
    mask = torch.zeros((t_len, m + l_len), dtype=torch.bool)
    for tt in range(t_len):
        mask[tt, : m + l_len - t_len + tt + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, attn_mask=mask)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# merge of two partial attentions over disjoint key sets
# ---------------------------------------------------------------------------

def _memory_only(q, ks, vs, scale):
    """Attention of every query row over the memory rows alone (brute force per row)."""
    b_, t_, hq, _ = q.shape
    g = hq // ks.shape[2]
    o = np.zeros_like(q)
    lse = np.zeros((b_, hq, t_))
    for b in range(b_):
        for h in range(hq):
            for t in range(t_):
                o[b, t, h], lse[b, h, t] = sparse_attention_rows(q[b, t, h], ks[b, :, h // g], vs[b, :, h // g], scale)
    return o, lse


@pytest.mark.parametrize("t_len,l_len", [(3, 5), (1, 4)])
def test_merge_of_disjoint_parts_equals_attention_over_their_union(t_len, l_len):
    # memory rows and visible local rows are disjoint key sets; merging the
    # attention over each must give the attention over all of them
    rng = np.random.default_rng(40 + t_len)
    q = rng.standard_normal((2, t_len, 4, 8))
    ks, vs = rng.standard_normal((2, 5, 2, 8)), rng.standard_normal((2, 5, 2, 8))
    kl, vl = rng.standard_normal((2, l_len, 2, 8)), rng.standard_normal((2, l_len, 2, 8))
    o, lse = sparse_attention(q, ks, vs, kl, vl, scale=0.6)
    empty = np.zeros((2, 0, 2, 8))
    o_loc, lse_loc = sparse_attention(q, empty, empty, kl, vl, scale=0.6)
    o_mem, lse_mem = _memory_only(q, ks, vs, 0.6)
    mo, mlse = merge_attention(o_loc, lse_loc, o_mem, lse_mem)
    np.testing.assert_allclose(mo, o, atol=1e-13)
    np.testing.assert_allclose(mlse, lse, atol=1e-13)
    # the merge is symmetric in its two parts
    mo2, mlse2 = merge_attention(o_mem, lse_mem, o_loc, lse_loc)
    np.testing.assert_allclose(mo2, o, atol=1e-13)
    np.testing.assert_allclose(mlse2, lse, atol=1e-13)


def test_merge_decode_memory_rows_passed_as_local_rows():
    # one query token sees every local row, so the memory rows' attention is
    # the attention over them passed as local rows of a call without memory
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 1, 4, 8))
    ks, vs = rng.standard_normal((3, 6, 2, 8)), rng.standard_normal((3, 6, 2, 8))
    kl, vl = rng.standard_normal((3, 9, 2, 8)), rng.standard_normal((3, 9, 2, 8))
    empty = np.zeros((3, 0, 2, 8))
    o, lse = sparse_attention(q, ks, vs, kl, vl)
    o_loc, lse_loc = sparse_attention(q, empty, empty, kl, vl)
    o_mem, lse_mem = sparse_attention(q, empty, empty, ks, vs)
    mo, mlse = merge_attention(o_loc, lse_loc, o_mem, lse_mem)
    np.testing.assert_allclose(mo, o, atol=1e-13)
    np.testing.assert_allclose(mlse, lse, atol=1e-13)


def test_merge_closed_forms():
    rng = np.random.default_rng(3)
    o_a, o_b = rng.standard_normal((2, 3, 4, 8)), rng.standard_normal((2, 3, 4, 8))
    lse_a = rng.standard_normal((2, 4, 3))
    # equal normalisers: the mean of the two outputs, log-sum-exp up by log 2
    mo, mlse = merge_attention(o_a, lse_a, o_b, lse_a)
    np.testing.assert_allclose(mo, (o_a + o_b) / 2, atol=1e-14)
    np.testing.assert_allclose(mlse, lse_a + math.log(2.0), atol=1e-14)
    # an empty part (lse = -inf) contributes nothing
    none = np.full((2, 4, 3), -np.inf)
    mo, mlse = merge_attention(o_a, lse_a, o_b, none)
    np.testing.assert_array_equal(mo, o_a)
    np.testing.assert_array_equal(mlse, lse_a)
    # both empty: zero output, -inf
    mo, mlse = merge_attention(o_a, none, o_b, none)
    np.testing.assert_array_equal(mo, np.zeros_like(o_a))
    assert np.all(np.isneginf(mlse))
    # one (b, h, t) weighted by hand: lse_a = log 1, lse_b = log 3 -> weights 1/4, 3/4
    la, lb = np.zeros((1, 1, 1)), np.full((1, 1, 1), math.log(3.0))
    xa, xb = np.array([[[[4.0, 0.0]]]]), np.array([[[[0.0, 8.0]]]])
    mo, mlse = merge_attention(xa, la, xb, lb)
    np.testing.assert_allclose(mo, [[[[1.0, 6.0]]]], atol=1e-15)
    np.testing.assert_allclose(mlse, [[[math.log(4.0)]]], atol=1e-15)
