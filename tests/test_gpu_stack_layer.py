"""GPU parity of one layer of the 18-layer stack at full size (10M-token bank,
19,532 documents; 8192-token prefill; top-32), through the C ABI: the launch
configurations that the stack workload times, with outputs sampled against the
oracle where the whole layer is too large for it."""

import math

import numpy as np
import pytest
import torch

import msa_inputs as mi
import routed_sparse_attention_msa_amd as msa
from oracle import gather_kv, route_scores, sparse_attention_rows, topk_docs
from tests.parity import ATTN_RTOL_BF16, case, row_rel_l2, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_stack_layer_full_size_sampled():
    cfg = mi.STACK18
    case(f"stack layer full size: {cfg.n_doc} docs, T = L = {cfg.q_len}, top-{cfg.topk}")
    cpd, n_ch, hkv, hq, d = cfg.chunks_per_doc, cfg.n_chunks, cfg.heads_kv, cfg.heads_q, cfg.dim
    t = mi.draw_layer(cfg, seed=5, device=DEV, with_raw=False)
    # pooled bank drawn directly (pooling has its own parity tests): the spread
    # of a mean of 64 N(0, 1) rows
    g = torch.Generator(device=DEV)
    g.manual_seed(6)
    pooled = lambda: (torch.randn((n_ch, hkv, d), generator=g, device=DEV) / 8).to(torch.bfloat16)
    kbar, vbar, kbar_r = pooled(), pooled(), pooled()
    knorm = torch.linalg.vector_norm(kbar_r.float(), dim=-1).contiguous()

    # S2: routing, sampled documents against the oracle on their chunks
    scores = msa.msa_route_scores(t["q_r"], kbar_r, knorm, cpd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    docs = np.unique(np.concatenate([[0, cfg.n_doc - 1], rng.integers(0, cfg.n_doc, 30)]))
    rows = torch.as_tensor((docs[:, None] * cpd + np.arange(cpd)).ravel(), device=DEV)
    ref = route_scores(to_f64(t["q_r"]), to_f64(kbar_r[rows]), cpd)
    err = np.abs(to_f64(scores)[:, docs] - ref)
    print(f"  max |route err| over {docs.size} sampled docs = {err.max():.3e}")
    assert err.max() <= 2e-5

    # S3: top-32 of 19,532, exact on the same scores
    ids, top = msa.msa_topk_docs(scores, cfg.topk)
    torch.cuda.synchronize()
    ref_ids, ref_vals = topk_docs(to_f64(scores), cfg.topk)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.array_equal(to_f64(top), ref_vals)

    # S4: gather of the 32 documents (256 pooled rows), exact
    k_sel, v_sel = msa.msa_gather_kv(kbar, vbar, ids, cpd)
    torch.cuda.synchronize()
    sel = torch.as_tensor((ref_ids[0][:, None] * cpd + np.arange(cpd)).ravel(), device=DEV)
    rk, rv = gather_kv(to_f64(kbar[sel]), to_f64(vbar[sel]),
                       np.arange(cfg.topk, dtype=np.int64)[None], cpd)
    assert np.array_equal(to_f64(k_sel), rk) and np.array_equal(to_f64(v_sel), rv)

    # S5: attention, T = L = 8192 with M = 256 memory rows; sampled rows
    out, lse = msa.msa_sparse_attn(t["q"], k_sel, v_sel, t["k_loc"], t["v_loc"])
    torch.cuda.synchronize()
    grp = hq // hkv
    t_len, loc = cfg.q_len, cfg.loc_len
    fo, fl = to_f64(out), to_f64(lse)
    qq, ks, vs = to_f64(t["q"]), to_f64(k_sel), to_f64(v_sel)
    kl, vl = to_f64(t["k_loc"]), to_f64(t["v_loc"])
    picks = [(0, 0), (t_len - 1, hq - 1)] + [(int(rng.integers(t_len)), int(rng.integers(hq))) for _ in range(40)]
    worst = 0.0
    for tt, h in picks:
        n_loc = loc - t_len + tt + 1
        keys = np.concatenate([ks[0, :, h // grp], kl[0, :n_loc, h // grp]])
        vals = np.concatenate([vs[0, :, h // grp], vl[0, :n_loc, h // grp]])
        o, l_ = sparse_attention_rows(qq[0, tt, h], keys, vals, 1.0 / math.sqrt(d))
        rel = row_rel_l2(fo[0, tt, h], o)
        worst = max(worst, rel)
        assert rel <= ATTN_RTOL_BF16
        assert abs(fl[0, h, tt] - l_) <= 2e-3
    print(f"  max attention row rel-L2 over {len(picks)} sampled rows = {worst:.3e}")
