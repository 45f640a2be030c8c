"""End-to-end parity of the whole routed layer (pool -> route -> top-k -> gather
-> attention) on the tiny fp32 workload and a scaled-down bf16 prefill, plus
sampled parity at the full 1M-token prefill size.

Each oracle stage consumes exactly the tensors the GPU stage consumed (the
GPU-stored bank, the GPU-chosen ids), so a legitimate tie inside the top-k
band cannot cascade into later stages."""

import math

import numpy as np
import pytest
import torch

import msa_inputs as mi
import routed_sparse_attention_msa_amd as msa
from oracle import (chunk_norms, gather_kv, pool_chunks_mean, route_scores, sparse_attention,
                    sparse_attention_rows)
from tests.parity import (ATTN_RTOL_BF16, ATTN_RTOL_F32, ROUTE_ATOL, bf16_ulp_distance, case,
                          row_rel_l2, to_f64, topk_band_check)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_layer(cfg, t):
    """The GPU path for one routed layer; returns every intermediate."""
    kbar, _ = msa.msa_pool_chunks(t["k"], cfg.chunk)
    vbar, _ = msa.msa_pool_chunks(t["v"], cfg.chunk)
    kbar_r, knorm = msa.msa_pool_chunks(t["k_r"], cfg.chunk, with_norm=True)
    if "q_r" not in t:
        t["q_r"] = mi.plant_router_queries(kbar_r, t["planted"], t["q_r_noise"], cfg)
    scores = msa.msa_route_scores(t["q_r"], kbar_r, knorm, cfg.chunks_per_doc)
    ids, top = msa.msa_topk_docs(scores, cfg.topk)
    k_sel, v_sel = msa.msa_gather_kv(kbar, vbar, ids, cfg.chunks_per_doc)
    out, lse = msa.msa_sparse_attn(t["q"], k_sel, v_sel, t["k_loc"], t["v_loc"])
    torch.cuda.synchronize()
    return dict(kbar=kbar, vbar=vbar, kbar_r=kbar_r, knorm=knorm, scores=scores, ids=ids, top=top,
                k_sel=k_sel, v_sel=v_sel, out=out, lse=lse)


def _stagewise(cfg, t, r, rtol):
    cpd = cfg.chunks_per_doc
    # S1
    for name, raw in (("kbar", "k"), ("vbar", "v"), ("kbar_r", "k_r")):
        exact = pool_chunks_mean(to_f64(t[raw]), cfg.chunk)
        if cfg.dtype == "bf16":
            assert bf16_ulp_distance(r[name], exact).max() <= 1, name
        else:
            assert np.abs(to_f64(r[name]) - exact).max() <= 64 * 2.0 ** -24 * np.abs(to_f64(t[raw])).max()
    np.testing.assert_allclose(to_f64(r["knorm"]), chunk_norms(to_f64(r["kbar_r"])), rtol=2e-6)
    # S2 on the GPU-stored bank
    ref_scores = route_scores(to_f64(t["q_r"]), to_f64(r["kbar_r"]), cpd)
    assert np.abs(to_f64(r["scores"]) - ref_scores).max() <= ROUTE_ATOL
    # S3 on the oracle's own scores, by the band rule
    ok, exact = topk_band_check(r["ids"].cpu().numpy(), ref_scores, cfg.topk)
    assert ok
    # S4 on the GPU-chosen ids: bit-exact
    ids = r["ids"].cpu().numpy().astype(np.int64)
    rk, rv = gather_kv(to_f64(r["kbar"]), to_f64(r["vbar"]), ids, cpd)
    assert np.array_equal(to_f64(r["k_sel"]), rk) and np.array_equal(to_f64(r["v_sel"]), rv)
    # S5 on the GPU-gathered memory
    ro, rlse = sparse_attention(to_f64(t["q"]), rk, rv, to_f64(t["k_loc"]), to_f64(t["v_loc"]))
    assert row_rel_l2(to_f64(r["out"]), ro).max() <= rtol
    assert np.abs(to_f64(r["lse"]) - rlse).max() <= 2e-3
    return exact


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_layer(seed):
    case(f"tiny layer seed={seed}")
    cfg = mi.TINY
    t = {k: v.to(DEV) for k, v in mi.draw_tiny(seed).items()}
    r = run_layer(cfg, t)
    assert int(r["ids"][0, 0]) == 7                  # the planted document wins
    _stagewise(cfg, t, r, ATTN_RTOL_F32)


SCALED_PREFILL = mi.scaled(mi.PREFILL, n_doc=96, q_len=256, loc_len=256, n_planted=4)
SCALED_DECODE = mi.scaled(mi.DECODE, n_doc=160, batch=4, loc_len=300)


@pytest.mark.parametrize("cfg", [SCALED_PREFILL, SCALED_DECODE], ids=lambda c: c.name)
def test_scaled_bf16_layer(cfg):
    case(f"scaled layer {cfg.name}")
    t = mi.draw_layer(cfg, seed=3, device=DEV)
    r = run_layer(cfg, t)
    if cfg.n_planted:
        planted = set(t["planted"].tolist())
        assert planted <= set(r["ids"][0].tolist())
    _stagewise(cfg, t, r, ATTN_RTOL_BF16)


def test_full_prefill_sampled():
    """The 1M-token bank with a 2048-token prefill, in the launch configuration
    the benchmark times; the oracle checks sampled outputs one by one."""
    cfg = mi.PREFILL
    case("full prefill 1M bank (sampled)")
    t = mi.draw_layer(cfg, seed=0, device=DEV)
    r = run_layer(cfg, t)
    rng = np.random.default_rng(0)
    cpd = cfg.chunks_per_doc
    # S1: sampled chunks of each tensor, against the oracle on those chunks' raw rows
    docs = rng.choice(cfg.n_doc, 6, replace=False)
    for name, raw in (("kbar", "k"), ("vbar", "v"), ("kbar_r", "k_r")):
        exact = pool_chunks_mean(to_f64(t[raw][torch.as_tensor(docs, device=DEV)]), cfg.chunk)
        rows = torch.as_tensor((docs[:, None] * cpd + np.arange(cpd)).ravel(), device=DEV)
        assert bf16_ulp_distance(r[name][rows], exact).max() <= 1, name
    # S2: sampled documents (each doc's score depends only on its own chunks)
    sample = np.concatenate([rng.choice(cfg.n_doc, 48, replace=False), t["planted"].cpu().numpy()])
    rows = torch.as_tensor((sample[:, None] * cpd + np.arange(cpd)).ravel(), device=DEV)
    ref = route_scores(to_f64(t["q_r"]), to_f64(r["kbar_r"][rows]), cpd)
    got = to_f64(r["scores"])[:, sample]
    assert np.abs(got - ref).max() <= ROUTE_ATOL
    # S3: all 16 planted docs are selected (the plant margin is far above the band)
    assert set(t["planted"].tolist()) == set(r["ids"][0].tolist())
    # S4: bit-exact
    ids = r["ids"].cpu().numpy().astype(np.int64)
    sel_rows = torch.as_tensor((ids[0][:, None] * cpd + np.arange(cpd)).ravel(), device=DEV)
    assert torch.equal(r["k_sel"][0], r["kbar"][sel_rows]) and torch.equal(r["v_sel"][0], r["vbar"][sel_rows])
    # S5: sampled (token, head) rows, including the first and the last token
    ks = to_f64(r["k_sel"][0])
    vs = to_f64(r["v_sel"][0])
    kl = to_f64(t["k_loc"][0])
    vl = to_f64(t["v_loc"][0])
    q = to_f64(t["q"][0])
    out = to_f64(r["out"][0])
    lse = to_f64(r["lse"][0])
    g = cfg.heads_q // cfg.heads_kv
    pairs = [(0, 0), (cfg.q_len - 1, cfg.heads_q - 1)] + [
        (int(a), int(b)) for a, b in zip(rng.integers(0, cfg.q_len, 30), rng.integers(0, cfg.heads_q, 30))]
    for tt, h in pairs:
        n_loc = cfg.loc_len - cfg.q_len + tt + 1
        keys = np.concatenate([ks[:, h // g], kl[:n_loc, h // g]])
        vals = np.concatenate([vs[:, h // g], vl[:n_loc, h // g]])
        o, l_ = sparse_attention_rows(q[tt, h], keys, vals, 1.0 / math.sqrt(cfg.dim))
        assert row_rel_l2(out[tt, h], o) <= ATTN_RTOL_BF16
        assert abs(lse[h, tt] - l_) <= 2e-3
