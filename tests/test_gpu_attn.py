"""GPU parity of S5/S6 (sparse GQA attention, prefill and decode) against the oracle."""

import math

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from oracle import sparse_attention
from tests.parity import ATTN_RTOL_BF16, ATTN_RTOL_F32, case, row_rel_l2, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _attn_inputs(batch, q_len, hq, hkv, dim, mem, loc, dtype, seed, scale_v=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    s = 1.0 / math.sqrt(dim) if dtype == torch.bfloat16 else 1.0

    def r(*shape):
        return (torch.randn(shape, generator=g, device=DEV) * s).to(dtype)

    q = r(batch, q_len, hq, dim) * 4          # sharper softmax than N(0, 1/d) alone
    ks = r(batch, mem, hkv, dim) if mem else None
    vs = r(batch, mem, hkv, dim) if mem else None
    kl = r(batch, loc, hkv, dim)
    vl = r(batch, loc, hkv, dim)
    return q.to(dtype), ks, vs, kl, vl


def _check(q, ks, vs, kl, vl, rtol, lse_atol):
    out, lse = msa.msa_sparse_attn(q, ks, vs, kl, vl)
    torch.cuda.synchronize()
    dim = q.shape[-1]
    empty = np.zeros((q.shape[0], 0, kl.shape[2], dim))
    ro, rlse = sparse_attention(to_f64(q), to_f64(ks) if ks is not None else empty,
                                to_f64(vs) if vs is not None else empty, to_f64(kl), to_f64(vl),
                                scale=1.0 / math.sqrt(dim))
    rel = row_rel_l2(to_f64(out), ro)
    lerr = np.abs(to_f64(lse) - rlse)
    print(f"  max row rel-L2 {rel.max():.3e}, max |lse err| {lerr.max():.3e}")
    assert rel.max() <= rtol
    assert lerr.max() <= lse_atol
    return out, lse


@pytest.mark.parametrize("batch,q_len,hq,hkv,dim,mem,loc,dtype", [
    (1, 32, 4, 2, 64, 32, 32, torch.float32),          # tiny workload shapes
    (1, 256, 8, 2, 128, 128, 256, torch.bfloat16),     # prefill, T = L_loc
    (1, 100, 8, 2, 128, 40, 300, torch.bfloat16),      # T < L_loc, ragged tiles
    (2, 64, 4, 1, 128, 0, 64, torch.bfloat16),         # no memory rows
    (1, 37, 4, 4, 128, 24, 37, torch.bfloat16),        # group size 1, odd T
    (4, 1, 8, 2, 128, 128, 700, torch.bfloat16),       # decode
    (3, 1, 32, 8, 128, 256, 1000, torch.bfloat16),     # decode, 256 memory rows
    (2, 3, 8, 2, 128, 64, 129, torch.bfloat16),        # short multi-token step
    (1, 16, 2, 1, 64, 16, 20, torch.bfloat16),         # head dim 64
    (1, 9, 2, 2, 96, 5, 9, torch.float32),             # odd head dim
    (1, 64, 4, 2, 128, 32, 64, torch.bfloat16),        # group size 2
    (1, 64, 4, 1, 128, 0, 100, torch.bfloat16),        # a key half whose first tile is past the
    (1, 40, 8, 2, 128, 0, 90, torch.bfloat16),         #   first queries' causal limit (all masked)
    (32, 1, 32, 8, 128, 32, 250, torch.bfloat16),      # decode, one workgroup per (sequence, KV head)
    (40, 2, 16, 8, 128, 16, 90, torch.bfloat16),       # more pairs than CUs, 2 tokens
    (2, 1, 32, 8, 128, 40, 1000, torch.bfloat16),      # decode, memory length not a multiple of 32 (per-row loads)
    (1, 1, 8, 1, 128, 64, 5000, torch.bfloat16),       # one pair: many runs of splits, combined
    (1, 96, 8, 2, 128, 64, 160, torch.bfloat16),       # 3 token blocks: a block pair and a middle block alone
    (1, 80, 16, 2, 128, 40, 100, torch.bfloat16),      # group of 8 heads (two head sub-groups), partial tiles
    (2, 8, 32, 8, 128, 64, 300, torch.bfloat16),       # decode at its widest: 8 tokens x 4 heads = 32 columns
    (1, 9, 32, 8, 128, 32, 300, torch.bfloat16),       # one token more: the prefill kernel, one ragged block
    (4, 1, 32, 8, 128, 0, 500, torch.bfloat16),        # decode without memory rows (the local part alone)
])
def test_attn_parity(batch, q_len, hq, hkv, dim, mem, loc, dtype):
    case(f"attn B={batch} T={q_len} Hq={hq} Hkv={hkv} d={dim} M={mem} L={loc} {dtype}")
    q, ks, vs, kl, vl = _attn_inputs(batch, q_len, hq, hkv, dim, mem, loc, dtype, seed=q_len + loc + mem)
    rtol = ATTN_RTOL_BF16 if dtype == torch.bfloat16 else ATTN_RTOL_F32
    _check(q, ks, vs, kl, vl, rtol, lse_atol=2e-3 if dtype == torch.bfloat16 else 1e-5)


def test_attn_many_workgroups_sampled():
    """More workgroups than one round on the GPU (partial memory and local
    tiles too); sampled rows against the oracle one by one."""
    from oracle import sparse_attention_rows
    case("attn many workgroups (sampled)")
    b_, t_, hq, hkv, d, mem, loc = 3, 1024, 32, 8, 128, 96, 1100
    q, ks, vs, kl, vl = _attn_inputs(b_, t_, hq, hkv, d, mem, loc, torch.bfloat16, seed=9)
    out, lse = msa.msa_sparse_attn(q, ks, vs, kl, vl)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    g = hq // hkv
    fo, fl = to_f64(out), to_f64(lse)
    qq, kks, vvs, kkl, vvl = to_f64(q), to_f64(ks), to_f64(vs), to_f64(kl), to_f64(vl)
    picks = [(0, 0, 0), (b_ - 1, t_ - 1, hq - 1)] + [
        (int(rng.integers(b_)), int(rng.integers(t_)), int(rng.integers(hq))) for _ in range(60)]
    for bb, tt, h in picks:
        n_loc = loc - t_ + tt + 1
        keys = np.concatenate([kks[bb, :, h // g], kkl[bb, :n_loc, h // g]])
        vals = np.concatenate([vvs[bb, :, h // g], vvl[bb, :n_loc, h // g]])
        o, l_ = sparse_attention_rows(qq[bb, tt, h], keys, vals, 1.0 / math.sqrt(d))
        assert row_rel_l2(fo[bb, tt, h], o) <= ATTN_RTOL_BF16
        assert abs(fl[bb, h, tt] - l_) <= 2e-3


def test_attn_constant_values_give_one():
    case("attn V=1")
    q, ks, vs, kl, vl = _attn_inputs(1, 128, 8, 2, 128, 64, 128, torch.bfloat16, seed=1)
    vs = torch.ones_like(vs)
    vl = torch.ones_like(vl)
    out, _ = msa.msa_sparse_attn(q, ks, vs, kl, vl)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 1.0)


def test_attn_deterministic():
    case("attn determinism")
    q, ks, vs, kl, vl = _attn_inputs(2, 1, 32, 8, 128, 128, 1024, torch.bfloat16, seed=2)
    a, la = msa.msa_sparse_attn(q, ks, vs, kl, vl)
    b, lb = msa.msa_sparse_attn(q, ks, vs, kl, vl)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
