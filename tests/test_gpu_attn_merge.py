"""msa_attn_merge against the oracle's merge of two partial attentions over
disjoint key sets (the attention of the model card's "Architecture summary"
and the README's "Inference Pipeline" stage 3, split into two parts), and the
split attention it enables against the oracle's attention over all keys."""

import math

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from oracle import merge_attention, sparse_attention
from tests.parity import ATTN_RTOL_BF16, bf16_ulp_distance, case, row_rel_l2, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _parts(shape, dtype, seed, empty_frac=0.0):
    batch, q_len, heads, dim = shape
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    o_a = torch.randn(shape, generator=g, device=DEV).to(dtype)
    o_b = torch.randn(shape, generator=g, device=DEV).to(dtype)
    lse_a = 3 * torch.randn((batch, heads, q_len), generator=g, device=DEV)
    lse_b = 3 * torch.randn((batch, heads, q_len), generator=g, device=DEV)
    if empty_frac:
        # some parts hold no visible key (lse -inf), a few rows have both empty
        na = torch.rand((batch, heads, q_len), generator=g, device=DEV) < empty_frac
        nb = torch.rand((batch, heads, q_len), generator=g, device=DEV) < empty_frac
        lse_a[na] = -math.inf
        lse_b[nb] = -math.inf
        lse_a[0, 0, 0] = lse_b[0, 0, 0] = -math.inf
    return o_a, lse_a, o_b, lse_b


@pytest.mark.parametrize("shape,dtype,empty", [
    ((2, 1, 32, 128), torch.bfloat16, 0.0),
    ((3, 5, 8, 128), torch.bfloat16, 0.2),
    ((1, 7, 6, 64), torch.bfloat16, 0.3),
    ((2, 3, 4, 256), torch.bfloat16, 0.1),
    ((2, 4, 4, 128), torch.float32, 0.2),
    ((1, 2, 3, 256), torch.float32, 0.0),
    ((1, 1, 1, 8), torch.bfloat16, 0.0),
])
def test_merge_matches_oracle(shape, dtype, empty):
    case(f"attn merge: shape {shape} {dtype} empty fraction {empty}")
    o_a, lse_a, o_b, lse_b = _parts(shape, dtype, seed=sum(shape), empty_frac=empty)
    out, lse = msa.msa_attn_merge(o_a, lse_a, o_b, lse_b)
    torch.cuda.synchronize()
    ro, rlse = merge_attention(to_f64(o_a), to_f64(lse_a), to_f64(o_b), to_f64(lse_b))
    got_lse = to_f64(lse)
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.abs(got_lse[fin] - rlse[fin]).max(initial=0.0) <= 1e-5
    if dtype == torch.bfloat16:
        # float32 arithmetic, one rounding to bf16: within one unit of the rounded exact merge
        assert bf16_ulp_distance(out, ro).max() <= 1
    else:
        assert np.abs(to_f64(out) - ro).max() <= 1e-5 * max(1.0, np.abs(ro).max())
    # both parts empty: zero output
    both = np.isneginf(rlse)                               # [B, H, T]
    zero_rows = np.transpose(both, (0, 2, 1))              # [B, T, H]
    assert np.all(to_f64(out)[zero_rows] == 0.0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_merge_in_place_matches_out_of_place(dtype):
    case(f"attn merge: in place, {dtype}")
    o_a, lse_a, o_b, lse_b = _parts((4, 3, 8, 128), dtype, seed=5, empty_frac=0.1)
    ref_o, ref_l = msa.msa_attn_merge(o_a, lse_a, o_b, lse_b)
    a2, la2 = o_a.clone(), lse_a.clone()
    msa.msa_attn_merge(a2, la2, o_b, lse_b, out=a2, lse=la2)        # into the first part
    b2, lb2 = o_b.clone(), lse_b.clone()
    msa.msa_attn_merge(o_a, lse_a, b2, lb2, out=b2, lse=lb2)        # into the second part
    torch.cuda.synchronize()
    for o, l in ((a2, la2), (b2, lb2)):
        assert torch.equal(o, ref_o)
        assert torch.equal(torch.nan_to_num(l, neginf=-1e30), torch.nan_to_num(ref_l, neginf=-1e30))


@pytest.mark.parametrize("batch,q_len,mem_len,loc_len", [(3, 1, 128, 1000), (2, 1, 40, 333), (4, 1, 256, 64)])
def test_split_decode_attention_matches_oracle(batch, q_len, mem_len, loc_len):
    """Local rows alone (mem_len = 0) and the memory rows passed as the local
    rows of a second call (one query token sees them all), merged: equal to
    the attention over [memory ; local] within the bf16 attention tolerance."""
    case(f"split decode attention: B={batch} M={mem_len} L={loc_len}")
    g = torch.Generator(device=DEV)
    g.manual_seed(batch * 1000 + mem_len)
    r = lambda *s: (torch.randn(s, generator=g, device=DEV) / 3).to(torch.bfloat16)
    q = r(batch, q_len, 32, 128)
    ks, vs, kl, vl = r(batch, mem_len, 8, 128), r(batch, mem_len, 8, 128), r(batch, loc_len, 8, 128), r(batch, loc_len, 8, 128)
    o_loc, l_loc = msa.msa_sparse_attn(q, None, None, kl, vl)
    o_mem, l_mem = msa.msa_sparse_attn(q, None, None, ks, vs)
    out, lse = msa.msa_attn_merge(o_loc, l_loc, o_mem, l_mem)
    torch.cuda.synchronize()
    ro, rlse = sparse_attention(to_f64(q), to_f64(ks), to_f64(vs), to_f64(kl), to_f64(vl))
    rel = row_rel_l2(to_f64(out), ro)
    print(f"  max row rel-L2 {rel.max():.2e}, max |lse err| {np.abs(to_f64(lse) - rlse).max():.2e}")
    assert rel.max() <= ATTN_RTOL_BF16
    assert np.abs(to_f64(lse) - rlse).max() <= 2e-3
