"""GPU parity of the sparse-attention backward against the oracle."""

import math

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from oracle import sparse_attention_backward
from tests.parity import case, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# bf16 gradients: dS is rounded to bf16 before the dQ/dK products, P before
# dV, and D comes from the stored bf16 output, each a relative 2^-9; the
# gradient tensors are compared by relative Frobenius norm, and every row
# (one key's or one query's d-vector) within the same bound of the tensor's
# RMS row norm.
BWD_RTOL_BF16 = 2e-2
BWD_RTOL_F32 = 1e-4


def _inputs(batch, q_len, hq, hkv, dim, mem, loc, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    s = 1.0 / math.sqrt(dim) if dtype == torch.bfloat16 else 1.0

    def r(*shape, scale=s):
        return (torch.randn(shape, generator=g, device=DEV) * scale).to(dtype)

    q = r(batch, q_len, hq, dim, scale=4 * s)
    ks = r(batch, mem, hkv, dim) if mem else None
    vs = r(batch, mem, hkv, dim) if mem else None
    kl = r(batch, loc, hkv, dim)
    vl = r(batch, loc, hkv, dim)
    do = r(batch, q_len, hq, dim, scale=1.0)
    return q, ks, vs, kl, vl, do


def _compare(name, got, ref, rtol):
    got = to_f64(got)
    err = got - ref
    fro = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    row_err = np.sqrt((err ** 2).sum(-1))
    rms_row = np.sqrt((ref ** 2).sum(-1).mean())
    worst = row_err.max() / max(rms_row, 1e-30)
    print(f"  {name}: rel Frobenius {fro:.2e}, worst row / RMS row {worst:.2e}")
    assert fro <= rtol and worst <= 2 * rtol


def _check(q, ks, vs, kl, vl, do, rtol):
    out, lse = msa.msa_sparse_attn(q, ks, vs, kl, vl)
    grads = msa.msa_sparse_attn_backward(q, ks, vs, kl, vl, out, lse, do)
    torch.cuda.synchronize()
    dim = q.shape[-1]
    empty = np.zeros((q.shape[0], 0, kl.shape[2], dim))
    ref = sparse_attention_backward(to_f64(q), to_f64(ks) if ks is not None else empty,
                                    to_f64(vs) if vs is not None else empty, to_f64(kl), to_f64(vl),
                                    to_f64(do), scale=1.0 / math.sqrt(dim))
    for name, g_, r_ in zip(("dq", "dk_sel", "dv_sel", "dk_loc", "dv_loc"), grads, ref):
        if r_.size == 0:
            assert g_ is None
            continue
        _compare(name, g_, r_, rtol)
    return grads


@pytest.mark.parametrize("batch,q_len,hq,hkv,dim,mem,loc,dtype", [
    (1, 32, 4, 2, 64, 32, 32, torch.float32),          # tiny workload shapes (vector-ALU kernels)
    (1, 256, 8, 2, 128, 128, 256, torch.bfloat16),     # MFMA, T = L_loc
    (1, 100, 8, 2, 128, 40, 300, torch.bfloat16),      # T < L_loc, ragged tiles of keys and queries
    (2, 64, 4, 1, 128, 0, 64, torch.bfloat16),         # no memory rows
    (1, 37, 4, 4, 128, 24, 37, torch.bfloat16),        # group size 1 (vector-ALU kernels)
    (2, 3, 8, 2, 128, 64, 129, torch.bfloat16),        # short multi-token step
    (3, 1, 32, 8, 128, 256, 1000, torch.bfloat16),     # decode-shaped
    (1, 16, 2, 1, 64, 16, 20, torch.bfloat16),         # head dim 64 (vector-ALU kernels)
    (1, 64, 4, 2, 128, 32, 64, torch.bfloat16),        # group size 2
    (1, 9, 2, 2, 96, 5, 9, torch.float32),             # odd head dim
    (1, 70, 8, 2, 128, 33, 70, torch.bfloat16),        # memory rows not a multiple of 32
    (1, 600, 8, 2, 128, 40, 700, torch.bfloat16),      # dk/dv over two parts (partials + reduce)
    (2, 520, 4, 1, 128, 64, 520, torch.bfloat16),      # two parts, two sequences
])
def test_attn_backward_parity(batch, q_len, hq, hkv, dim, mem, loc, dtype):
    case(f"attn backward B={batch} T={q_len} Hq={hq} Hkv={hkv} d={dim} M={mem} L={loc} {dtype}")
    q, ks, vs, kl, vl, do = _inputs(batch, q_len, hq, hkv, dim, mem, loc, dtype, seed=q_len + loc + mem)
    _check(q, ks, vs, kl, vl, do, BWD_RTOL_BF16 if dtype == torch.bfloat16 else BWD_RTOL_F32)


def test_attn_backward_full_layer_one_group():
    """The 1M-token prefill layer's shapes (T = L = 2048, M = 128, 32/8 heads);
    the oracle on one KV group (its 4 query heads), which is independent of
    the other groups."""
    case("attn backward full layer, one KV group checked")
    q, ks, vs, kl, vl, do = _inputs(1, 2048, 32, 8, 128, 128, 2048, torch.bfloat16, seed=11)
    out, lse = msa.msa_sparse_attn(q, ks, vs, kl, vl)
    grads = msa.msa_sparse_attn_backward(q, ks, vs, kl, vl, out, lse, do)
    again = msa.msa_sparse_attn_backward(q, ks, vs, kl, vl, out, lse, do)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert torch.equal(a, b)                     # deterministic: no atomics
    g = 5
    hs = slice(4 * g, 4 * g + 4)
    gs = slice(g, g + 1)
    ref = sparse_attention_backward(to_f64(q[:, :, hs]), to_f64(ks[:, :, gs]), to_f64(vs[:, :, gs]),
                                    to_f64(kl[:, :, gs]), to_f64(vl[:, :, gs]), to_f64(do[:, :, hs]),
                                    scale=1.0 / math.sqrt(128))
    got = (grads[0][:, :, hs], grads[1][:, :, gs], grads[2][:, :, gs], grads[3][:, :, gs], grads[4][:, :, gs])
    for name, g_, r_ in zip(("dq", "dk_sel", "dv_sel", "dk_loc", "dv_loc"), got, ref):
        _compare(name, g_, r_, BWD_RTOL_BF16)
