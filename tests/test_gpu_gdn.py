"""GPU parity of the linear-layer variant (state injection and the gated delta
rule from that initial state) against the oracle."""

import math

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from oracle import gated_delta_rule, inject_states
from tests.parity import bf16_ulp_distance, case, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _seq(batch, t_len, heads, dk, dv, dtype, seed, g_lo=-0.5, with_init=True):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    rn = lambda *s: torch.randn(s, generator=gen, device=DEV)
    q = (rn(batch, t_len, heads, dk) / math.sqrt(dk)).to(dtype)
    k = rn(batch, t_len, heads, dk)
    k = (k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)).to(dtype)
    v = rn(batch, t_len, heads, dv).to(dtype)
    g = (torch.rand((batch, t_len, heads), generator=gen, device=DEV) * g_lo).contiguous()
    beta = torch.rand((batch, t_len, heads), generator=gen, device=DEV).contiguous()
    h0 = rn(batch, heads, dk, dv) * 0.1 if with_init else None
    return q, k, v, g, beta, h0


def _check(out, fs, ro, rh, dtype):
    fs64 = to_f64(fs)
    herr = np.abs(fs64 - rh).max() / max(np.abs(rh).max(), 1e-30)
    print(f"  final state: max err / max |h| {herr:.2e}")
    assert herr <= 1e-4
    if out is None:
        return
    o64 = to_f64(out)
    oerr = np.abs(o64 - ro).max() / max(np.abs(ro).max(), 1e-30)
    if dtype == torch.bfloat16:
        # one rounding to bf16 of a float32 result within 1e-4 of the scale
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ro), 1e-30))) - 7)
        assert np.all(np.abs(o64 - ro) <= ulp + 1e-4 * np.abs(ro).max())
        print(f"  out: max ulp {bf16_ulp_distance(out, ro).max()}, max err / max |o| {oerr:.2e}")
    else:
        print(f"  out: max err / max |o| {oerr:.2e}")
        assert oerr <= 1e-4


@pytest.mark.parametrize("batch,t_len,heads,dk,dv,dtype,g_lo", [
    (2, 37, 3, 64, 48, torch.float32, -0.5),        # ragged token chunk, one partial column slice
    (1, 100, 2, 128, 128, torch.bfloat16, -0.5),    # the layer's head size
    (3, 1, 4, 128, 200, torch.bfloat16, -0.5),      # one token (decode), several column slices
    (1, 70, 2, 64, 64, torch.float32, -60.0),       # strong decay: the lazy scale renormalises
    (1, 40, 1, 128, 64, torch.float32, -300.0),     # decays that underflow float32 (state to zero)
])
def test_gated_delta_rule_parity(batch, t_len, heads, dk, dv, dtype, g_lo):
    case(f"gated delta rule B={batch} T={t_len} H={heads} dk={dk} dv={dv} {dtype} g>={g_lo}")
    q, k, v, g, beta, h0 = _seq(batch, t_len, heads, dk, dv, dtype, seed=t_len + dv, g_lo=g_lo)
    out, fs = msa.msa_gated_delta_rule(q, k, v, g, beta, initial_state=h0)
    torch.cuda.synchronize()
    ro, rh = gated_delta_rule(to_f64(q), to_f64(k), to_f64(v), to_f64(g), to_f64(beta),
                              initial_state=to_f64(h0))
    _check(out, fs, ro, rh, dtype)


def test_document_encoding_final_states_only():
    """Outputs skipped (q absent): the final states equal those of the full run."""
    case("gated delta rule, final states only")
    q, k, v, g, beta, _ = _seq(6, 65, 2, 128, 128, torch.bfloat16, seed=3, with_init=False)
    _, fs = msa.msa_gated_delta_rule(None, k, v, g, beta, with_out=False)
    out, fs_full = msa.msa_gated_delta_rule(q, k, v, g, beta)
    torch.cuda.synchronize()
    assert torch.equal(fs, fs_full)
    _, rh = gated_delta_rule(to_f64(q), to_f64(k), to_f64(v), to_f64(g), to_f64(beta))
    _check(None, fs, None, rh, torch.bfloat16)


def test_split_sequence_carries_the_state():
    case("gated delta rule, split sequence")
    q, k, v, g, beta, h0 = _seq(2, 90, 2, 128, 128, torch.float32, seed=4)
    out, fs = msa.msa_gated_delta_rule(q, k, v, g, beta, initial_state=h0)
    o1, f1 = msa.msa_gated_delta_rule(q[:, :41].contiguous(), k[:, :41].contiguous(), v[:, :41].contiguous(),
                                      g[:, :41].contiguous(), beta[:, :41].contiguous(), initial_state=h0)
    o2, f2 = msa.msa_gated_delta_rule(q[:, 41:].contiguous(), k[:, 41:].contiguous(), v[:, 41:].contiguous(),
                                      g[:, 41:].contiguous(), beta[:, 41:].contiguous(), initial_state=f1)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_f64(torch.cat([o1, o2], dim=1)), to_f64(out), rtol=0, atol=1e-5 * float(out.abs().max()))
    np.testing.assert_allclose(to_f64(f2), to_f64(fs), rtol=0, atol=1e-5 * float(fs.abs().max()))


@pytest.mark.parametrize("batch,t_len,heads,g_lo,with_init", [
    (2, 100, 3, -0.5, True),     # three chunks and a ragged fourth
    (1, 300, 2, -0.1, True),     # ten chunks: crosses a group of eight
    (3, 1, 2, -0.5, True),       # one token
    (1, 64, 1, -0.5, False),     # whole chunks, no initial state
    (2, 37, 2, -0.5, False),
    (1, 70, 2, -60.0, True),     # strong decay inside a chunk
    (1, 40, 1, -300.0, True),    # decays that underflow float32 (state to zero)
    (1, 513, 1, -0.05, True),    # two full groups and one token of a third
])
def test_gated_delta_rule_chunked_parity(batch, t_len, heads, g_lo, with_init):
    """The chunked form against the oracle's token-by-token rule, outputs and final states."""
    case(f"chunked gated delta rule B={batch} T={t_len} H={heads} g>={g_lo} init={with_init}")
    q, k, v, g, beta, h0 = _seq(batch, t_len, heads, 128, 128, torch.bfloat16, seed=t_len + 7 * heads, g_lo=g_lo,
                                with_init=with_init)
    out, fs = msa.msa_gated_delta_rule_chunked(q, k, v, g, beta, initial_state=h0)
    torch.cuda.synchronize()
    ro, rh = gated_delta_rule(to_f64(q), to_f64(k), to_f64(v), to_f64(g), to_f64(beta),
                              initial_state=None if h0 is None else to_f64(h0))
    _check(out, fs, ro, rh, torch.bfloat16)


def test_gated_delta_rule_chunked_empty_and_states_only():
    """T = 0 returns the initial state; final states without outputs equal those with outputs."""
    case("chunked gated delta rule: empty sequence, states only")
    q, k, v, g, beta, h0 = _seq(2, 0, 2, 128, 128, torch.bfloat16, seed=5)
    _, fs = msa.msa_gated_delta_rule_chunked(None, k, v, g, beta, initial_state=h0, with_out=False)
    torch.cuda.synchronize()
    assert torch.equal(fs, h0)
    q, k, v, g, beta, h0 = _seq(3, 200, 2, 128, 128, torch.bfloat16, seed=6)
    _, fs = msa.msa_gated_delta_rule_chunked(None, k, v, g, beta, initial_state=h0, with_out=False)
    _, fs_full = msa.msa_gated_delta_rule_chunked(q, k, v, g, beta, initial_state=h0)
    torch.cuda.synchronize()
    assert (fs - fs_full).abs().max().item() <= 1e-6 * fs_full.abs().max().item()


def test_document_states_chunked_full_bank():
    """The offline encoding of the 1M-token bank's 2048 document states (512 tokens, 8 heads) in the
    chunked form: sampled documents against the oracle, and every state against the token-by-token
    kernel."""
    case("chunked gated delta rule: 2048 documents x 512 tokens x 8 heads, states only")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    n_doc, t_len, heads, d = 2048, 512, 8, 128
    k = torch.randn((n_doc, t_len, heads, d), generator=gen, device=DEV)
    k = (k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)).to(torch.bfloat16)
    v = torch.randn((n_doc, t_len, heads, d), generator=gen, device=DEV).to(torch.bfloat16)
    g = (torch.rand((n_doc, t_len, heads), generator=gen, device=DEV) * -0.5).contiguous()
    beta = torch.rand((n_doc, t_len, heads), generator=gen, device=DEV).contiguous()
    _, fs = msa.msa_gated_delta_rule_chunked(None, k, v, g, beta, with_out=False)
    _, fr = msa.msa_gated_delta_rule(None, k, v, g, beta, with_out=False)
    torch.cuda.synchronize()
    rel = ((fs - fr).abs().amax(dim=(1, 2, 3)) / fr.abs().amax(dim=(1, 2, 3))).max().item()
    print(f"  chunked vs token-by-token over all 2048 x 8 states: max err / max |h| {rel:.2e}")
    assert rel <= 2e-4
    for doc in (0, 777, n_doc - 1):
        sl = slice(doc, doc + 1)
        _, rh = gated_delta_rule(to_f64(k[sl]), to_f64(k[sl]), to_f64(v[sl]), to_f64(g[sl]), to_f64(beta[sl]))
        _check(None, fs[sl], None, rh, torch.bfloat16)


@pytest.mark.parametrize("n_docs,batch,k,heads,dk,dv", [
    (50, 3, 5, 2, 64, 64),
    (2048, 32, 16, 8, 128, 128),     # the 1M-token bank's states, a decode batch
])
def test_state_sum(n_docs, batch, k, heads, dk, dv):
    case(f"state sum N={n_docs} B={batch} k={k} H={heads}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(n_docs)
    states = torch.randn((n_docs, heads, dk, dv), generator=gen, device=DEV)
    ids = torch.stack([torch.randperm(n_docs, generator=gen, device=DEV)[:k] for _ in range(batch)]).to(torch.int32)
    ids[0, -1] = -1                                       # out-of-range entries contribute nothing
    s = msa.msa_gdn_state_sum(states, ids)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    rows = range(batch) if batch <= 4 else [0, 7, batch - 1]
    for b in rows:
        keep = ids_h[b][ids_h[b] >= 0]
        want = inject_states(to_f64(states[torch.as_tensor(keep, device=DEV)]), np.arange(len(keep))[None])[0]
        err = np.abs(to_f64(s[b]) - want).max()
        assert err <= k * 2.0 ** -22 * np.abs(want).max() + 1e-6


def test_linear_layer_chain():
    """Route -> top-k -> state sum -> gated delta rule, stage by stage: the
    oracle's state sum of the GPU's picks, then its rule from that state."""
    case("linear layer chain")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    n_docs, cpd, heads, dk = 300, 8, 4, 128
    raw = (torch.randn((n_docs, cpd * 64, heads, dk), generator=gen, device=DEV) / math.sqrt(dk)).to(torch.bfloat16)
    kbar_r, knorm = msa.msa_pool_chunks(raw, 64, with_norm=True)
    states = torch.randn((n_docs, heads, dk, dk), generator=gen, device=DEV) * 0.05
    q_r = kbar_r[torch.arange(16, device=DEV)].unsqueeze(0).contiguous()          # doc 0..1's chunks
    scores = msa.msa_route_scores(q_r, kbar_r, knorm, cpd)
    ids, _ = msa.msa_topk_docs(scores, 8)
    s_ext = msa.msa_gdn_state_sum(states, ids)
    q, k, v, g, beta, _ = _seq(1, 48, heads, dk, dk, torch.bfloat16, seed=22, with_init=False)
    out, fs = msa.msa_gated_delta_rule(q, k, v, g, beta, initial_state=s_ext)
    torch.cuda.synchronize()
    assert set(ids[0].tolist()) >= {0, 1}
    s_ref = inject_states(to_f64(states), ids.cpu().numpy())
    assert np.abs(to_f64(s_ext) - s_ref).max() <= 8 * 2.0 ** -22 * np.abs(s_ref).max()
    ro, rh = gated_delta_rule(to_f64(q), to_f64(k), to_f64(v), to_f64(g), to_f64(beta), initial_state=s_ref)
    _check(out, fs, ro, rh, torch.bfloat16)
