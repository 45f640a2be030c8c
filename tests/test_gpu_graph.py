"""A routed decode step captured in a HIP graph: every replay reproduces the
eager step bit for bit (the kernels are deterministic), with eager work and
synchronisations between the replays, and a replay after the inputs change
matches an eager step on the new inputs."""

import math

import pytest
import torch

import routed_sparse_attention_msa_amd as msa

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    n_docs, cpd, heads_kv, heads_q, dim, batch, loc = 256, 8, 4, 16, 128, 8, 700
    r = lambda *s: (torch.randn(s, generator=g, device=DEV) / math.sqrt(dim)).to(torch.bfloat16)
    raw_k, raw_v, raw_r = r(n_docs, cpd * 64, heads_kv, dim), r(n_docs, cpd * 64, heads_kv, dim), r(n_docs, cpd * 64, heads_kv, dim)
    kbar, _ = msa.msa_pool_chunks(raw_k, 64)
    vbar, _ = msa.msa_pool_chunks(raw_v, 64)
    kbar_r, knorm = msa.msa_pool_chunks(raw_r, 64, with_norm=True)
    return dict(kbar=kbar, vbar=vbar, kbar_r=kbar_r, knorm=knorm, cpd=cpd, topk=8,
                q_r=r(batch, 1, heads_kv, dim), q=r(batch, 1, heads_q, dim) * 4,
                k_loc=r(batch, loc, heads_kv, dim), v_loc=r(batch, loc, heads_kv, dim))


class _Step:
    def __init__(self, t):
        self.t = t
        b = t["q"].shape[0]
        e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=DEV)
        self.scores = e(b, t["kbar"].shape[0] // t["cpd"], dt=torch.float32)
        self.ids = e(b, t["topk"], dt=torch.int32)
        self.top = e(b, t["topk"], dt=torch.float32)
        self.k_sel = e(b, t["topk"] * t["cpd"], t["kbar"].shape[1], t["kbar"].shape[2])
        self.v_sel = torch.empty_like(self.k_sel)
        self.out = torch.empty_like(t["q"])
        self.lse = e(b, t["q"].shape[2], 1, dt=torch.float32)

    def __call__(self):
        t = self.t
        msa.msa_route_scores(t["q_r"], t["kbar_r"], t["knorm"], t["cpd"], doc_scores=self.scores)
        msa.msa_topk_docs(self.scores, t["topk"], topk_ids=self.ids, topk_scores=self.top)
        msa.msa_gather_kv(t["kbar"], t["vbar"], self.ids, t["cpd"], k_sel=self.k_sel, v_sel=self.v_sel)
        msa.msa_sparse_attn(t["q"], self.k_sel, self.v_sel, t["k_loc"], t["v_loc"], out=self.out, lse=self.lse)

    def results(self):
        return [x.clone() for x in (self.scores, self.ids, self.top, self.out, self.lse)]


def test_graph_replays_match_eager_steps():
    t = _inputs(5)
    step = _Step(t)
    step()
    torch.cuda.synchronize()
    want = step.results()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = _Step(_inputs(6))
    for rep in range(4):
        for x in (step.scores, step.out, step.lse):           # clobber the outputs with a fill kernel
            x.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = step.results()
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        other()                                              # eager work between replays
        torch.cuda.synchronize()
    # new inputs in place: a replay equals an eager step on them
    t["q_r"].copy_(_inputs(7)["q_r"])
    t["q"].mul_(0.5)
    g.replay()
    torch.cuda.synchronize()
    got = step.results()
    step()
    torch.cuda.synchronize()
    for a, b in zip(got, step.results()):
        assert torch.equal(a, b)


class _OverlapStep(_Step):
    """The same step with the attention in two parts, as the decode bench runs
    it: the local rows' attention forked onto a second stream at the start,
    the memory rows' attention after the gather, a log-sum-exp merge after the
    join."""

    def __init__(self, t):
        super().__init__(t)
        self.aux = torch.cuda.Stream()
        self.o_loc, self.o_mem = torch.empty_like(self.out), torch.empty_like(self.out)
        self.l_loc, self.l_mem = torch.empty_like(self.lse), torch.empty_like(self.lse)

    def __call__(self):
        t = self.t
        cur = torch.cuda.current_stream()
        self.aux.wait_stream(cur)
        with torch.cuda.stream(self.aux):
            msa.msa_sparse_attn(t["q"], None, None, t["k_loc"], t["v_loc"], out=self.o_loc, lse=self.l_loc)
        msa.msa_route_scores(t["q_r"], t["kbar_r"], t["knorm"], t["cpd"], doc_scores=self.scores)
        msa.msa_topk_docs(self.scores, t["topk"], topk_ids=self.ids, topk_scores=self.top)
        msa.msa_gather_kv(t["kbar"], t["vbar"], self.ids, t["cpd"], k_sel=self.k_sel, v_sel=self.v_sel)
        msa.msa_sparse_attn(t["q"], None, None, self.k_sel, self.v_sel, out=self.o_mem, lse=self.l_mem)
        cur.wait_stream(self.aux)
        msa.msa_attn_merge(self.o_loc, self.l_loc, self.o_mem, self.l_mem, out=self.out, lse=self.lse)


def test_two_stream_graph_replays_match_eager_steps():
    t = _inputs(8)
    step = _OverlapStep(t)
    step()
    torch.cuda.synchronize()
    want = step.results()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = _OverlapStep(_inputs(9))
    for rep in range(4):
        for x in (step.scores, step.out, step.lse, step.o_loc, step.o_mem):
            x.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(step.results(), want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        other()
        torch.cuda.synchronize()
    # the overlapped step agrees with the one-call attention to the bf16 tolerance
    plain = _Step(t)
    plain()
    torch.cuda.synchronize()
    rel = ((step.out.float() - plain.out.float()).norm(dim=-1) / plain.out.float().norm(dim=-1)).max().item()
    assert rel <= 2e-2, rel
    assert (step.lse - plain.lse).abs().max().item() <= 2e-3
