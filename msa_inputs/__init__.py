"""Seeded synthetic inputs for the MSA routed-layer hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
only *draws* inputs: Gaussian values, rounding to the storage dtype, a
rotary position rotation of the tensors the model would have rotated, and
planting of router queries by copying rows of a pooled bank that the caller
passes in.  It holds none of the method's own arithmetic (no pooling,
routing, selection, gathering or attention), and imports neither the oracle
nor the HIP path.

Workloads (sizes from the method's single-layer, decode, large-bank and
stacked configurations):

* ``TINY``     fp32; 64 docs x 512 tokens, chunk 64; 4 query heads, 2 KV heads,
               head dim 64 = router dim; 32 query tokens with 32 local tokens;
               top-4; every tensor N(0,1); doc 7 planted.
* ``PREFILL``  bf16, Qwen3-4B-like: 32 query heads, 8 KV heads, head dim 128
               = router dim; 2048 docs x 512 tokens (a 1M-token bank, 16,384
               pooled chunks); 2048-token prefill with 2048 local tokens; top-16;
               values N(0,1)/sqrt(128); memory K rotated at doc-local positions
               0..511, query and local K at 512 + t; 16 planted docs.
* ``DECODE``   the PREFILL bank; 32 sequences x 1 new token; 4096 cached local
               tokens; top-16 (memory rows M = 16 x 8 = 128).
* ``SCAN100M`` 195,313 docs x 512 tokens (1,562,504 pooled router chunks,
               8 heads x 128, bf16); 4 x 512 router query tokens; top-16; docs
               drawn around 1024 Gaussian cluster centres with sigma 0.3.
* ``STACK18``  18 routed layers, 19,532 docs x 512 tokens per layer; 8192-token
               prefill; top-32.
"""

from dataclasses import dataclass, replace
import math

import numpy as np
import torch

__all__ = [
    "LayerConfig", "TINY", "PREFILL", "DECODE", "SCAN100M", "STACK18", "CONFIGS",
    "scaled", "draw_tiny", "draw_layer", "plant_router_queries", "rope_rotate",
    "draw_scan_bank_slab", "draw_scan_queries", "draw_scan_content_slab",
]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    dtype: str            # "f32" or "bf16"
    n_doc: int
    doc_len: int
    chunk: int
    heads_q: int
    heads_kv: int
    dim: int              # head dim = router dim per KV head
    batch: int
    q_len: int
    loc_len: int
    topk: int
    n_planted: int        # planted documents (0: router queries are plain Gaussian)
    plant_sigma: float    # plant noise, absolute
    value_scale: float    # std of the Gaussian draws
    rope: bool
    rope_base: float = 1.0e6
    pos0: int = 512       # first position of the query-side tokens
    layers: int = 1
    clusters: int = 0     # >0: router keys drawn around cluster centres
    cluster_sigma: float = 0.0

    @property
    def chunks_per_doc(self):
        return self.doc_len // self.chunk

    @property
    def n_chunks(self):
        return self.n_doc * self.chunks_per_doc

    @property
    def mem_len(self):
        return self.topk * self.chunks_per_doc

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


TINY = LayerConfig("tiny-fp32", "f32", n_doc=64, doc_len=512, chunk=64, heads_q=4, heads_kv=2,
                   dim=64, batch=1, q_len=32, loc_len=32, topk=4, n_planted=1,
                   plant_sigma=0.1, value_scale=1.0, rope=False)
PREFILL = LayerConfig("prefill-1M-bf16", "bf16", n_doc=2048, doc_len=512, chunk=64, heads_q=32,
                      heads_kv=8, dim=128, batch=1, q_len=2048, loc_len=2048, topk=16,
                      n_planted=16, plant_sigma=0.1 / math.sqrt(128), value_scale=1 / math.sqrt(128),
                      rope=True)
DECODE = LayerConfig("decode-1M-bf16", "bf16", n_doc=2048, doc_len=512, chunk=64, heads_q=32,
                     heads_kv=8, dim=128, batch=32, q_len=1, loc_len=4096, topk=16,
                     n_planted=0, plant_sigma=0.0, value_scale=1 / math.sqrt(128), rope=True)
SCAN100M = LayerConfig("scan-100M-share-bf16", "bf16", n_doc=195313, doc_len=512, chunk=64,
                       heads_q=32, heads_kv=8, dim=128, batch=4, q_len=512, loc_len=512, topk=16,
                       n_planted=0, plant_sigma=0.0, value_scale=1 / math.sqrt(128), rope=False,
                       clusters=1024, cluster_sigma=0.3)
STACK18 = LayerConfig("stack18-10M-bf16", "bf16", n_doc=19532, doc_len=512, chunk=64, heads_q=32,
                      heads_kv=8, dim=128, batch=1, q_len=8192, loc_len=8192, topk=32,
                      n_planted=0, plant_sigma=0.0, value_scale=1.0, rope=False, layers=18)

CONFIGS = {c.name: c for c in (TINY, PREFILL, DECODE, SCAN100M, STACK18)}


def scaled(cfg, **kw):
    """A smaller copy of a workload with the same recipe (for parity tests)."""
    return replace(cfg, name=cfg.name + "-scaled", **kw)


# ---------------------------------------------------------------------------
# drawing helpers
# ---------------------------------------------------------------------------

def _np_normal(rng, shape, scale):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _store(x_f32, cfg, device):
    """float32 tensor -> storage dtype on ``device`` (torch's RNE conversion)."""
    return x_f32.to(device=device, dtype=cfg.torch_dtype).contiguous()


def rope_rotate(x, positions, base):
    """Rotate-half rotary embedding of ``x`` [..., L, H, d] at ``positions`` [L].

    Part of *input synthesis*: it produces the rotated K/Q a model would feed
    to the routed layer.  Neither the oracle nor the HIP path applies it.
    """
    d = x.shape[-1]
    half = d // 2
    inv_freq = base ** (-torch.arange(0, half, dtype=torch.float64, device=x.device) * 2.0 / d)
    ang = positions.to(torch.float64)[:, None] * inv_freq[None, :]          # [L, half]
    cos = ang.cos().to(torch.float32)[:, None, :]                           # [L, 1, half]
    sin = ang.sin().to(torch.float32)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def _randn(gen, shape, device, scale):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale


def draw_tiny(seed, cfg=TINY):
    """Tiny fp32 workload from NumPy's default generator (device independent).

    Draw order: K, V, K_r [N_doc, L_doc, H_kv, d]; Q [B, T, H_q, d];
    K_loc, V_loc [B, L_loc, H_kv, d]; the noise for Q_r [B, T, H_kv, d].
    Returns CPU float32 torch tensors; ``q_r_noise`` is to be passed to
    :func:`plant_router_queries` with the pooled K_r bank.
    """
    rng = np.random.default_rng(seed)
    s = cfg.value_scale
    raw = (cfg.n_doc, cfg.doc_len, cfg.heads_kv, cfg.dim)
    out = {
        "k": _np_normal(rng, raw, s),
        "v": _np_normal(rng, raw, s),
        "k_r": _np_normal(rng, raw, s),
        "q": _np_normal(rng, (cfg.batch, cfg.q_len, cfg.heads_q, cfg.dim), s),
        "k_loc": _np_normal(rng, (cfg.batch, cfg.loc_len, cfg.heads_kv, cfg.dim), s),
        "v_loc": _np_normal(rng, (cfg.batch, cfg.loc_len, cfg.heads_kv, cfg.dim), s),
        "q_r_noise": _np_normal(rng, (cfg.batch, cfg.q_len, cfg.heads_kv, cfg.dim), 1.0),
    }
    t = {k: torch.from_numpy(v) for k, v in out.items()}
    if cfg.dtype == "bf16":
        for name in ("k", "v", "k_r", "q", "k_loc", "v_loc"):
            t[name] = t[name].to(torch.bfloat16)
    t["planted"] = torch.tensor([7] * cfg.batch if cfg.n_planted else [], dtype=torch.int64)
    return t


def draw_layer(cfg, seed, device="cpu", with_raw=True):
    """One routed layer's inputs for the bf16 recipes, drawn with torch on ``device``.

    Values are N(0, value_scale^2) float32, rotated where the recipe says so,
    then rounded to the storage dtype.  Draw order: K, V, K_r (raw document
    tensors, only when ``with_raw``), Q, K_loc, V_loc, Q_r noise, planted ids.
    The same seed on the same device type reproduces the same tensors.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    s = cfg.value_scale
    out = {}
    raw = (cfg.n_doc, cfg.doc_len, cfg.heads_kv, cfg.dim)
    if with_raw:
        k = _randn(gen, raw, device, s)
        if cfg.rope:
            k = rope_rotate(k, torch.arange(cfg.doc_len, device=device), cfg.rope_base)
        out["k"] = _store(k, cfg, device)
        del k
        out["v"] = _store(_randn(gen, raw, device, s), cfg, device)
        out["k_r"] = _store(_randn(gen, raw, device, s), cfg, device)
    q = _randn(gen, (cfg.batch, cfg.q_len, cfg.heads_q, cfg.dim), device, s)
    k_loc = _randn(gen, (cfg.batch, cfg.loc_len, cfg.heads_kv, cfg.dim), device, s)
    if cfg.rope:
        loc_pos = cfg.pos0 + torch.arange(cfg.loc_len, device=device)
        q_pos = loc_pos[cfg.loc_len - cfg.q_len:]
        q = rope_rotate(q, q_pos, cfg.rope_base)
        k_loc = rope_rotate(k_loc, loc_pos, cfg.rope_base)
    out["q"] = _store(q, cfg, device)
    out["k_loc"] = _store(k_loc, cfg, device)
    out["v_loc"] = _store(_randn(gen, (cfg.batch, cfg.loc_len, cfg.heads_kv, cfg.dim), device, s), cfg, device)
    noise = _randn(gen, (cfg.batch, cfg.q_len, cfg.heads_kv, cfg.dim), device, 1.0)
    out["q_r_noise"] = noise
    if cfg.n_planted:
        perm = torch.randperm(cfg.n_doc, generator=gen, device=device)
        out["planted"] = perm[: cfg.n_planted].to(torch.int64)
    else:
        out["planted"] = torch.empty(0, dtype=torch.int64, device=device)
        out["q_r"] = _store(noise * s, cfg, device)
    return out


def plant_router_queries(kbar_r, planted, noise, cfg):
    """Router queries that copy rows of planted documents' pooled K_r, plus noise.

    ``kbar_r`` [N_doc*C, H_kv, d] is the pooled bank (whichever side pooled it);
    ``planted`` holds the planted doc ids; ``noise`` [B, T, H_kv, d] is N(0,1).
    Every sequence uses all planted docs: its T tokens are split into
    ``len(planted)`` equal groups, and token t of group g copies chunk
    (t mod C) of doc planted[g]:  Q_r[b, t] = kbar_r[planted[g]*C + t mod C] + sigma * noise.
    Only copying and adding noise happens here.
    """
    n_p = planted.numel()
    if n_p == 0:
        raise ValueError("no planted documents")
    t_len = noise.shape[1]
    c = cfg.chunks_per_doc
    t = torch.arange(t_len, device=noise.device)
    group = (t * n_p) // t_len
    rows = planted.to(noise.device)[group] * c + (t % c)
    src = kbar_r.to(device=noise.device, dtype=torch.float32)[rows]             # [T, H, d]
    q = src[None] + cfg.plant_sigma * noise
    return _store(q, cfg, noise.device)


# ---------------------------------------------------------------------------
# large routing bank drawn around cluster centres
# ---------------------------------------------------------------------------

def _cluster_centres(cfg, seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    centres = torch.randn((cfg.clusters, cfg.heads_kv, cfg.dim), generator=gen, device=device)
    doc_cluster = torch.randint(0, cfg.clusters, (cfg.n_doc,), generator=gen, device=device)
    query_cluster = torch.randint(0, cfg.clusters, (cfg.batch,), generator=gen, device=device)
    return centres, doc_cluster, query_cluster


def draw_scan_bank_slab(cfg, seed, doc0, doc1, device):
    """Raw router keys of documents [doc0, doc1): centre of the doc's cluster
    plus cluster_sigma * N(0,1), rounded to the storage dtype.  Each slab has
    its own generator stream (seed, doc0) so slabs can be drawn in any order."""
    centres, doc_cluster, _ = _cluster_centres(cfg, seed, device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + doc0 + 1)
    n = doc1 - doc0
    x = torch.randn((n, cfg.doc_len, cfg.heads_kv, cfg.dim), generator=gen, device=device)
    # in place (one float32 temporary): sigma * eps, then + centre -- the same
    # float32 operations, in the same order, as centre + sigma * eps
    x.mul_(cfg.cluster_sigma).add_(centres[doc_cluster[doc0:doc1]][:, None])
    return _store(x, cfg, device)


def draw_scan_content_slab(cfg, seed, doc0, doc1, device):
    """Pooled content K-bar and V-bar rows of documents [doc0, doc1) for the
    large bank's host tier: N(0, value_scale^2) drawn directly at the pooled
    shape [(doc1-doc0)*C, H_kv, d] (the bank stores only pooled content; its
    values do not enter the routing), rounded to the storage dtype.  Each slab
    has its own generator stream (seed, doc0)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + 2_000_000_000 + doc0)
    shape = ((doc1 - doc0) * cfg.chunks_per_doc, cfg.heads_kv, cfg.dim)
    k = _store(_randn(gen, shape, device, cfg.value_scale), cfg, device)
    v = _store(_randn(gen, shape, device, cfg.value_scale), cfg, device)
    return k, v


def draw_scan_queries(cfg, seed, device):
    """Router queries for the large bank: each sequence b sits around one
    cluster centre (drawn uniformly), Q_r = centre + cluster_sigma * N(0,1)."""
    centres, _, query_cluster = _cluster_centres(cfg, seed, device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + 7)
    eps = torch.randn((cfg.batch, cfg.q_len, cfg.heads_kv, cfg.dim), generator=gen, device=device)
    q = centres[query_cluster][:, None] + cfg.cluster_sigma * eps
    return _store(q, cfg, device)
