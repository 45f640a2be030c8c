"""Plain float64 CPU oracle of the MSA routed-layer hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module.  It shares no code with the HIP path.

Sources (the pages this follows):

* [Design]   MSA README (github.com/EverMind-AI/MSA), section "Overall Design":
  document latent states K, V and the router key K_r are compressed by taking
  the mean over fixed-size chunks; a router scores each document by cosine
  similarity, averaged over heads and then maximised over query tokens; the
  top-k documents are selected and their compressed K/V are concatenated with
  the query's own local K/V for attention.
* [Pipeline] Same page, section "Inference Pipeline": stage 1 caches the
  chunk-pooled (K, V, K_r) offline; stage 2 projects the query to Q_r, matches
  it against the pooled K_r, picks the top-k and loads only the selected pooled
  K/V next to the local context; stage 3 generates over that sparse context.
* [Card]     william-0g/MSA-Qwen3.5 model card, opening paragraph and
  "Architecture summary": a per-layer router retrieves the top-k documents
  from the chunk-pooled bank by cosine routing; in the full (softmax) layers
  the top-k chunks' K/V are concatenated with the local KV inside sparse
  attention.
* [Blog]     moses-y.github.io "MSA" code walk, section "What This Does":
  restates chunk-mean pooling, cosine routing, top-k and concatenation.

Shapes (row-major, as in the C ABI):
    raw document tensors   x      [N_doc, L_doc, H, d]
    pooled bank            xbar   [N_doc * C, H, d]     C = L_doc / chunk
    router query           q_r    [B, T, H_kv, d_r]
    doc scores                    [B, N_doc]
    top-k ids / scores            [B, k]
    gathered memory        k_sel  [B, k * C, H_kv, d]
    query                  q      [B, T, H_q, d]
    local KV               k_loc  [B, L_loc, H_kv, d]
    output                 o      [B, T, H_q, d]
    log-sum-exp            lse    [B, H_q, T]
"""

import numpy as np

from .bf16 import round_bf16, round_f32

EPS = 1e-12


# ---------------------------------------------------------------------------
# S1: chunk-mean pooling
# ---------------------------------------------------------------------------

def pool_chunks_mean(x, chunk):
    """Exact chunk mean of each document's rows  ([Design]; [Pipeline] stage 1).

    ``x``: float64 [N_doc, L_doc, H, d].  Returns float64 [N_doc * C, H, d]
    where row ``n*C + j`` is (1/chunk) * sum_{i<chunk} x[n, j*chunk + i].

    Reading: the pages give no chunk size and never exercise a partial last
    chunk; L_doc must be a multiple of ``chunk``.
    """
    x = np.asarray(x, dtype=np.float64)
    n_doc, l_doc, h, d = x.shape
    if l_doc % chunk != 0:
        raise ValueError("document length must be a multiple of the chunk size")
    c = l_doc // chunk
    out = np.empty((n_doc, c, h, d), dtype=np.float64)
    for j in range(c):
        rows = x[:, j * chunk:(j + 1) * chunk]          # [N_doc, chunk, H, d]
        out[:, j] = rows.sum(axis=1) / chunk
    return out.reshape(n_doc * c, h, d)


def pool_chunks_stored(x, chunk, dtype):
    """Chunk mean rounded to the storage dtype ("bf16" or "f32"), as float64.

    Reading: the pooled bank is stored in the dtype of the raw tensors.
    """
    m = pool_chunks_mean(x, chunk)
    if dtype == "bf16":
        return round_bf16(m)
    if dtype == "f32":
        return round_f32(m)
    raise ValueError(dtype)


def chunk_norms(xbar_stored):
    """Euclidean norm of each stored pooled row, per (chunk, head): [N_ch, H].

    Reading: the norm is taken of the *stored* (rounded) pooled row, because
    routing consumes the stored rows.
    """
    x = np.asarray(xbar_stored, dtype=np.float64)
    return np.sqrt((x * x).sum(axis=-1))


# ---------------------------------------------------------------------------
# Offline encoder over variable-length documents (S1 at scale)
# ---------------------------------------------------------------------------

def rope_rotate_half(x, positions, base):
    """Rotary position embedding, rotate-half form, in float64.

    ``x`` [L, H, d] (d even), ``positions`` [L].  For k < d/2 the pair
    (x_k, x_{k+d/2}) is rotated by the angle positions * theta_k with
    theta_k = base ** (-2k / d):
        x'_k       = x_k cos - x_{k+d/2} sin
        x'_{k+d/2} = x_{k+d/2} cos + x_k sin

    Reading ([README] "Overall Design"; [Card] "Architecture summary"): the
    pages name document-wise RoPE but neither its form nor its base; the
    rotate-half form with base 1e6 is a Qwen-like assumption, and only K is
    rotated (V and the router key K_r are not).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("rotary embedding needs an even head dim")
    half = d // 2
    theta = np.power(float(base), -2.0 * np.arange(half) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]   # [L, half]
    cos, sin = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def chunk_offsets(doc_off, chunk):
    """First pooled chunk of each document: chunk_off[n] = sum_{m<n} ceil(L_m / chunk)."""
    doc_off = np.asarray(doc_off, dtype=np.int64)
    lens = np.diff(doc_off)
    if np.any(lens < 0) or doc_off[0] != 0:
        raise ValueError("doc_off must start at 0 and be nondecreasing")
    n_ch = (lens + chunk - 1) // chunk
    return np.concatenate([[0], np.cumsum(n_ch)]).astype(np.int64)


def encode_docs(x, doc_off, chunk, rope_base=None):
    """Chunk means of variable-length documents, optionally after document-wise RoPE.

    ``x`` [total_rows, H, d]; document n is rows doc_off[n] .. doc_off[n+1]-1.
    Chunk j of document n is the mean of its rows j*chunk .. min((j+1)*chunk,
    L_n) - 1 -- the last chunk of a document may be shorter, and its mean is
    over the rows present.  With ``rope_base`` the rows are first rotated at
    their document-local positions 0 .. L_n - 1 (rope_rotate_half).  Returns
    the exact float64 means [total_chunks, H, d] and chunk_offsets.

    Follows [README] "Overall Design" (chunk-mean compression) and "Inference
    Pipeline" stage 1 (offline encoding of the memory).  Reading: the pages
    never show a partial last chunk; the mean over the rows present is the
    plainest reading of a chunk mean.
    """
    x = np.asarray(x, dtype=np.float64)
    c_off = chunk_offsets(doc_off, chunk)
    out = np.empty((int(c_off[-1]),) + x.shape[1:], dtype=np.float64)
    for n in range(len(doc_off) - 1):
        rows = x[doc_off[n]:doc_off[n + 1]]
        if rope_base is not None and len(rows):
            rows = rope_rotate_half(rows, np.arange(len(rows)), rope_base)
        for j in range(int(c_off[n + 1] - c_off[n])):
            seg = rows[j * chunk:(j + 1) * chunk]
            out[c_off[n] + j] = seg.sum(axis=0) / len(seg)
    return out, c_off


# ---------------------------------------------------------------------------
# S2: cosine routing
# ---------------------------------------------------------------------------

def route_scores(q_r, kbar_r, chunks_per_doc, eps=EPS, doc_block=None):
    """Document scores by cosine routing  ([Design]; [Card] opening; [Pipeline] stage 2).

    For sequence b, token t, pooled chunk n and head h:
        cos[b,t,n,h] = <q_r[b,t,h], kbar_r[n,h]> / (max(|q_r[b,t,h]|, eps) * max(|kbar_r[n,h]|, eps))
    then the mean over heads,
        s[b,t,n] = (1/H) * sum_h cos[b,t,n,h]
    then the maximum over the query tokens and over the chunks of each document,
        score[b,doc] = max_{t < T, j < C} s[b, t, doc*C + j].

    Readings: the head mean is taken of per-head cosines (the similarity is
    pooled, not the vectors); the chunk-to-document reduction is a max; the
    router has one head per KV head; every query token of the sequence takes
    part (no causal restriction); ``eps`` only matters for all-zero rows.

    ``doc_block`` optionally evaluates the documents in independent groups to
    bound memory; each document's score depends only on its own chunks, so
    the result is identical.
    """
    q = np.asarray(q_r, dtype=np.float64)
    k = np.asarray(kbar_r, dtype=np.float64)
    b_, t_, h_, d_ = q.shape
    n_ch = k.shape[0]
    if k.shape[1:] != (h_, d_):
        raise ValueError("router query and pooled keys disagree on heads/dim")
    if n_ch % chunks_per_doc != 0:
        raise ValueError("chunk count must be a multiple of chunks per document")
    n_doc = n_ch // chunks_per_doc
    qn = np.maximum(np.sqrt((q * q).sum(axis=-1)), eps)     # [B, T, H]
    kn = np.maximum(np.sqrt((k * k).sum(axis=-1)), eps)     # [N_ch, H]
    if doc_block is None:
        doc_block = n_doc
    out = np.empty((b_, n_doc), dtype=np.float64)
    for d0 in range(0, n_doc, doc_block):
        d1 = min(n_doc, d0 + doc_block)
        c0, c1 = d0 * chunks_per_doc, d1 * chunks_per_doc
        s = np.zeros((b_, t_, c1 - c0), dtype=np.float64)
        for h in range(h_):
            dots = q[:, :, h, :] @ k[c0:c1, h, :].T                 # [B, T, n]
            s += dots / (qn[:, :, h, None] * kn[None, None, c0:c1, h])
        s /= h_
        per_chunk = s.max(axis=1)                                    # max over tokens
        out[:, d0:d1] = per_chunk.reshape(b_, d1 - d0, chunks_per_doc).max(axis=2)
    return out


# ---------------------------------------------------------------------------
# S3: top-k document selection
# ---------------------------------------------------------------------------

def topk_docs(scores, k):
    """The k best documents per sequence  ([Design]; [Pipeline] stage 2).

    Order: score descending; equal scores go to the lower document id.  Returns
    (ids int64 [B, k], values float64 [B, k]).  Reading: the pages leave the
    tie rule and output order open; this total order makes the answer unique.
    """
    s = np.asarray(scores, dtype=np.float64)
    b_, n = s.shape
    if not 1 <= k <= n:
        raise ValueError("k must lie in [1, N_doc]")
    ids = np.empty((b_, k), dtype=np.int64)
    vals = np.empty((b_, k), dtype=np.float64)
    doc = np.arange(n)
    for b in range(b_):
        # lexsort sorts by the last key first: score descending, then id ascending.
        order = np.lexsort((doc, -s[b]))
        ids[b] = order[:k]
        vals[b] = s[b, order[:k]]
    return ids, vals


# ---------------------------------------------------------------------------
# Memory Interleave: several routing rounds, each excluding earlier picks
# ---------------------------------------------------------------------------

def topk_docs_excluding(scores, k, exclude):
    """The k best documents per sequence among those not in its exclusion set.

    ``exclude[b]`` lists the ids sequence b may not select (a list per
    sequence, or a [B, n] integer array); ids outside [0, N_doc) are ignored,
    so -1 may pad a row, and repeated ids count once.  The order and the tie
    rule are those of :func:`topk_docs`.  Raises ValueError when fewer than k
    documents remain.  Returns (ids int64 [B, k], values float64 [B, k]).

    Reading ([README] "Inference Pipeline", Figure 3, and the page's FAQ on
    Memory Interleave: routing may run for several rounds, each round jumping
    to further memory segments): a later round does not pick a document an
    earlier round already brought into the context.
    """
    s = np.asarray(scores, dtype=np.float64)
    b_, n = s.shape
    if not 1 <= k <= n:
        raise ValueError("k must lie in [1, N_doc]")
    ids = np.empty((b_, k), dtype=np.int64)
    vals = np.empty((b_, k), dtype=np.float64)
    for b in range(b_):
        banned = {int(i) for i in np.asarray(exclude[b]).reshape(-1) if 0 <= int(i) < n}
        allowed = np.array([d for d in range(n) if d not in banned], dtype=np.int64)
        if allowed.size < k:
            raise ValueError("fewer than k documents remain after the exclusion")
        order = np.lexsort((allowed, -s[b, allowed]))
        ids[b] = allowed[order[:k]]
        vals[b] = s[b, ids[b]]
    return ids, vals


def route_rounds(q_r_rounds, kbar_r, chunks_per_doc, k, eps=EPS):
    """Multi-round routing (Memory Interleave), kernel level.

    Round r routes its own router query ``q_r_rounds[r]`` ([B, T, H, d]; the
    model produces it between rounds) against the bank as in
    :func:`route_scores`, then takes the top-k among the documents no earlier
    round selected (:func:`topk_docs_excluding`).  Returns (ids int64 [B, R*k],
    values float64 [B, R*k]): round r's picks in columns [r*k, (r+1)*k), each
    round in rank order.  Reading: the rounds' documents are concatenated in
    round order, and the gathered memory follows that order.
    """
    q = [np.asarray(x, dtype=np.float64) for x in q_r_rounds]
    if not q:
        raise ValueError("at least one round")
    b_ = q[0].shape[0]
    ids = np.empty((b_, 0), dtype=np.int64)
    vals = np.empty((b_, 0), dtype=np.float64)
    for qr in q:
        s = route_scores(qr, kbar_r, chunks_per_doc, eps=eps)
        i_r, v_r = topk_docs_excluding(s, k, ids)
        ids = np.concatenate([ids, i_r], axis=1)
        vals = np.concatenate([vals, v_r], axis=1)
    return ids, vals


# ---------------------------------------------------------------------------
# S4: gather of the selected documents' pooled K/V
# ---------------------------------------------------------------------------

def gather_kv(kbar, vbar, ids, chunks_per_doc):
    """Selected documents' pooled K/V, in rank order  ([Pipeline] stage 2).

    k_sel[b, i*C + j] = kbar[ids[b, i]*C + j] and likewise for V.  Reading: the
    memory rows follow the rank order of the top-k list (softmax does not
    depend on the order of keys).  Ids outside [0, N_doc) are an error.
    """
    kb = np.asarray(kbar)
    vb = np.asarray(vbar)
    ids = np.asarray(ids)
    n_doc = kb.shape[0] // chunks_per_doc
    if ids.min() < 0 or ids.max() >= n_doc:
        raise IndexError("document id out of range")
    b_, k = ids.shape
    rows = (ids[:, :, None] * chunks_per_doc + np.arange(chunks_per_doc)[None, None, :]).reshape(b_, k * chunks_per_doc)
    return kb[rows], vb[rows]


# ---------------------------------------------------------------------------
# S5/S6: GQA softmax attention over [selected memory ; local causal KV]
# ---------------------------------------------------------------------------

def sparse_attention_rows(q_row, keys, values, scale):
    """Softmax attention of one query row over the given visible keys.

    Returns (o [d], lse).  lse = m + log(sum exp(l - m)), with l = scale*q.k
    and m = max l.
    """
    logits = scale * (keys @ q_row)
    m = logits.max()
    p = np.exp(logits - m)
    l_sum = p.sum()
    return (p @ values) / l_sum, m + np.log(l_sum)


def sparse_attention(q, k_sel, v_sel, k_loc, v_loc, scale=None):
    """Sparse GQA attention of the MSA layer  ([Card] "Architecture summary";
    [Design]; [Pipeline] stage 3).

    For sequence b, query token t < T and query head h, with KV head
    g = h // (H_q / H_kv), the keys are the M gathered memory rows followed by
    the local rows 0 .. L_loc - T + t (bottom-right causal alignment: the last
    query token sees every local row), and

        o[b,t,h] = softmax(scale * q[b,t,h] . keys^T) . values.

    Readings: scale defaults to 1/sqrt(d); memory rows are visible to every
    query token; query heads map to KV heads in contiguous groups; no dropout,
    window, sink or soft-cap.  For decode (T = 1) the local rows include the
    new token's own key.

    Returns (o float64 [B, T, H_q, d], lse float64 [B, H_q, T]).
    """
    q = np.asarray(q, dtype=np.float64)
    ks = np.asarray(k_sel, dtype=np.float64)
    vs = np.asarray(v_sel, dtype=np.float64)
    kl = np.asarray(k_loc, dtype=np.float64)
    vl = np.asarray(v_loc, dtype=np.float64)
    b_, t_, hq, d = q.shape
    m_len = ks.shape[1]
    l_len = kl.shape[1]
    hkv = ks.shape[2]
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if l_len < t_:
        raise ValueError("local KV must hold at least the query tokens")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((b_, t_, hq, d), dtype=np.float64)
    lse = np.empty((b_, hq, t_), dtype=np.float64)
    for b in range(b_):
        for h in range(hq):
            g = h // group
            keys = np.concatenate([ks[b, :, g], kl[b, :, g]], axis=0)    # [M + L_loc, d]
            vals = np.concatenate([vs[b, :, g], vl[b, :, g]], axis=0)
            for t in range(t_):
                visible = m_len + (l_len - t_ + t + 1)
                o[b, t, h], lse[b, h, t] = sparse_attention_rows(
                    q[b, t, h], keys[:visible], vals[:visible], scale)
    return o, lse


def merge_attention(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key sets, from the attention over each.

    The attention of [Card] "Architecture summary" / [Pipeline] stage 3 runs
    over the memory rows followed by the local rows; split into two disjoint
    key sets A and B, the softmax over A u B weights each part by its share of
    the normaliser: with lse_X = log sum_{j in X} exp(l_j),

        lse = log(exp(lse_a) + exp(lse_b)),
        o   = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b.

    A part with lse = -inf holds no visible key and gets weight 0; when both
    are -inf the result is o = 0, lse = -inf (a reading: nothing is visible).

    o_* [B, T, H, d], lse_* [B, H, T]; returns (o float64, lse float64).
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    empty = np.isneginf(lse)
    safe = np.where(empty, 0.0, lse)
    w_a = np.where(empty, 0.0, np.exp(lse_a - safe))          # [B, H, T]
    w_b = np.where(empty, 0.0, np.exp(lse_b - safe))
    to_o = lambda w: np.transpose(w, (0, 2, 1))[..., None]     # -> [B, T, H, 1]
    return to_o(w_a) * o_a + to_o(w_b) * o_b, lse


# ---------------------------------------------------------------------------
# Backward of the sparse attention (the method is trained end to end)
# ---------------------------------------------------------------------------

def sparse_attention_backward(q, k_sel, v_sel, k_loc, v_loc, d_out, scale=None):
    """Gradients of :func:`sparse_attention` ([README] "Abstract" and the
    Figure 1 caption: top-k selection is fused with sparse attention so that
    the model stays end-to-end differentiable; [Card] "Architecture summary"
    and "Training (CPT)": the router and adapters are trained through the
    routed layers).

    Given dL/do = ``d_out`` [B, T, H_q, d], for each (b, h) with KV head g and
    each query row t over its visible keys (as in the forward):
        p      = softmax(scale * q_t . keys^T)
        dv_j  += p_j * dO_t                      (V of key j)
        dp_j   = dO_t . v_j
        ds_j   = p_j * (dp_j - sum_l p_l dp_l)   (softmax Jacobian)
        dq_t   = scale * sum_j ds_j k_j
        dk_j  += scale * ds_j * q_t
    A KV head's gradients sum over the query heads of its group and over the
    query tokens that see it.  Written per (b, h) as masked matrix products.

    Returns float64 (dq [B,T,H_q,d], dk_sel [B,M,H_kv,d], dv_sel [B,M,H_kv,d],
    dk_loc [B,L,H_kv,d], dv_loc [B,L,H_kv,d]).
    """
    q = np.asarray(q, dtype=np.float64)
    ks = np.asarray(k_sel, dtype=np.float64)
    vs = np.asarray(v_sel, dtype=np.float64)
    kl = np.asarray(k_loc, dtype=np.float64)
    vl = np.asarray(v_loc, dtype=np.float64)
    do = np.asarray(d_out, dtype=np.float64)
    b_, t_, hq, d = q.shape
    m_len, l_len, hkv = ks.shape[1], kl.shape[1], ks.shape[2]
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if l_len < t_:
        raise ValueError("local KV must hold at least the query tokens")
    if do.shape != q.shape:
        raise ValueError("d_out must have the query's shape")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n_keys = m_len + l_len
    # visible[t, j]: memory rows always; local row i when i <= L - T + t
    j = np.arange(n_keys)
    t = np.arange(t_)
    visible = (j[None, :] < m_len) | ((j[None, :] - m_len) <= (l_len - t_ + t)[:, None])
    dq = np.zeros_like(q)
    dkeys = np.zeros((b_, n_keys, hkv, d))
    dvals = np.zeros((b_, n_keys, hkv, d))
    for b in range(b_):
        for h in range(hq):
            g = h // group
            keys = np.concatenate([ks[b, :, g], kl[b, :, g]], axis=0)    # [n_keys, d]
            vals = np.concatenate([vs[b, :, g], vl[b, :, g]], axis=0)
            logits = np.where(visible, scale * (q[b, :, h] @ keys.T), -np.inf)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)                               # [T, n_keys]
            dp = do[b, :, h] @ vals.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, :, h] = scale * (ds @ keys)
            dkeys[b, :, g] += scale * (ds.T @ q[b, :, h])
            dvals[b, :, g] += p.T @ do[b, :, h]
    return dq, dkeys[:, :m_len], dvals[:, :m_len], dkeys[:, m_len:], dvals[:, m_len:]


# ---------------------------------------------------------------------------
# Linear-layer variant: document states injected as the initial state
# ---------------------------------------------------------------------------

def gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None):
    """Gated delta rule over a sequence, one step per token, in float64.

    [Card] "Architecture summary": in the linear (DGA) layers each document is
    encoded through the layer's recurrence, and the query path runs the
    chunked gated delta rule starting from an injected initial state.  The
    pages name the rule but not its equations; the reading here is the
    published gated delta rule (decay gate alpha = exp(g), writing strength
    beta), with the state h[k_dim, v_dim] of each (sequence, head):

        h   <- alpha_t * h                       (decay)
        u    = h^T k_t                           (what the memory predicts for k_t)
        h   <- h + k_t (beta_t (v_t - u))^T      (delta-rule write)
        o_t  = scale * h^T q_t

    q, k [B, T, H, dk]; v [B, T, H, dv]; g, beta [B, T, H]; initial_state
    [B, H, dk, dv] or None (zeros).  scale defaults to 1/sqrt(dk).  Keys are
    used as given (the caller normalises them if the model does).
    Returns (o float64 [B, T, H, dv], final state float64 [B, H, dk, dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    b_, t_, h_, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    h = np.zeros((b_, h_, dk, dv)) if initial_state is None else np.array(initial_state, dtype=np.float64)
    o = np.empty((b_, t_, h_, dv))
    for t in range(t_):
        alpha = np.exp(g[:, t])[:, :, None, None]                     # [B, H, 1, 1]
        h = alpha * h
        kt = k[:, t]                                                  # [B, H, dk]
        u = np.einsum("bhkv,bhk->bhv", h, kt)
        delta = beta[:, t][:, :, None] * (v[:, t] - u)                # [B, H, dv]
        h = h + kt[:, :, :, None] * delta[:, :, None, :]
        o[:, t] = scale * np.einsum("bhkv,bhk->bhv", h, q[:, t])
    return o, h


def inject_states(doc_states, ids):
    """Initial state of the query path: the sum of the selected documents'
    states, S_ext[b, h] = sum_i doc_states[ids[b, i], h]  ([Card]
    "Architecture summary": the top-k documents' recurrent states are summed
    into S_ext).  doc_states [N_doc, H, dk, dv]; ids [B, k] in [0, N_doc).
    """
    s = np.asarray(doc_states, dtype=np.float64)
    ids = np.asarray(ids)
    if ids.size and (ids.min() < 0 or ids.max() >= s.shape[0]):
        raise IndexError("document id out of range")
    return s[ids].sum(axis=1)
