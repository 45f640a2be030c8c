/*
 * msa.h -- C ABI of libmsa, the MI355X (gfx950) hot path of Memory Sparse
 * Attention (MSA) for one routed layer.
 *
 * The method (MSA README, github.com/EverMind-AI/MSA, "Overall Design" and
 * "Inference Pipeline"; william-0g/MSA-Qwen3.5 model card, opening paragraph
 * and "Architecture summary"):
 *   1. document K, V and router keys K_r are mean-pooled over fixed-size
 *      chunks into a memory bank (K-bar, V-bar, K_r-bar);
 *   2. each document is scored by the cosine similarity between the query's
 *      router projection Q_r and K_r-bar, averaged over heads and maximised
 *      over query tokens (and over the document's chunks);
 *   3. the top-k documents are selected;
 *   4. only their pooled K/V are loaded and placed before the local K/V;
 *   5. GQA softmax attention runs over that sparse context.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, row-major, in the layouts stated per call.  Pointers
 *   are device pointers unless stated otherwise, 16-byte aligned.
 * - The caller owns every buffer.  No entry point allocates device memory;
 *   scratch space comes from the caller's workspace (`ws`, `ws_bytes`),
 *   sized by the matching *_workspace call (or by msa_workspace_size).
 *   (msa_gather_kv keeps a library-owned side stream per device and a pool
 *   of staging slots, each a few events, a pinned id buffer and one device
 *   error word; a call takes a slot of its own for its duration.  They are
 *   created on first use and kept until the process ends.)
 * - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *   All work is enqueued on it, asynchronously; a call returns before the
 *   GPU has finished unless stated otherwise.
 * - Argument errors are detected on the host before anything is enqueued and
 *   returned as MSA_ERR_INVALID (bad value) or MSA_ERR_UNSUPPORTED (valid
 *   but not implemented).  A failed launch returns MSA_ERR_HIP.  Faults of
 *   enqueued work surface at the caller's next synchronisation, as in HIP.
 *   msa_last_error() then returns a description (thread-local).
 * - No C++ exception crosses this boundary.  Calls are thread-safe: the
 *   only state shared between calls is the host tier's staging pool, taken
 *   and returned under a lock that is never held while waiting.  Calls on one
 *   stream execute in order.
 * - dtype MSA_BF16 stores bfloat16 bit patterns (uint16); MSA_F32 stores
 *   IEEE float32.  Arithmetic is float32 in either case; rounding to the
 *   storage dtype is round-to-nearest-even.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID = 1,
  MSA_ERR_UNSUPPORTED = 2,
  MSA_ERR_HIP = 3
} msa_status;

typedef enum msa_dtype { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

/* Gather flags (msa_gather_kv). */
#define MSA_GATHER_CHECKED 1     /* synchronise and report out-of-range ids as MSA_ERR_INVALID */
#define MSA_GATHER_HOST_MEMCPY 2 /* host tier: per-document hipMemcpyAsync on a side stream     */

/* Operations, for msa_workspace_size. */
typedef enum msa_op {
  MSA_OP_POOL_CHUNKS = 0,
  MSA_OP_ROUTE_SCORES = 1,
  MSA_OP_TOPK_DOCS = 2,
  MSA_OP_GATHER_KV = 3,
  MSA_OP_SPARSE_ATTN = 4,
  MSA_OP_SPARSE_ATTN_BACKWARD = 5,
  MSA_OP_ROUTE_ROUNDS = 6,
  MSA_OP_TOPK_DOCS_EXCLUDING = 7,
  MSA_OP_ENCODE_DOCS = 8,
  MSA_OP_GDN_STATE_SUM = 9,
  MSA_OP_GATED_DELTA_RULE = 10,
  MSA_OP_GATED_DELTA_RULE_CHUNKED = 11
} msa_op;

/* Version of this ABI (bumped on any incompatible change). */
int msa_abi_version(void);

/* Text describing the last non-OK status returned on the calling thread. */
const char* msa_last_error(void);

/* ------------------------------------------------------------------------
 * Workspace size of one call, by operation (MSA README "Inference Pipeline":
 * the three stages whose steps the entry points below implement).  One
 * entry point in front of the per-operation *_workspace calls, for callers
 * that size scratch generically.
 *
 * op     an msa_op value
 * dims   the integer arguments of the operation's *_workspace call, in that
 *        call's order, the dtype given as its msa_dtype value:
 *          MSA_OP_ROUTE_SCORES          {batch, q_len, heads, dim, n_docs, chunks_per_doc, dtype}
 *          MSA_OP_TOPK_DOCS(_EXCLUDING) {batch, n_docs, k}
 *          MSA_OP_ROUTE_ROUNDS          {rounds, batch, q_len, heads, dim, n_docs, chunks_per_doc, k, dtype}
 *          MSA_OP_SPARSE_ATTN(_BACKWARD) {batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dtype}
 *        The other operations use no scratch: *bytes = 0 whatever dims hold.
 * ndims  the number of entries in dims; a count that does not match the
 *        operation, an unknown op or an argument the per-operation call
 *        rejects returns MSA_ERR_INVALID.
 * bytes  output: the workspace size in bytes (host pointer).
 * ---------------------------------------------------------------------- */
msa_status msa_workspace_size(int32_t op, const int64_t* dims, int32_t ndims, size_t* bytes);

/* ------------------------------------------------------------------------
 * S1  Chunk-mean pooling (MSA README "Overall Design"; "Inference Pipeline",
 *     stage 1: the offline encoding caches chunk-pooled K, V and K_r).
 *
 *   xbar[n*C + j, h, :] = (1/chunk) * sum_{i<chunk} x[n, j*chunk + i, h, :]
 *
 * x          [n_docs, doc_len, heads, dim]   input rows (dtype dt)
 * xbar       [n_docs*C, heads, dim]          output, C = doc_len/chunk (dtype dt)
 * xbar_norm  [n_docs*C, heads] float32, or NULL: Euclidean norm of each
 *            *stored* (rounded) pooled row; the routing step consumes it.
 * Requires doc_len % chunk == 0; heads*dim*sizeof(dt) % 16 == 0; when
 * xbar_norm is given, dim*sizeof(dt) must be a power of two in [16, 1024].
 * ---------------------------------------------------------------------- */
msa_status msa_pool_chunks(const void* x, void* xbar, float* xbar_norm, int64_t n_docs,
                           int32_t doc_len, int32_t chunk, int32_t heads, int32_t dim,
                           msa_dtype dt, void* stream);

/* ------------------------------------------------------------------------
 * Offline encoder over variable-length documents (MSA README "Overall
 * Design": chunk-mean compression of document K, V and K_r, K rotated by
 * document-wise RoPE; "Inference Pipeline", stage 1: offline encoding).
 *
 * Documents are row ranges of one tensor: document n is rows
 * doc_off[n] .. doc_off[n+1]-1.  Each is cut into chunks of `chunk` rows; the
 * last chunk of a document may be shorter and its mean is over the rows
 * present (a reading: the pages never show one).
 *
 * msa_chunk_offsets: chunk_off[0] = 0,
 *   chunk_off[n+1] = chunk_off[n] + ceil((doc_off[n+1] - doc_off[n]) / chunk).
 *   doc_off, chunk_off: device int64 arrays of n_docs + 1 entries.  doc_off
 *   must start at 0 and be nondecreasing (not checked on the device).
 *
 * msa_encode_docs:
 *   xbar[chunk_off[n] + j, h, :] = (1/cnt) * sum_{i<cnt} R(j*chunk + i) x[doc_off[n] + j*chunk + i, h, :]
 *   with cnt = min(chunk, L_n - j*chunk) and R(p) the identity when
 *   rope_base == 0, else the rotate-half rotary embedding at position p: for
 *   k < dim/2 the pair (x_k, x_{k+dim/2}) turns by p * rope_base^(-2k/dim).
 *   x          [total_rows, heads, dim]          input rows (dtype dt)
 *   xbar       [total_chunks, heads, dim]        output (dtype dt), total_chunks = chunk_off[n_docs]
 *   xbar_norm  [total_chunks, heads] float32, or NULL: norms of the stored rows
 *   doc_off, chunk_off: as above (chunk_off from msa_chunk_offsets).
 *   Requires heads*dim*sizeof(dt) % 16 == 0; with xbar_norm or rope_base > 0,
 *   dim*sizeof(dt) must be a power of two in [32, 1024].  Offsets that point
 *   outside x read nothing (the chunk comes out as zeros); they are not
 *   reported.  rope_base == 0 and equal lengths reproduce msa_pool_chunks.
 * ---------------------------------------------------------------------- */
msa_status msa_chunk_offsets(const int64_t* doc_off, int64_t n_docs, int32_t chunk,
                             int64_t* chunk_off, void* stream);
msa_status msa_encode_docs(const void* x, void* xbar, float* xbar_norm, const int64_t* doc_off,
                           const int64_t* chunk_off, int64_t n_docs, int64_t total_rows,
                           int64_t total_chunks, int32_t chunk, int32_t heads, int32_t dim,
                           float rope_base, msa_dtype dt, void* stream);

/* ------------------------------------------------------------------------
 * S2  Cosine routing scores (MSA README "Overall Design": cosine similarity
 *     averaged over heads, then maximised over query tokens; model card
 *     opening paragraph: per-layer router over the chunk-pooled bank).
 *
 *   cos[b,t,n,h] = <q_r[b,t,h], kbar_r[n,h]> / (max(|q_r[b,t,h]|,1e-12) * max(kbar_r_norm[n,h],1e-12))
 *   doc_scores[b, doc] = max_{t<q_len, j<C} (1/heads) * sum_h cos[b, t, doc*C + j, h]
 *
 * q_r          [batch, q_len, heads, dim]       router queries (dtype dt)
 * kbar_r       [n_docs*C, heads, dim]            pooled router keys (dtype dt)
 * kbar_r_norm  [n_docs*C, heads] float32         their norms (from msa_pool_chunks)
 * doc_scores   [batch, n_docs] float32           output
 * ws           msa_route_scores_workspace() bytes of device scratch (may be 0)
 * Products of bf16 values are exact in float32; per-head dot products are
 * scaled by the float32 inverse norms (normalised vectors are never rounded).
 * ---------------------------------------------------------------------- */
msa_status msa_route_scores_workspace(int32_t batch, int32_t q_len, int32_t heads, int32_t dim,
                                      int64_t n_docs, int32_t chunks_per_doc, msa_dtype dt,
                                      size_t* bytes);
msa_status msa_route_scores(const void* q_r, const void* kbar_r, const float* kbar_r_norm,
                            int32_t batch, int32_t q_len, int32_t heads, int32_t dim,
                            int64_t n_docs, int32_t chunks_per_doc, msa_dtype dt,
                            float* doc_scores, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * msa_route_scores without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, same result, same kernels
 * as msa_route_scores; the scratch the tiled path needs (the inverse query
 * norms, msa_route_scores_workspace() bytes: 32 bytes per router token at 8
 * heads) comes from a library-resident device array of 32 MiB per device,
 * which each device the library runs on holds until the process ends.  The
 * call allocates nothing.  A call needing more scratch than that (more than
 * 1,048,576 router tokens at 8 heads) returns MSA_ERR_INVALID before any
 * launch.
 * Every call on one device shares that array: calls that overlap in time on
 * one device (on different streams, or from several threads) race on it and
 * give undefined scores; serialise them (one stream per device suffices).
 * Each call overwrites every byte it later reads, so nothing needs clearing.
 * ---------------------------------------------------------------------- */
msa_status msa_route_scores_noalloc(const void* q_r, const void* kbar_r, const float* kbar_r_norm,
                                    int32_t batch, int32_t q_len, int32_t heads, int32_t dim, int64_t n_docs,
                                    int32_t chunks_per_doc, msa_dtype dt, float* doc_scores, void* stream);

/* ------------------------------------------------------------------------
 * S3  Top-k documents (MSA README "Overall Design" and "Inference Pipeline",
 *     stage 2: pick the top-k documents by routing score).
 *
 * The k largest scores of each row, in descending order; equal scores are
 * ordered by ascending document id (a total order: the result is unique).
 * -0.0 compares equal to +0.0.  NaN scores are outside the contract.
 *
 * doc_scores   [batch, n_docs] float32
 * topk_ids     [batch, k] int32 output
 * topk_scores  [batch, k] float32 output, or NULL
 * Requires 1 <= k <= min(n_docs, 1024), n_docs < 2^31.
 * ---------------------------------------------------------------------- */
msa_status msa_topk_docs_workspace(int32_t batch, int64_t n_docs, int32_t k, size_t* bytes);
msa_status msa_topk_docs(const float* doc_scores, int32_t batch, int64_t n_docs, int32_t k,
                         int32_t* topk_ids, float* topk_scores, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * Multi-round routing, "Memory Interleave" (MSA README "Inference Pipeline",
 *     Figure 3: an optional multi-round interleave for multi-hop questions;
 *     the same page's FAQ: the rounds jump across scattered memory segments).
 *     Kernel level only: how the model forms each round's router query is
 *     not part of this library.  Reading: a round never re-selects a document
 *     an earlier round selected, and the rounds' picks are concatenated in
 *     round order.
 *
 * msa_topk_docs_excluding: msa_topk_docs over the documents of row b that are
 *   not among excl_ids[b*excl_stride + 0 .. n_excl-1] (int32, device).
 *   Excluded ids outside [0, n_docs) are ignored (-1 may pad a row); repeated
 *   ids count once.  Row b's results go to topk_ids[b*out_stride + 0 .. k-1]
 *   (and topk_scores likewise, or NULL).  Requires k + n_excl <= n_docs (k
 *   documents always remain), excl_stride >= n_excl, out_stride >= k; the
 *   workspace is msa_topk_docs_workspace(batch, n_docs, k).  The exclusion
 *   entries may share the output buffer only in the multi-round layout (equal
 *   strides, row b's outputs after its n_excl entries, e.g. excl_ids = ids,
 *   topk_ids = ids + n_excl); other overlaps return MSA_ERR_INVALID.
 *
 * msa_route_rounds: `rounds` rounds on `stream`; round r routes
 *   q_r[r] as msa_route_scores does, then keeps the top-k of the documents no
 *   earlier round selected (msa_topk_docs_excluding).  A round's scores do
 *   not depend on the earlier picks, so when the tiled routing kernel takes
 *   both shapes the routing of all rounds runs as one launch over
 *   rounds*batch sequences (same results as round-by-round calls).
 *   q_r          [rounds, batch, q_len, heads, dim]  (dtype dt)
 *   kbar_r, kbar_r_norm as for msa_route_scores
 *   topk_ids     [batch, rounds*k] int32 output: round r in columns [r*k, (r+1)*k)
 *   topk_scores  [batch, rounds*k] float32 output, or NULL
 *   ws           msa_route_rounds_workspace() bytes (the per-round scores
 *                plus the route / top-k scratch); 16-byte aligned
 *   Requires 1 <= rounds, rounds*k <= n_docs, k <= 1024.  The batch*rounds*k
 *   ids are distinct per row; msa_gather_kv with k' = rounds*k then gives the
 *   memory rows in round order.
 * ---------------------------------------------------------------------- */
msa_status msa_topk_docs_excluding(const float* doc_scores, int32_t batch, int64_t n_docs, int32_t k,
                                   const int32_t* excl_ids, int32_t n_excl, int64_t excl_stride,
                                   int32_t* topk_ids, float* topk_scores, int64_t out_stride, void* ws,
                                   size_t ws_bytes, void* stream);
msa_status msa_route_rounds_workspace(int32_t rounds, int32_t batch, int32_t q_len, int32_t heads,
                                      int32_t dim, int64_t n_docs, int32_t chunks_per_doc, int32_t k,
                                      msa_dtype dt, size_t* bytes);
msa_status msa_route_rounds(const void* q_r, const void* kbar_r, const float* kbar_r_norm,
                            int32_t rounds, int32_t batch, int32_t q_len, int32_t heads, int32_t dim,
                            int64_t n_docs, int32_t chunks_per_doc, int32_t k, msa_dtype dt,
                            int32_t* topk_ids, float* topk_scores, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * S4  Gather of the selected documents' pooled K/V ("Inference Pipeline",
 *     stage 2: load only the selected pooled K/V; the content tier may live
 *     in host DRAM and be fetched when selected).
 *
 *   k_sel[b, i*C + j] = kbar[topk_ids[b,i]*C + j]   (and v_sel from vbar)
 *
 * kbar, vbar   [n_docs*C, heads_kv, dim] (dtype dt).  With src_on_host = 0
 *              they are device pointers; with src_on_host = 1 they point to
 *              pinned host memory (hipHostMalloc / torch pin_memory), which
 *              the GPU reads directly over the host link (no host round
 *              trip), or, with MSA_GATHER_HOST_MEMCPY, which is copied per
 *              selected document with hipMemcpyAsync on a library side stream
 *              after the ids are read back.  In that mode the call records an
 *              event on `stream`, copies the ids to the host on the side
 *              stream once that event has passed, and blocks until they
 *              arrive: it waits for the work queued on `stream` before the
 *              call, nothing later and no other stream (so work queued on
 *              another stream beforehand, e.g. the next routing, keeps the
 *              GPU busy during the wait and the copies).  `stream` then waits
 *              on the copies.
 * topk_ids     [batch, k] int32 device pointer
 * k_sel, v_sel [batch, k*C, heads_kv, dim] device outputs
 * flags        0 or MSA_GATHER_CHECKED | MSA_GATHER_HOST_MEMCPY.
 * Ids outside [0, n_docs) never cause an out-of-bounds read: their rows are
 * written as zeros.  With MSA_GATHER_CHECKED the call waits for `stream` up
 * to its own gather and returns MSA_ERR_INVALID if any id was out of range
 * (each call has its own error word).  In MSA_GATHER_HOST_MEMCPY mode an id
 * out of range returns MSA_ERR_INVALID before any copy is enqueued.  Requires
 * n_docs*chunks_per_doc rows in kbar and vbar; the library cannot see their
 * length, so the caller guarantees it.
 * ---------------------------------------------------------------------- */
msa_status msa_gather_kv(const void* kbar, const void* vbar, int32_t src_on_host,
                         const int32_t* topk_ids, int32_t batch, int32_t k, int64_t n_docs,
                         int32_t chunks_per_doc, int32_t heads_kv, int32_t dim, msa_dtype dt,
                         void* k_sel, void* v_sel, int32_t flags, void* stream);

/* ------------------------------------------------------------------------
 * S5/S6  Sparse GQA attention (model card "Architecture summary": in the
 *     softmax layers the top-k chunks' K/V are concatenated with the local
 *     KV; README "Inference Pipeline", stage 3: generate over that context).
 *
 * For sequence b, query token t, query head h, KV head g = h / (heads_q/heads_kv):
 *   keys  = [k_sel[b, 0..mem_len-1, g] ; k_loc[b, 0 .. loc_len-q_len+t, g]]
 *   o[b,t,h] = softmax(scale * q[b,t,h] . keys^T) . values
 * (bottom-right causal alignment: the last query token sees all local rows;
 * memory rows are visible to every token).  lse[b,h,t] = log-sum-exp of the
 * scaled logits (natural log), for combining partial attentions.
 *
 * q            [batch, q_len, heads_q, dim]
 * k_sel, v_sel [batch, mem_len, heads_kv, dim]  (may be NULL iff mem_len == 0)
 * k_loc, v_loc [batch, loc_len, heads_kv, dim]  (loc_len >= q_len >= 1)
 * out          [batch, q_len, heads_q, dim] output (dtype dt)
 * lse          [batch, heads_q, q_len] float32 output, or NULL
 * ws           msa_sparse_attn_workspace() bytes (split-KV partials for decode)
 * Requires heads_q % heads_kv == 0.  scale is typically 1/sqrt(dim).
 * ---------------------------------------------------------------------- */
msa_status msa_sparse_attn_workspace(int32_t batch, int32_t q_len, int32_t heads_q,
                                     int32_t heads_kv, int32_t dim, int32_t mem_len,
                                     int32_t loc_len, msa_dtype dt, size_t* bytes);
msa_status msa_sparse_attn(const void* q, const void* k_sel, const void* v_sel, int32_t mem_len,
                           const void* k_loc, const void* v_loc, int32_t loc_len, int32_t batch,
                           int32_t q_len, int32_t heads_q, int32_t heads_kv, int32_t dim,
                           float scale, msa_dtype dt, void* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Merge of two partial attentions over disjoint key sets (the attention of
 *     S5/S6 runs over [selected memory rows ; local rows], model card
 *     "Architecture summary" and README "Inference Pipeline" stage 3; a
 *     softmax over a union of disjoint key sets is the log-sum-exp weighted
 *     sum of the softmaxes over each set).
 *
 * For every (b, t, h), with la = lse_a[b,h,t], lb = lse_b[b,h,t]:
 *   lse[b,h,t] = log(exp(la) + exp(lb))
 *   out[b,t,h] = exp(la - lse) out_a[b,t,h] + exp(lb - lse) out_b[b,t,h]
 * A part with lse -inf (no visible key) has weight 0; with both at -inf,
 * out is 0 and lse is -inf.  Use: a decode step's local rows do not depend
 * on routing, so msa_sparse_attn over them (mem_len = 0) can run on a second
 * stream beside route, top-k and gather; the selected memory rows' attention
 * follows the gather, and this call combines the two.  (With q_len = 1 the
 * memory rows may be passed as the local rows of a call with mem_len = 0:
 * the one token sees every local row.)
 *
 * out_a, out_b, out  [batch, q_len, heads_q, dim]  dtype dt, 16-byte aligned
 * lse_a, lse_b       [batch, heads_q, q_len]  float32 (natural log)
 * lse                [batch, heads_q, q_len]  float32 output, or NULL
 * out may alias out_a or out_b, lse may alias lse_a or lse_b.  No workspace.
 * ---------------------------------------------------------------------- */
msa_status msa_attn_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b,
                          int32_t batch, int32_t q_len, int32_t heads_q, int32_t dim, msa_dtype dt, void* out,
                          float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the sparse attention (MSA README "Abstract" and Figure 1
 *     caption: top-k selection fused with a sparse attention that stays
 *     end-to-end differentiable; model card "Training (CPT)": the router and
 *     adapters train through the routed layers).
 *
 * Given the forward's inputs, its output `out` and log-sum-exp `lse` (from
 * msa_sparse_attn with the same scale), and d_out = dL/d out, writes
 *   d_q    [batch, q_len, heads_q, dim]
 *   d_k_sel, d_v_sel [batch, mem_len, heads_kv, dim]   (NULL iff mem_len == 0)
 *   d_k_loc, d_v_loc [batch, loc_len, heads_kv, dim]
 * all in dtype dt (float32 accumulation).  With P the forward's softmax over
 * the visible keys and D_t = sum_d d_out[t,d] * out[t,d]:
 *   dP = d_out V^T,  dS = P o (dP - D),  d_q = scale dS K,
 *   d_k = scale dS^T Q,  d_v = P^T d_out,
 * a KV head's gradients summing over its query heads and the tokens that see
 * it.  Rows no token sees get zero gradients.  ws: msa_sparse_attn_backward_
 * workspace() bytes (D per query row).  Deterministic (no atomics).
 * ---------------------------------------------------------------------- */
msa_status msa_sparse_attn_backward_workspace(int32_t batch, int32_t q_len, int32_t heads_q,
                                              int32_t heads_kv, int32_t dim, int32_t mem_len,
                                              int32_t loc_len, msa_dtype dt, size_t* bytes);
msa_status msa_sparse_attn_backward(const void* q, const void* k_sel, const void* v_sel, int32_t mem_len,
                                    const void* k_loc, const void* v_loc, int32_t loc_len, const void* out,
                                    const void* d_out, const float* lse, int32_t batch, int32_t q_len,
                                    int32_t heads_q, int32_t heads_kv, int32_t dim, float scale,
                                    msa_dtype dt, void* d_q, void* d_k_sel, void* d_v_sel, void* d_k_loc,
                                    void* d_v_loc, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Linear-layer variant (model card "Architecture summary": in the linear
 *     gated-delta layers each document is encoded through the layer's
 *     recurrence, the routed top-k documents' recurrent states are summed
 *     into S_ext, and the query path runs the gated delta rule with S_ext as
 *     its initial state).  Routing is msa_route_scores / msa_topk_docs.
 *
 * msa_gdn_state_sum: s_ext[b] = sum_{i<k} doc_states[topk_ids[b,i]], in rank
 *   order.  doc_states [n_docs, heads, dk, dv] float32; s_ext [batch, heads,
 *   dk, dv] float32; ids outside [0, n_docs) contribute nothing.
 *
 * msa_gated_delta_rule: per (sequence b, head h), state S[dk][dv] starting at
 *   initial_state[b,h] (or zeros when NULL), for each token t in order:
 *       S <- exp(g[b,t,h]) * S
 *       u  = S^T k[b,t,h]
 *       S <- S + k[b,t,h] (beta[b,t,h] * (v[b,t,h] - u))^T
 *       out[b,t,h] = scale * S^T q[b,t,h]
 *   (the published gated delta rule; the pages name it without equations).
 *   q, k [batch, seq_len, heads, dk]; v, out [batch, seq_len, heads, dv]
 *   (dtype dt); g (log decay), beta [batch, seq_len, heads] float32;
 *   initial_state, final_state [batch, heads, dk, dv] float32.  out or
 *   final_state may be NULL (not both); q may be NULL when out is NULL (the
 *   offline document encoding: final states only).  dk is 64 or 128.
 *   Keys are used as given (normalise them first if the model does).
 * ---------------------------------------------------------------------- */
msa_status msa_gdn_state_sum(const float* doc_states, const int32_t* topk_ids, int32_t batch, int32_t k,
                             int64_t n_docs, int32_t heads, int32_t dk, int32_t dv, float* s_ext, void* stream);
msa_status msa_gated_delta_rule(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                float scale, const float* initial_state, int32_t batch, int32_t seq_len,
                                int32_t heads, int32_t dk, int32_t dv, msa_dtype dt, void* out,
                                float* final_state, void* stream);

/* ------------------------------------------------------------------------
 * The same rule in its chunked form (model card "Architecture summary": the
 *     linear layers run the chunked gated delta rule, from the injected
 *     state on the query side; the offline document encoding uses it too).
 *
 * Same arguments and result as msa_gated_delta_rule, computed 32 tokens at a
 * time: inside a chunk the delta-rule writes solve a unit lower-triangular
 * system (I + A) D = R, with A[t][j] = beta_t exp(G_t - G_j) (k_t . k_j)
 * for j < t (G the running sum of g inside the chunk) and
 * R = beta o (V - exp(G) o K S0); then S_C = exp(G_C) S0 + K^T (exp(G_C - G) o D)
 * and O = scale (exp(G) o Q S0 + (M o Q K^T) D), M[t][j] = exp(G_t - G_j)
 * for j <= t.  The contractions run on bf16 MFMA with float32 operands
 * split into two bf16 terms, so the result agrees with the token-by-token
 * form to about 1e-5 of the state's scale, not bit for bit.
 *
 * Supported: dt = MSA_BF16, dk = dv = 128, and one sequence's rows
 * (seq_len * heads * 256 bytes) spanning less than 4 GiB (other shapes return
 * MSA_ERR_INVALID; msa_gated_delta_rule covers them).  q and k 16-byte
 * aligned.  One workgroup per (sequence, head); no workspace.
 * ---------------------------------------------------------------------- */
msa_status msa_gated_delta_rule_chunked(const void* q, const void* k, const void* v, const float* g,
                                        const float* beta, float scale, const float* initial_state,
                                        int32_t batch, int32_t seq_len, int32_t heads, int32_t dk, int32_t dv,
                                        msa_dtype dt, void* out, float* final_state, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
