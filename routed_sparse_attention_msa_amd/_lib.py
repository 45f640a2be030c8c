"""ctypes binding of libmsa (include/msa.h).

Argument marshalling only: each function checks device, dtype, shape and
contiguity of the torch tensors it is given, allocates missing outputs and
workspace with torch, and calls the C entry point of the same name on the
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no CPU path, and a missing library is an ImportError.
"""

import ctypes
import math
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK, MSA_ERR_INVALID, MSA_ERR_UNSUPPORTED, MSA_ERR_HIP = 0, 1, 2, 3
MSA_F32, MSA_BF16 = 0, 1
MSA_GATHER_CHECKED = 1
MSA_GATHER_HOST_MEMCPY = 2
(MSA_OP_POOL_CHUNKS, MSA_OP_ROUTE_SCORES, MSA_OP_TOPK_DOCS, MSA_OP_GATHER_KV, MSA_OP_SPARSE_ATTN,
 MSA_OP_SPARSE_ATTN_BACKWARD, MSA_OP_ROUTE_ROUNDS, MSA_OP_TOPK_DOCS_EXCLUDING, MSA_OP_ENCODE_DOCS,
 MSA_OP_GDN_STATE_SUM, MSA_OP_GATED_DELTA_RULE, MSA_OP_GATED_DELTA_RULE_CHUNKED) = range(12)

# Every entry point declared in include/msa.h: name -> (restype, argtypes).
_STATUS = c_int
SIGNATURES = {
    "msa_abi_version": (c_int, []),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_workspace_size": (_STATUS, [c_int32, POINTER(c_int64), c_int32, POINTER(c_size_t)]),
    "msa_pool_chunks": (_STATUS, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_int32, c_int32,
                                  c_int32, c_int, c_void_p]),
    "msa_chunk_offsets": (_STATUS, [c_void_p, c_int64, c_int32, c_void_p, c_void_p]),
    "msa_encode_docs": (_STATUS, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                  c_int64, c_int32, c_int32, c_int32, c_float, c_int, c_void_p]),
    "msa_route_scores_workspace": (_STATUS, [c_int32, c_int32, c_int32, c_int32, c_int64, c_int32,
                                             c_int, POINTER(c_size_t)]),
    "msa_route_scores": (_STATUS, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                   c_int64, c_int32, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "msa_route_scores_noalloc": (_STATUS, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                           c_int64, c_int32, c_int, c_void_p, c_void_p]),
    "msa_topk_docs_workspace": (_STATUS, [c_int32, c_int64, c_int32, POINTER(c_size_t)]),
    "msa_topk_docs": (_STATUS, [c_void_p, c_int32, c_int64, c_int32, c_void_p, c_void_p, c_void_p,
                                c_size_t, c_void_p]),
    "msa_topk_docs_excluding": (_STATUS, [c_void_p, c_int32, c_int64, c_int32, c_void_p, c_int32, c_int64,
                                          c_void_p, c_void_p, c_int64, c_void_p, c_size_t, c_void_p]),
    "msa_route_rounds_workspace": (_STATUS, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int64, c_int32,
                                             c_int32, c_int, POINTER(c_size_t)]),
    "msa_route_rounds": (_STATUS, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                   c_int64, c_int32, c_int32, c_int, c_void_p, c_void_p, c_void_p, c_size_t,
                                   c_void_p]),
    "msa_gather_kv": (_STATUS, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int64,
                                c_int32, c_int32, c_int32, c_int, c_void_p, c_void_p, c_int32,
                                c_void_p]),
    "msa_sparse_attn_workspace": (_STATUS, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                            c_int32, c_int, POINTER(c_size_t)]),
    "msa_sparse_attn": (_STATUS, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                  c_int32, c_int32, c_int32, c_int32, c_int32, c_float, c_int,
                                  c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "msa_attn_merge": (_STATUS, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                 c_int, c_void_p, c_void_p, c_void_p]),
    "msa_sparse_attn_backward_workspace": (_STATUS, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                                     c_int32, c_int, POINTER(c_size_t)]),
    "msa_sparse_attn_backward": (_STATUS, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                           c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                           c_int32, c_float, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_size_t, c_void_p]),
    "msa_gdn_state_sum": (_STATUS, [c_void_p, c_void_p, c_int32, c_int32, c_int64, c_int32, c_int32, c_int32,
                                    c_void_p, c_void_p]),
    "msa_gated_delta_rule": (_STATUS, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_int32,
                                       c_int32, c_int32, c_int32, c_int32, c_int, c_void_p, c_void_p, c_void_p]),
    "msa_gated_delta_rule_chunked": (_STATUS, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p,
                                               c_int32, c_int32, c_int32, c_int32, c_int32, c_int, c_void_p,
                                               c_void_p, c_void_p]),
}


class MsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libmsa status {status}: {message}")
        self.status = status


_lib = None


def lib():
    """Load libmsa.so (built in-tree by ``python -m routed_sparse_attention_msa_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m routed_sparse_attention_msa_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status):
    if status != MSA_OK:
        raise MsaError(status, lib().msa_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return MSA_F32
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _dev(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the HIP path has no CPU fallback)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elif ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {nbytes}")
    return ws, ws.numel() * ws.element_size()


def msa_workspace_size(op, dims):
    """Workspace bytes of operation ``op`` (an MSA_OP_* code) for the integer
    arguments ``dims`` of its *_workspace call (the dtype as its MSA_* code)."""
    arr = (c_int64 * max(1, len(dims)))(*[int(d) for d in dims])
    n = c_size_t(0)
    _check(lib().msa_workspace_size(int(op), arr, len(dims), ctypes.byref(n)))
    return n.value


# ---------------------------------------------------------------------------
# S1
# ---------------------------------------------------------------------------

def msa_pool_chunks(x, chunk, xbar=None, xbar_norm=None, with_norm=False):
    """Chunk-mean pool ``x`` [n_docs, doc_len, heads, dim] -> (xbar [n_docs*C, heads, dim],
    xbar_norm [n_docs*C, heads] float32 or None)."""
    _dev(x, "x", ndim=4)
    n_docs, doc_len, heads, dim = x.shape
    if doc_len % chunk:
        raise ValueError("doc_len must be a multiple of chunk")
    n_ch = n_docs * (doc_len // chunk)
    if xbar is None:
        xbar = torch.empty((n_ch, heads, dim), dtype=x.dtype, device=x.device)
    _dev(xbar, "xbar", dtype=x.dtype)
    if xbar.shape != (n_ch, heads, dim):
        raise ValueError(f"xbar must be {(n_ch, heads, dim)}")
    if with_norm and xbar_norm is None:
        xbar_norm = torch.empty((n_ch, heads), dtype=torch.float32, device=x.device)
    if xbar_norm is not None:
        _dev(xbar_norm, "xbar_norm", dtype=torch.float32)
        if xbar_norm.shape != (n_ch, heads):
            raise ValueError(f"xbar_norm must be {(n_ch, heads)}")
    _check(lib().msa_pool_chunks(_ptr(x), _ptr(xbar), _ptr(xbar_norm), n_docs, doc_len, chunk, heads,
                                 dim, _dtype_code(x), _stream(x.device)))
    return xbar, xbar_norm


def msa_chunk_offsets(doc_off, chunk, chunk_off=None):
    """First pooled chunk of each document (device int64 [n_docs + 1]) from the
    document row offsets ``doc_off`` (device int64 [n_docs + 1])."""
    _dev(doc_off, "doc_off", dtype=torch.int64, ndim=1)
    n_docs = doc_off.numel() - 1
    if n_docs < 0:
        raise ValueError("doc_off needs n_docs + 1 >= 1 entries")
    if chunk_off is None:
        chunk_off = torch.empty_like(doc_off)
    _dev(chunk_off, "chunk_off", dtype=torch.int64, ndim=1)
    if chunk_off.numel() != n_docs + 1:
        raise ValueError("chunk_off must have n_docs + 1 entries")
    _check(lib().msa_chunk_offsets(_ptr(doc_off), n_docs, chunk, _ptr(chunk_off), _stream(doc_off.device)))
    return chunk_off


def msa_encode_docs(x, doc_off, chunk_off, total_chunks, chunk, rope_base=0.0, xbar=None,
                    xbar_norm=None, with_norm=False):
    """Chunk means of variable-length documents: ``x`` [total_rows, heads, dim]
    with document n at rows doc_off[n] .. doc_off[n+1]-1, optionally rotated by
    document-wise RoPE (``rope_base`` > 0) first.  ``total_chunks`` must equal
    chunk_off[-1] (known on the host from the document lengths).  Returns
    (xbar [total_chunks, heads, dim], xbar_norm [total_chunks, heads] or None)."""
    _dev(x, "x", ndim=3)
    _dev(doc_off, "doc_off", dtype=torch.int64, ndim=1)
    _dev(chunk_off, "chunk_off", dtype=torch.int64, ndim=1)
    total_rows, heads, dim = x.shape
    n_docs = doc_off.numel() - 1
    if chunk_off.numel() != n_docs + 1:
        raise ValueError("chunk_off must have as many entries as doc_off")
    if xbar is None:
        xbar = torch.empty((total_chunks, heads, dim), dtype=x.dtype, device=x.device)
    _dev(xbar, "xbar", dtype=x.dtype)
    if xbar.shape != (total_chunks, heads, dim):
        raise ValueError(f"xbar must be {(total_chunks, heads, dim)}")
    if with_norm and xbar_norm is None:
        xbar_norm = torch.empty((total_chunks, heads), dtype=torch.float32, device=x.device)
    if xbar_norm is not None:
        _dev(xbar_norm, "xbar_norm", dtype=torch.float32)
        if xbar_norm.shape != (total_chunks, heads):
            raise ValueError(f"xbar_norm must be {(total_chunks, heads)}")
    _check(lib().msa_encode_docs(_ptr(x), _ptr(xbar), _ptr(xbar_norm), _ptr(doc_off), _ptr(chunk_off),
                                 n_docs, total_rows, total_chunks, chunk, heads, dim, float(rope_base),
                                 _dtype_code(x), _stream(x.device)))
    return xbar, xbar_norm


# ---------------------------------------------------------------------------
# S2
# ---------------------------------------------------------------------------

def msa_route_scores_workspace(batch, q_len, heads, dim, n_docs, chunks_per_doc, dtype):
    n = c_size_t(0)
    code = MSA_F32 if dtype == torch.float32 else MSA_BF16
    _check(lib().msa_route_scores_workspace(batch, q_len, heads, dim, n_docs, chunks_per_doc, code,
                                            ctypes.byref(n)))
    return n.value


def msa_route_scores(q_r, kbar_r, kbar_r_norm, chunks_per_doc, doc_scores=None, ws=None):
    """Routing scores [batch, n_docs] float32 of router queries ``q_r`` [batch, q_len, heads, dim]
    against the pooled router keys ``kbar_r`` [n_docs*C, heads, dim] and their norms."""
    _dev(q_r, "q_r", ndim=4)
    _dev(kbar_r, "kbar_r", dtype=q_r.dtype, ndim=3)
    _dev(kbar_r_norm, "kbar_r_norm", dtype=torch.float32, ndim=2)
    batch, q_len, heads, dim = q_r.shape
    n_ch = kbar_r.shape[0]
    if kbar_r.shape[1:] != (heads, dim) or kbar_r_norm.shape != (n_ch, heads):
        raise ValueError("router query, pooled keys and norms disagree in shape")
    if n_ch % chunks_per_doc:
        raise ValueError("chunk count is not a multiple of chunks_per_doc")
    n_docs = n_ch // chunks_per_doc
    if doc_scores is None:
        doc_scores = torch.empty((batch, n_docs), dtype=torch.float32, device=q_r.device)
    _dev(doc_scores, "doc_scores", dtype=torch.float32)
    _shape(doc_scores, "doc_scores", (batch, n_docs))
    nbytes = msa_route_scores_workspace(batch, q_len, heads, dim, n_docs, chunks_per_doc, q_r.dtype)
    ws, ws_bytes = _workspace(nbytes, q_r.device, ws)
    _check(lib().msa_route_scores(_ptr(q_r), _ptr(kbar_r), _ptr(kbar_r_norm), batch, q_len, heads, dim,
                                  n_docs, chunks_per_doc, _dtype_code(q_r), _ptr(doc_scores), _ptr(ws),
                                  ws_bytes, _stream(q_r.device)))
    return doc_scores


# ---------------------------------------------------------------------------
# S3
# ---------------------------------------------------------------------------

def msa_topk_docs_workspace(batch, n_docs, k):
    n = c_size_t(0)
    _check(lib().msa_topk_docs_workspace(batch, n_docs, k, ctypes.byref(n)))
    return n.value


def msa_topk_docs(doc_scores, k, topk_ids=None, topk_scores=None, with_scores=True, ws=None):
    """Top-k document ids [batch, k] int32 (and scores) of ``doc_scores`` [batch, n_docs]."""
    _dev(doc_scores, "doc_scores", dtype=torch.float32, ndim=2)
    batch, n_docs = doc_scores.shape
    if topk_ids is None:
        topk_ids = torch.empty((batch, k), dtype=torch.int32, device=doc_scores.device)
    _dev(topk_ids, "topk_ids", dtype=torch.int32)
    _shape(topk_ids, "topk_ids", (batch, k))
    if with_scores and topk_scores is None:
        topk_scores = torch.empty((batch, k), dtype=torch.float32, device=doc_scores.device)
    if topk_scores is not None:
        _dev(topk_scores, "topk_scores", dtype=torch.float32)
        _shape(topk_scores, "topk_scores", (batch, k))
    ws, ws_bytes = _workspace(msa_topk_docs_workspace(batch, n_docs, k), doc_scores.device, ws)
    _check(lib().msa_topk_docs(_ptr(doc_scores), batch, n_docs, k, _ptr(topk_ids), _ptr(topk_scores),
                               _ptr(ws), ws_bytes, _stream(doc_scores.device)))
    return topk_ids, topk_scores


# ---------------------------------------------------------------------------
# Multi-round routing (Memory Interleave)
# ---------------------------------------------------------------------------

def msa_topk_docs_excluding(doc_scores, k, excl_ids, topk_ids=None, topk_scores=None, with_scores=True,
                            ws=None):
    """Top-k document ids [batch, k] int32 (and scores) of ``doc_scores`` [batch, n_docs] among the
    documents not listed in ``excl_ids`` [batch, n_excl] int32 (ids outside [0, n_docs) ignored)."""
    _dev(doc_scores, "doc_scores", dtype=torch.float32, ndim=2)
    _dev(excl_ids, "excl_ids", dtype=torch.int32, ndim=2)
    batch, n_docs = doc_scores.shape
    if excl_ids.shape[0] != batch:
        raise ValueError("excl_ids must have one row per sequence")
    n_excl = excl_ids.shape[1]
    if topk_ids is None:
        topk_ids = torch.empty((batch, k), dtype=torch.int32, device=doc_scores.device)
    _dev(topk_ids, "topk_ids", dtype=torch.int32)
    if topk_ids.shape != (batch, k):
        raise ValueError("topk_ids must be [batch, k]")
    if with_scores and topk_scores is None:
        topk_scores = torch.empty((batch, k), dtype=torch.float32, device=doc_scores.device)
    if topk_scores is not None:
        _dev(topk_scores, "topk_scores", dtype=torch.float32)
        if topk_scores.shape != (batch, k):
            raise ValueError("topk_scores must be [batch, k]")
    ws, ws_bytes = _workspace(msa_topk_docs_workspace(batch, n_docs, k), doc_scores.device, ws)
    _check(lib().msa_topk_docs_excluding(_ptr(doc_scores), batch, n_docs, k, _ptr(excl_ids), n_excl, n_excl,
                                         _ptr(topk_ids), _ptr(topk_scores), k, _ptr(ws), ws_bytes,
                                         _stream(doc_scores.device)))
    return topk_ids, topk_scores


def msa_route_rounds_workspace(rounds, batch, q_len, heads, dim, n_docs, chunks_per_doc, k, dtype):
    n = c_size_t(0)
    code = MSA_F32 if dtype == torch.float32 else MSA_BF16
    _check(lib().msa_route_rounds_workspace(rounds, batch, q_len, heads, dim, n_docs, chunks_per_doc, k, code,
                                            ctypes.byref(n)))
    return n.value


def msa_route_rounds(q_r, kbar_r, kbar_r_norm, chunks_per_doc, k, topk_ids=None, topk_scores=None,
                     with_scores=True, ws=None):
    """Multi-round routing: ``q_r`` [rounds, batch, q_len, heads, dim] holds one router query per
    round; round r routes its query and keeps the top-k documents no earlier round selected.
    Returns ids [batch, rounds*k] int32 (round r in columns [r*k, (r+1)*k)) and their scores."""
    _dev(q_r, "q_r", ndim=5)
    _dev(kbar_r, "kbar_r", dtype=q_r.dtype, ndim=3)
    _dev(kbar_r_norm, "kbar_r_norm", dtype=torch.float32, ndim=2)
    rounds, batch, q_len, heads, dim = q_r.shape
    n_ch = kbar_r.shape[0]
    if kbar_r.shape[1:] != (heads, dim) or kbar_r_norm.shape != (n_ch, heads):
        raise ValueError("router queries, pooled keys and norms disagree in shape")
    if n_ch % chunks_per_doc:
        raise ValueError("chunk count is not a multiple of chunks_per_doc")
    n_docs = n_ch // chunks_per_doc
    dev = q_r.device
    if topk_ids is None:
        topk_ids = torch.empty((batch, rounds * k), dtype=torch.int32, device=dev)
    _dev(topk_ids, "topk_ids", dtype=torch.int32)
    if topk_ids.shape != (batch, rounds * k):
        raise ValueError("topk_ids must be [batch, rounds*k]")
    if with_scores and topk_scores is None:
        topk_scores = torch.empty((batch, rounds * k), dtype=torch.float32, device=dev)
    if topk_scores is not None:
        _dev(topk_scores, "topk_scores", dtype=torch.float32)
        if topk_scores.shape != (batch, rounds * k):
            raise ValueError("topk_scores must be [batch, rounds*k]")
    nbytes = msa_route_rounds_workspace(rounds, batch, q_len, heads, dim, n_docs, chunks_per_doc, k, q_r.dtype)
    ws, ws_bytes = _workspace(nbytes, dev, ws)
    _check(lib().msa_route_rounds(_ptr(q_r), _ptr(kbar_r), _ptr(kbar_r_norm), rounds, batch, q_len, heads, dim,
                                  n_docs, chunks_per_doc, k, _dtype_code(q_r), _ptr(topk_ids), _ptr(topk_scores),
                                  _ptr(ws), ws_bytes, _stream(dev)))
    return topk_ids, topk_scores


# ---------------------------------------------------------------------------
# S4
# ---------------------------------------------------------------------------

def msa_gather_kv(kbar, vbar, topk_ids, chunks_per_doc, k_sel=None, v_sel=None, checked=False,
                  host_memcpy=False):
    """Gather the selected documents' pooled K/V -> (k_sel, v_sel) [batch, k*C, heads_kv, dim].

    ``kbar``/``vbar`` [n_docs*C, heads_kv, dim] are GPU tensors, or pinned CPU
    tensors (host tier: read by the GPU over the host link, or copied per
    document with ``host_memcpy=True``)."""
    on_host = not kbar.is_cuda
    for name, t in (("kbar", kbar), ("vbar", vbar)):
        if on_host:
            if not t.is_pinned():
                raise ValueError(f"{name} on the host must be pinned memory")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        else:
            _dev(t, name, ndim=3)
    if vbar.dtype != kbar.dtype or vbar.shape != kbar.shape or vbar.is_cuda != kbar.is_cuda:
        raise ValueError("kbar and vbar must match")
    _dev(topk_ids, "topk_ids", dtype=torch.int32, ndim=2)
    if kbar.dim() != 3:
        raise ValueError(f"kbar must be [n_docs*C, heads_kv, dim], got {tuple(kbar.shape)}")
    n_ch, heads_kv, dim = kbar.shape
    batch, k = topk_ids.shape
    if chunks_per_doc <= 0 or n_ch % chunks_per_doc:
        raise ValueError(f"the bank's {n_ch} rows are not a whole number of {chunks_per_doc}-chunk documents")
    n_docs = n_ch // chunks_per_doc
    shape = (batch, k * chunks_per_doc, heads_kv, dim)
    dev = topk_ids.device
    if k_sel is None:
        k_sel = torch.empty(shape, dtype=kbar.dtype, device=dev)
    if v_sel is None:
        v_sel = torch.empty(shape, dtype=kbar.dtype, device=dev)
    _dev(k_sel, "k_sel", dtype=kbar.dtype)
    _dev(v_sel, "v_sel", dtype=kbar.dtype)
    _shape(k_sel, "k_sel", shape)
    _shape(v_sel, "v_sel", shape)
    flags = (MSA_GATHER_CHECKED if checked else 0) | (MSA_GATHER_HOST_MEMCPY if host_memcpy else 0)
    _check(lib().msa_gather_kv(_ptr(kbar), _ptr(vbar), 1 if on_host else 0, _ptr(topk_ids), batch, k,
                               n_docs, chunks_per_doc, heads_kv, dim, _dtype_code(kbar), _ptr(k_sel),
                               _ptr(v_sel), flags, _stream(dev)))
    return k_sel, v_sel


# ---------------------------------------------------------------------------
# S5 / S6
# ---------------------------------------------------------------------------

def msa_sparse_attn_workspace(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dtype):
    n = c_size_t(0)
    code = MSA_F32 if dtype == torch.float32 else MSA_BF16
    _check(lib().msa_sparse_attn_workspace(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, code,
                                           ctypes.byref(n)))
    return n.value


def msa_sparse_attn(q, k_sel, v_sel, k_loc, v_loc, scale=None, out=None, lse=None, with_lse=True,
                    ws=None):
    """Sparse GQA attention of ``q`` [batch, q_len, heads_q, dim] over
    [k_sel/v_sel [batch, mem_len, heads_kv, dim] ; causal k_loc/v_loc [batch, loc_len, heads_kv, dim]]
    -> (out [batch, q_len, heads_q, dim], lse [batch, heads_q, q_len] float32 or None)."""
    _dev(q, "q", ndim=4)
    _dev(k_loc, "k_loc", dtype=q.dtype, ndim=4)
    _dev(v_loc, "v_loc", dtype=q.dtype, ndim=4)
    batch, q_len, heads_q, dim = q.shape
    loc_len, heads_kv = k_loc.shape[1], k_loc.shape[2]
    if k_sel is None:
        mem_len = 0
    else:
        _dev(k_sel, "k_sel", dtype=q.dtype, ndim=4)
        _dev(v_sel, "v_sel", dtype=q.dtype, ndim=4)
        mem_len = k_sel.shape[1]
        if k_sel.shape != (batch, mem_len, heads_kv, dim) or v_sel.shape != k_sel.shape:
            raise ValueError("k_sel/v_sel shape mismatch")
    if k_loc.shape != (batch, loc_len, heads_kv, dim) or v_loc.shape != k_loc.shape:
        raise ValueError("k_loc/v_loc shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", dtype=q.dtype)
    _shape(out, "out", q.shape)
    if with_lse and lse is None:
        lse = torch.empty((batch, heads_q, q_len), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32)
        _shape(lse, "lse", (batch, heads_q, q_len))
    nbytes = msa_sparse_attn_workspace(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, q.dtype)
    ws, ws_bytes = _workspace(nbytes, q.device, ws)
    _check(lib().msa_sparse_attn(_ptr(q), _ptr(k_sel), _ptr(v_sel), mem_len, _ptr(k_loc), _ptr(v_loc),
                                 loc_len, batch, q_len, heads_q, heads_kv, dim, float(scale),
                                 _dtype_code(q), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                 _stream(q.device)))
    return out, lse


def msa_attn_merge(out_a, lse_a, out_b, lse_b, out=None, lse=None, with_lse=True):
    """Log-sum-exp merge of two partial attentions over disjoint key sets:
    ``out_*`` [batch, q_len, heads_q, dim], ``lse_*`` [batch, heads_q, q_len] float32
    -> (out, lse or None).  ``out`` may be ``out_a`` or ``out_b`` and ``lse`` may be
    ``lse_a`` or ``lse_b`` (in place)."""
    _dev(out_a, "out_a", ndim=4)
    _dev(out_b, "out_b", dtype=out_a.dtype)
    _shape(out_b, "out_b", out_a.shape)
    batch, q_len, heads_q, dim = out_a.shape
    for t, name in ((lse_a, "lse_a"), (lse_b, "lse_b")):
        _dev(t, name, dtype=torch.float32)
        _shape(t, name, (batch, heads_q, q_len))
    if out is None:
        out = torch.empty_like(out_a)
    _dev(out, "out", dtype=out_a.dtype)
    _shape(out, "out", out_a.shape)
    if with_lse and lse is None:
        lse = torch.empty_like(lse_a)
    if lse is not None:
        _dev(lse, "lse", dtype=torch.float32)
        _shape(lse, "lse", (batch, heads_q, q_len))
    _check(lib().msa_attn_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), batch, q_len, heads_q, dim,
                                _dtype_code(out_a), _ptr(out), _ptr(lse), _stream(out_a.device)))
    return out, lse


def msa_sparse_attn_backward_workspace(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, dtype):
    n = c_size_t(0)
    code = MSA_F32 if dtype == torch.float32 else MSA_BF16
    _check(lib().msa_sparse_attn_backward_workspace(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len,
                                                    code, ctypes.byref(n)))
    return n.value


def msa_sparse_attn_backward(q, k_sel, v_sel, k_loc, v_loc, out, lse, d_out, scale=None, grads=None, ws=None):
    """Gradients of :func:`msa_sparse_attn` given its output ``out``, its ``lse`` (same scale) and
    ``d_out`` = dL/d out: returns (d_q, d_k_sel, d_v_sel, d_k_loc, d_v_loc), d_k_sel/d_v_sel None when
    there are no memory rows.  ``grads`` may hold preallocated outputs in that order."""
    _dev(q, "q", ndim=4)
    _dev(k_loc, "k_loc", dtype=q.dtype, ndim=4)
    _dev(v_loc, "v_loc", dtype=q.dtype, ndim=4)
    _dev(out, "out", dtype=q.dtype, ndim=4)
    _dev(d_out, "d_out", dtype=q.dtype, ndim=4)
    _dev(lse, "lse", dtype=torch.float32, ndim=3)
    batch, q_len, heads_q, dim = q.shape
    loc_len, heads_kv = k_loc.shape[1], k_loc.shape[2]
    if k_sel is None:
        mem_len = 0
    else:
        _dev(k_sel, "k_sel", dtype=q.dtype, ndim=4)
        _dev(v_sel, "v_sel", dtype=q.dtype, ndim=4)
        mem_len = k_sel.shape[1]
        if k_sel.shape != (batch, mem_len, heads_kv, dim) or v_sel.shape != k_sel.shape:
            raise ValueError("k_sel/v_sel shape mismatch")
    if k_loc.shape != (batch, loc_len, heads_kv, dim) or v_loc.shape != k_loc.shape:
        raise ValueError("k_loc/v_loc shape mismatch")
    if out.shape != q.shape or d_out.shape != q.shape or lse.shape != (batch, heads_q, q_len):
        raise ValueError("out, d_out and lse must match the query")
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if grads is None:
        grads = (torch.empty_like(q),
                 torch.empty_like(k_sel) if mem_len else None, torch.empty_like(v_sel) if mem_len else None,
                 torch.empty_like(k_loc), torch.empty_like(v_loc))
    d_q, d_ks, d_vs, d_kl, d_vl = grads
    for name, t, ref in (("d_q", d_q, q), ("d_k_loc", d_kl, k_loc), ("d_v_loc", d_vl, v_loc),
                         ("d_k_sel", d_ks, k_sel), ("d_v_sel", d_vs, v_sel)):
        if ref is None:
            continue
        _dev(t, name, dtype=q.dtype)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have shape {tuple(ref.shape)}")
    nbytes = msa_sparse_attn_backward_workspace(batch, q_len, heads_q, heads_kv, dim, mem_len, loc_len, q.dtype)
    ws, ws_bytes = _workspace(nbytes, q.device, ws)
    _check(lib().msa_sparse_attn_backward(_ptr(q), _ptr(k_sel), _ptr(v_sel), mem_len, _ptr(k_loc), _ptr(v_loc),
                                          loc_len, _ptr(out), _ptr(d_out), _ptr(lse), batch, q_len, heads_q,
                                          heads_kv, dim, float(scale), _dtype_code(q), _ptr(d_q), _ptr(d_ks),
                                          _ptr(d_vs), _ptr(d_kl), _ptr(d_vl), _ptr(ws), ws_bytes,
                                          _stream(q.device)))
    return d_q, d_ks, d_vs, d_kl, d_vl


# ---------------------------------------------------------------------------
# Linear-layer variant
# ---------------------------------------------------------------------------

def msa_gdn_state_sum(doc_states, topk_ids, s_ext=None):
    """S_ext [batch, heads, dk, dv] = sum of ``doc_states`` [n_docs, heads, dk, dv] (float32) over the
    documents in ``topk_ids`` [batch, k] (int32), in rank order."""
    _dev(doc_states, "doc_states", dtype=torch.float32, ndim=4)
    _dev(topk_ids, "topk_ids", dtype=torch.int32, ndim=2)
    n_docs, heads, dk, dv = doc_states.shape
    batch, k = topk_ids.shape
    if s_ext is None:
        s_ext = torch.empty((batch, heads, dk, dv), dtype=torch.float32, device=doc_states.device)
    _dev(s_ext, "s_ext", dtype=torch.float32)
    if s_ext.shape != (batch, heads, dk, dv):
        raise ValueError("s_ext must be [batch, heads, dk, dv]")
    _check(lib().msa_gdn_state_sum(_ptr(doc_states), _ptr(topk_ids), batch, k, n_docs, heads, dk, dv, _ptr(s_ext),
                                   _stream(doc_states.device)))
    return s_ext


def msa_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None, out=None, final_state=None,
                         with_out=True, with_final_state=True):
    """Gated delta rule over each sequence, token by token: q, k [batch, T, heads, dk]; v [batch, T, heads, dv];
    g (log decay), beta [batch, T, heads] float32; initial_state [batch, heads, dk, dv] float32 or None.
    Returns (out [batch, T, heads, dv] or None, final_state [batch, heads, dk, dv] float32 or None).
    ``q`` may be None when ``with_out`` is False (document encoding: final states only)."""
    return _gated_delta_rule("msa_gated_delta_rule", q, k, v, g, beta, scale, initial_state, out, final_state,
                             with_out, with_final_state)


def msa_gated_delta_rule_chunked(q, k, v, g, beta, scale=None, initial_state=None, out=None, final_state=None,
                                 with_out=True, with_final_state=True):
    """The same rule in its chunked form (32 tokens per chunk on MFMA); bf16, dk = dv = 128 only.
    Arguments and results as ``msa_gated_delta_rule``."""
    return _gated_delta_rule("msa_gated_delta_rule_chunked", q, k, v, g, beta, scale, initial_state, out,
                             final_state, with_out, with_final_state)


def _gated_delta_rule(name, q, k, v, g, beta, scale, initial_state, out, final_state, with_out, with_final_state):
    _dev(k, "k", ndim=4)
    _dev(v, "v", dtype=k.dtype, ndim=4)
    _dev(g, "g", dtype=torch.float32, ndim=3)
    _dev(beta, "beta", dtype=torch.float32, ndim=3)
    batch, seq_len, heads, dk = k.shape
    dv = v.shape[-1]
    if v.shape[:3] != (batch, seq_len, heads) or g.shape != (batch, seq_len, heads) or beta.shape != g.shape:
        raise ValueError("k, v, g and beta disagree in shape")
    if with_out:
        _dev(q, "q", dtype=k.dtype, ndim=4)
        if q.shape != k.shape:
            raise ValueError("q and k must have the same shape")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    if initial_state is not None:
        _dev(initial_state, "initial_state", dtype=torch.float32)
        if initial_state.shape != (batch, heads, dk, dv):
            raise ValueError("initial_state must be [batch, heads, dk, dv]")
    if with_out and out is None:
        out = torch.empty((batch, seq_len, heads, dv), dtype=k.dtype, device=k.device)
    if out is not None:
        _dev(out, "out", dtype=k.dtype)
        if out.shape != (batch, seq_len, heads, dv):
            raise ValueError("out must be [batch, T, heads, dv]")
    if with_final_state and final_state is None:
        final_state = torch.empty((batch, heads, dk, dv), dtype=torch.float32, device=k.device)
    if final_state is not None:
        _dev(final_state, "final_state", dtype=torch.float32)
        if final_state.shape != (batch, heads, dk, dv):
            raise ValueError("final_state must be [batch, heads, dk, dv]")
    _check(getattr(lib(), name)(_ptr(q) if with_out else None, _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                float(scale), _ptr(initial_state), batch, seq_len, heads, dk, dv,
                                _dtype_code(k), _ptr(out), _ptr(final_state), _stream(k.device)))
    return out, final_state
