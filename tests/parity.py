"""Comparators for GPU-vs-oracle parity (used by the gpu tests and smoke())."""

import numpy as np
import torch

from oracle.bf16 import f64_to_bf16_bits

# Tolerances.  Routing scores: 1e-3 absolute; attention: per-row relative L2
# 2e-2 for bf16 storage, 1e-4 for float32; the top-k band 1e-4 (a difference
# of scores inside the band may legitimately reorder the k-th place).
ROUTE_ATOL = 1e-3
ATTN_RTOL_BF16 = 2e-2
ATTN_RTOL_F32 = 1e-4
TOPK_BAND = 1e-4


def to_f64(t):
    """Exact float64 copy of a float32/bf16 tensor (bf16 and fp32 widen exactly)."""
    return t.detach().float().cpu().double().numpy()


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _ordered(bits):
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_ulp_distance(gpu_bf16, ref_f64):
    """Distance in bf16 ulps between a GPU bf16 tensor and float64 values rounded to bf16."""
    return np.abs(_ordered(bf16_bits(gpu_bf16)) - _ordered(f64_to_bf16_bits(ref_f64)))


def row_rel_l2(got, ref, axis=-1):
    num = np.sqrt(((got - ref) ** 2).sum(axis=axis))
    den = np.sqrt((ref ** 2).sum(axis=axis))
    return num / np.maximum(den, 1e-30)


def topk_band_check(gpu_ids, scores_ref, k, band=TOPK_BAND):
    """The GPU's k ids must be distinct and in range, contain every doc whose
    oracle score is >= tau + band, and only docs whose oracle score is > tau -
    band, where tau is the oracle's k-th best score.  Returns (ok, exact)."""
    gpu_ids = np.asarray(gpu_ids)
    ok = True
    exact = True
    for b in range(gpu_ids.shape[0]):
        s = scores_ref[b]
        ids = gpu_ids[b]
        if len(set(ids.tolist())) != k or ids.min() < 0 or ids.max() >= len(s):
            return False, False
        order = np.lexsort((np.arange(len(s)), -s))
        tau = s[order[k - 1]]
        must = set(np.nonzero(s >= tau + band)[0].tolist())
        may = set(np.nonzero(s > tau - band)[0].tolist())
        got = set(ids.tolist())
        ok &= must <= got <= may
        exact &= list(ids) == list(order[:k])
    return bool(ok), bool(exact)


def case(msg):
    """Print and flush the name of the case about to touch the GPU."""
    print(f"[case] {msg}", flush=True)
