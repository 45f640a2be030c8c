"""GPU parity of the offline encoder (document-wise RoPE + chunk means over
variable-length documents) and of the chunk-offset scan, against the oracle."""

import numpy as np
import pytest
import torch

import routed_sparse_attention_msa_amd as msa
from oracle import chunk_norms, chunk_offsets, encode_docs
from tests.parity import bf16_ulp_distance, case, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _docs(lens, heads, dim, dtype, seed, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    lens = np.asarray(lens, dtype=np.int64)
    doc_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = (torch.randn((int(doc_off[-1]), heads, dim), generator=g, device=DEV) * scale).to(dtype)
    return x, doc_off


def _check_rotated_bf16(xbar, exact, x_max, chunk):
    """Rotated rows are float32 products (not exact like sums of bf16 values),
    so a mean that cancels towards zero may land a few bf16 ulps from the
    float64 value.  Bound: one ulp of the exact mean plus the float32 error of
    the rotation and the sum, (8 * chunk * 2^-24 + 4e-6) * max|x|."""
    got = to_f64(xbar)
    mag = np.abs(exact)
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-38))) - 7)
    slack = (8 * chunk * 2.0 ** -24 + 4e-6) * x_max
    err = np.abs(got - exact)
    ulps = bf16_ulp_distance(xbar, exact)
    print(f"  max ulp {ulps.max()}, exact-match rate {(ulps == 0).mean():.4f}, "
          f"max err / bound {(err / (ulp + slack)).max():.3f}")
    assert np.all(err <= ulp + slack)


def _encode(x, doc_off, chunk, rope_base, with_norm):
    d_off = torch.as_tensor(doc_off, device=DEV)
    c_off = msa.msa_chunk_offsets(d_off, chunk)
    ref_off = chunk_offsets(doc_off, chunk)
    total = int(ref_off[-1])
    xbar, norm = msa.msa_encode_docs(x, d_off, c_off, total, chunk, rope_base=rope_base, with_norm=with_norm)
    torch.cuda.synchronize()
    assert c_off.cpu().numpy().tolist() == ref_off.tolist()
    return xbar, norm, total


def test_chunk_offsets_scan_many_documents():
    case("chunk offsets, 3000 documents")
    rng = np.random.default_rng(0)
    lens = rng.integers(0, 200, 3000)
    lens[::7] = 0
    doc_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    for chunk in (1, 64, 100):
        c_off = msa.msa_chunk_offsets(torch.as_tensor(doc_off, device=DEV), chunk)
        torch.cuda.synchronize()
        assert c_off.cpu().numpy().tolist() == chunk_offsets(doc_off, chunk).tolist()


@pytest.mark.parametrize("lens,chunk,heads,dim,dtype,rope_base", [
    ([0, 1, 63, 64, 65, 130, 0, 512, 7], 64, 8, 128, torch.bfloat16, 0.0),
    ([0, 1, 63, 64, 65, 130, 0, 512, 7], 64, 8, 128, torch.bfloat16, 1.0e6),
    ([5, 300, 33, 1000], 32, 2, 128, torch.bfloat16, 1.0e4),        # strong rotation, long doc
    ([17, 64, 3, 90], 16, 4, 64, torch.bfloat16, 1.0e4),             # head dim 64
    ([40, 9, 100], 8, 2, 64, torch.float32, 1.0e4),                  # float32
    ([2000, 1, 2047], 64, 32, 128, torch.bfloat16, 1.0e6),          # 8 KiB rows: two column segments
    ([300, 513, 1], 256, 8, 128, torch.bfloat16, 1.0e6),            # long chunks: many rotation steps per row group
    ([70, 250, 3], 100, 4, 64, torch.bfloat16, 1.0e4),              # chunk not a power of two
    ([130, 64], 64, 2, 256, torch.float32, 1.0e4),                  # float32, 1 KiB heads
])
def test_encode_parity(lens, chunk, heads, dim, dtype, rope_base):
    case(f"encode lens={lens} chunk={chunk} H={heads} d={dim} {dtype} rope={rope_base}")
    x, doc_off = _docs(lens, heads, dim, dtype, seed=sum(lens) + chunk)
    with_norm = (dim * x.element_size()) >= 32
    xbar, norm, total = _encode(x, doc_off, chunk, rope_base, with_norm)
    exact, _ = encode_docs(to_f64(x), doc_off, chunk, rope_base if rope_base > 0 else None)
    assert xbar.shape[0] == total == exact.shape[0]
    if dtype == torch.bfloat16 and rope_base > 0:
        _check_rotated_bf16(xbar, exact, float(x.float().abs().max()), chunk)
    elif dtype == torch.bfloat16:
        ulps = bf16_ulp_distance(xbar, exact)
        print(f"  max ulp {ulps.max()}, exact-match rate {(ulps == 0).mean():.4f}")
        assert ulps.max() <= 1
    else:
        # float32 sum of up to `chunk` rotated rows: a few ulps of the row scale
        err = np.abs(to_f64(xbar) - exact)
        assert err.max() <= 8 * chunk * 2.0 ** -24 * (np.abs(to_f64(x)).max() + 1)
    if norm is not None:
        np.testing.assert_allclose(to_f64(norm), chunk_norms(to_f64(xbar)), rtol=2e-6, atol=1e-30)


def test_encode_equal_lengths_matches_pool_bitwise():
    case("encode == pool on equal lengths")
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    x = torch.randn((40, 512, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    pooled, pnorm = msa.msa_pool_chunks(x, 64, with_norm=True)
    doc_off = np.arange(41, dtype=np.int64) * 512
    xbar, norm, _ = _encode(x.view(40 * 512, 8, 128), doc_off, 64, 0.0, True)
    assert torch.equal(xbar, pooled) and torch.equal(norm, pnorm)


def test_encode_full_bank_sampled():
    """About 1M tokens in 2048 documents of 256..768 rows, 8 heads x 128, bf16,
    K rotated (base 1e6); sampled chunks against the oracle."""
    case("encode 1M tokens, variable lengths (sampled)")
    rng = np.random.default_rng(7)
    lens = rng.integers(256, 769, 2048)
    x, doc_off = _docs(lens, 8, 128, torch.bfloat16, seed=7, scale=1 / 11.3)
    xbar, norm, total = _encode(x, doc_off, 64, 1.0e6, True)
    ref_off = chunk_offsets(doc_off, 64)
    docs = np.unique(np.concatenate([[0, 2047], rng.integers(0, 2048, 40)]))
    for n in docs:
        rows = to_f64(x[doc_off[n]:doc_off[n + 1]])
        exact, _ = encode_docs(rows, [0, len(rows)], 64, 1.0e6)
        got = xbar[ref_off[n]:ref_off[n + 1]]
        _check_rotated_bf16(got, exact, float(x[doc_off[n]:doc_off[n + 1]].float().abs().max()), 64)
        np.testing.assert_allclose(to_f64(norm[ref_off[n]:ref_off[n + 1]]), chunk_norms(to_f64(got)),
                                   rtol=2e-6, atol=1e-30)
