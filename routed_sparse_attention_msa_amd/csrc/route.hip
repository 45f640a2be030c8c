// S2: cosine routing scores on bf16 MFMA (gfx950, head dim 128).
//
// Method: MSA README (EverMind-AI/MSA), "Overall Design" -- each document is
// scored by the cosine similarity of the query's router projection Q_r with
// the pooled router keys, averaged over heads and maximised over the query
// tokens; this implementation also maximises over the document's chunks.
//
//   score[b, doc] = max_{t, j} (1/H) sum_h <q[b,t,h], k[doc*C+j,h]> * iq[b,t,h] * ik[doc*C+j,h]
//
// with iq, ik the float32 inverse norms (max(norm, 1e-12)).  The raw dot
// products run on bf16 MFMA: a product of two bf16 values is exact in
// float32, and the normalised vectors are never rounded to bf16.
//
// Because every head carries its own (row, column) scale, the head sum is
// not one long GEMM.  Per head the 32x32 MFMA accumulators are rescaled in
// place ("chained" scaling): before head h the accumulator holds
// sum_{h'<h} dot_h' * w_h' / w_{h-1} (w = iq * ik), is multiplied by
// w_{h-1}/w_h, and after the last head by w_{H-1}/H.  This keeps a single
// accumulator set per output tile; the per-head ratios come from small LDS
// tables.
//
// MFMA operand k-order: within each 64-wide slice of a head, lane half hf
// supplies the 32 contiguous elements [32*hf, 32*hf+32) in four 8-element
// steps, so a lane reads 64 contiguous bytes per slice (16-byte loads).  A
// (queries) and B (keys) use the same order, so each step still pairs
// matching elements; only the float32 summation order changes.
//
// Three kernels:
//  * route_scan    (up to 128 query rows, 2/4/8 heads): persistent workgroups
//    stream the bank once through LDS, tile by tile; the HBM-bound case.
//  * route_stream  (other few-row shapes): one workgroup owns 32 pooled
//    chunks; each wave owns two heads, keeps their key fragments in registers
//    (loaded straight from HBM, read exactly once), and loops over 32-row
//    query tiles; the waves' head partials meet in LDS.
//  * route_tiled   (many query rows): 256x256 output tile per workgroup,
//    8 waves (2 x 4), each wave 128 rows x 64 columns (4 x 2 MFMA blocks);
//    query and key slices are staged through XOR-swizzled, double-buffered
//    LDS, 64 k-elements of one head per stage; persistent workgroups.
//    MFMA-bound.  A sequence longer than one 256-row tile gets its maximum
//    over the tiles by atomic maxima into the scores (set to -inf by the
//    query-norm kernel that runs first).
// All end with the max over each document's chunks (cross-lane shuffles)
// and over the query tokens of each sequence.
#include <algorithm>
#include <mutex>

#include "internal.h"

namespace msa {
namespace {

constexpr float kEps = 1e-12f;
constexpr int kDim = 128;  // head dim of the MFMA path

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Row of the 32x32 MFMA accumulator held in element i of lane-half hf.
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }

// ---------------------------------------------------------------------------
// inverse query norms  iq[r][h] = 1 / max(|q_r[r,h]|, eps)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_qnorm_kernel(const uint16_t* __restrict__ q_r,
                                                          int64_t rows, int heads,
                                                          float* __restrict__ iq,
                                                          float* __restrict__ fill, int64_t n_fill) {
  // (With `fill`, also set fill[0 .. n_fill) to -inf: the scores that the
  // tiled kernel then raises with atomic maxima.)
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_fill; i += (int64_t)gridDim.x * 256)
    fill[i] = -INFINITY;
  // 16 lanes per (row, head): 16 lanes x 8 elements = 128.
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  float ss = 0.f;
  const bool ok = item < rows * heads;
  if (ok) {
    float f[8];
    Vec16<uint16_t>::widen(load16(q_r + item * kDim + sub * 8), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (ok && sub == 0) iq[item] = 1.f / fmaxf(sqrtf(ss), kEps);
}

// ---------------------------------------------------------------------------
// epilogue helpers
// ---------------------------------------------------------------------------

// Atomic maximum of float values through integer atomics (the scores start
// at -inf): a non-negative value orders like its bits as a signed integer,
// a negative one inversely to its bits as an unsigned integer, so the larger
// float always wins.  The result does not depend on the order of the calls.
__device__ __forceinline__ void atomic_max_float(float* p, float v) {
  if (__float_as_int(v) >= 0)
    atomicMax(reinterpret_cast<int*>(p), __float_as_int(v));
  else
    atomicMin(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

// Max over the C consecutive columns (lanes) of each document.
__device__ __forceinline__ float doc_max(float v, int cpd) {
  for (int off = 1; off < cpd; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// The same with DPP lane permutes (no LDS round trip): xor 1 and xor 2 inside
// quads, then the half-row mirror pairs the two quads of each 8-lane group and
// the row mirror the two halves of each 16-lane row.  Documents start at
// multiples of C inside a 32-column tile, so they align with these groups.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const int x = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(x));
}
__device__ __forceinline__ float doc_max_dpp(float v, int cpd) {
  if (cpd >= 2) v = dpp_max<0xB1>(v);     // quad_perm [1,0,3,2]
  if (cpd >= 4) v = dpp_max<0x4E>(v);     // quad_perm [2,3,0,1]
  if (cpd >= 8) v = dpp_max<0x141>(v);    // row_half_mirror
  if (cpd >= 16) v = dpp_max<0x140>(v);   // row_mirror
  if (cpd >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}

// ---------------------------------------------------------------------------
// scan kernel: T_tot <= 128 (up to four 32-row query blocks), HBM streaming
// ---------------------------------------------------------------------------
// Persistent: each workgroup walks a contiguous range of column tiles of 32
// pooled chunks (all heads: 32 x H x 256 B, 64 KiB at H = 8).  The next tile
// is prefetched into registers with fully coalesced 16-byte loads (a wave
// instruction reads 1 KiB of one chunk row) while the current tile is read
// from LDS, where rows are padded by
// 16 bytes so the MFMA operand reads (one row per lane, 16 bytes each) fall
// in distinct banks; every operand address is then one per-thread base plus
// a constant offset, which keeps the address registers out of the way of the
// query operands.
//
// The waves form G groups of H/2; in a group, wave hp owns heads 2hp, 2hp+1
// for QW query blocks (the group's blocks), whose query operands stay in
// registers for the whole kernel.  A wave reads each key fragment from LDS
// once and feeds it to the MFMAs of all its query blocks.  Its two heads share
// one accumulator by chained scaling (x w0/w1 between them, x w1 after), and
// the head-pair partials of a group's waves meet in LDS.
template <int H, int QW, int G, int TLC>
__global__ __launch_bounds__(H / 2 * G * 64, (QW == 1 && G == 1) ? 2 : 1) void route_scan_kernel(
    const uint16_t* __restrict__ q_r, const uint16_t* __restrict__ kbar,
    const float* __restrict__ knorm, int t_tot, int t_len, int64_t n_ch, int64_t n_docs, int cpd,
    int n_tiles, float* __restrict__ out) {
  constexpr int NWH = H / 2;                 // waves per group (one per head pair)
  constexpr int NW = NWH * G;
  constexpr int QB = QW * G;                 // 32-row query blocks
  constexpr int kThreads = NW * 64;
  constexpr int kRowBytes = H * kDim * 2;    // one pooled chunk, all heads
  constexpr int kSegs = kRowBytes / 16;      // 16-byte segments per chunk row
  constexpr int kRowStride = kRowBytes + 16; // LDS row pitch (padded)
  constexpr int kPerThread = 32 * kSegs / kThreads;
  static_assert(kThreads % kSegs == 0 || kSegs % kThreads == 0, "tile rows must split evenly");
  constexpr int kQuads = 4 * QW;             // accumulator quads (4 rows x 2 halves) per wave
  constexpr int kSlots = kQuads - kQuads / NWH;   // quads a wave hands to their owners
  constexpr int kSlotsAlloc = kSlots > 0 ? kSlots : 1;
  static_assert(4 % NWH == 0, "head pairs per group must divide 4");
  // TLC: sequence length class, 0: t_len in {1, 2, 4}; 1: t_len == 8; 2: t_len >= 16
  static_assert(TLC >= 0 && TLC <= 2, "bad sequence length class");
  extern __shared__ __align__(16) uint8_t smem_raw[];
  uint8_t* ktile = smem_raw;                                             // [32][kRowStride]
  f32x4* part = reinterpret_cast<f32x4*>(smem_raw + 32 * kRowStride);   // [NW][kSlots][64]
  float* qmax = reinterpret_cast<float*>(part + NW * kSlotsAlloc * 64);  // [QB * 4][64]
  float* iqr = qmax + QB * 4 * 64;   // [QB][NWH][hf][ratio | last][16], accumulator-row order
  // (then, with two query blocks per wave, the pending scores [NW][4 * kQuads / NWH][64])

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hp = wave % NWH, grp = wave / NWH;
  const int cl = lane & 31, hf = lane >> 5;
  constexpr size_t kRowElems = (size_t)H * kDim;

  // query operands of this wave's heads and blocks (zero rows past t_tot);
  // inverse norms go through LDS into the per-row tables iqr
  bf16x8 qf[QW][2][8];
  {
    float* iq_row = reinterpret_cast<float*>(ktile);      // scratch [QB * 32][H] before the loop
#pragma unroll
    for (int qw = 0; qw < QW; ++qw) {
      const int row = (grp * QW + qw) * 32 + cl;
      const bool ok = row < t_tot;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int h = 2 * hp + j;
        const uint16_t* src = q_r + (ok ? (size_t)row * kRowElems + (size_t)h * kDim : 0);
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 raw = ok ? load16(src + 64 * (k >> 2) + 32 * hf + 8 * (k & 3)) : z;
          float f[8];
          Vec16<uint16_t>::widen(raw, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
          qf[qw][j][k] = as_bf16x8(raw);
        }
        ss += __shfl_xor(ss, 32);
        if (hf == 0) iq_row[row * H + h] = 1.f / fmaxf(sqrtf(ss), kEps);
      }
    }
    __syncthreads();
    for (int idx = tid; idx < QB * NWH * 2 * 16; idx += kThreads) {
      const int i = idx & 15, hh = (idx >> 4) & 1, php = (idx >> 5) % NWH, qb = (idx >> 5) / NWH;
      const int row = qb * 32 + acc_row(i, hh);
      const float iq0 = iq_row[row * H + 2 * php], iq1 = iq_row[row * H + 2 * php + 1];
      float* dst = iqr + ((qb * NWH + php) * 2 + hh) * 32;
      dst[i] = iq0 / iq1;
      dst[16 + i] = iq1;
    }
    __syncthreads();
  }

  // register prefetch of one tile: chunk c = tid + kThreads*i -> row c/kSegs, segment c%kSegs
  u32x4 pf[kPerThread];
  float pnorm[2];
  auto prefetch = [&](int tile) {
    const int64_t col0 = (int64_t)tile * 32;
    // norms first: loads retire in order, and the inverse is only taken when the
    // tile is consumed, so nothing here waits for the 64 KiB in flight
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = col0 + cl;
      pnorm[j] = col < n_ch ? knorm[col * H + 2 * hp + j] : 0.f;
    }
    // chunk-row-major tile: thread tid's i-th 16 bytes sit at (tid + kThreads*i)*16.
    // The resource ends at the bank's end, so a ragged last tile reads zeros.
    const int64_t left = (n_ch - col0) * (int64_t)kRowBytes;
    const int n_rec = left < 32 * kRowBytes ? (int)left : 32 * kRowBytes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kbar + (size_t)col0 * kRowElems), 0, n_rec, 0x00020000);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      pf[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, kThreads * 16 * i, 2));
  };
  auto lds_at = [](int r, int sg) { return r * kRowStride + sg * 16; };
  // slot of accumulator quad Q among the quads wave w of a group hands over:
  // Q minus the number of quads below Q that w owns (w owns Q with Q % NWH == w)
  auto slot = [](int w, int Q) { return Q - (Q + NWH - 1 - w) / NWH; };

  // Scores of a tile go out one iteration later, before the next prefetch is
  // issued.  Stores and loads share one in-order vector-memory counter: a
  // store issued after a prefetch would make the wait for that prefetch wait
  // for the store's completion too.  Slot oq * 4 + e holds the score of row e
  // of the wave's oq-th own quad (Q = hp + NWH * oq) for this lane.
  constexpr int kPend = 4 * kQuads / NWH;
  // with two query blocks per wave the registers are full: the slots live in
  // this wave's own LDS area (written and read by the wave alone)
  constexpr bool kPendLds = QW > 1;
  float pend_r[kPendLds ? 1 : kPend];
  float* pend_l = iqr + QB * NWH * 2 * 32 + (size_t)wave * kPend * 64;   // [NW][kPend][64]
  auto set_pend = [&](int k, float v) {
    if constexpr (kPendLds) pend_l[k * 64 + lane] = v; else pend_r[k] = v;
  };
  auto get_pend = [&](int k) -> float {
    if constexpr (kPendLds) return pend_l[k * 64 + lane]; else return pend_r[k];
  };
  // slot (owned quad oq, row e) -> sequence of the score, if the slot holds one
  auto out_slot = [&](int oq, int e, int& seq) -> bool {
    const int Q = hp + NWH * oq;                 // this wave's oq-th quad
    const int r0 = 32 * (grp * QW + (Q >> 2)) + 8 * (Q & 3);
    if constexpr (TLC == 0) {
      const int r = r0 + 4 * hf + e;
      seq = r / t_len;
      return e % t_len == 0 && r0 < t_tot && r < t_tot;
    }
    if (e != 0 || hf != 0) return false;
    if constexpr (TLC == 1) {
      seq = r0 / 8;
      return r0 < t_tot;
    }
    const int gq = grp * kQuads + Q, quads = t_len >> 3;
    seq = gq / quads;
    return gq % quads == 0 && 8 * gq < t_tot;
  };
  auto flush = [&](int tl) {
    const int64_t col = (int64_t)tl * 32 + cl;
    const int64_t doc = col / cpd;
    if ((cl % cpd) != 0 || col >= n_ch || doc >= n_docs) return;
    // an opaque copy of n_docs keeps the per-slot row offsets from being
    // hoisted out of the tile loop (they would pin registers for its length)
    int64_t nd = n_docs;
    asm volatile("" : "+s"(nd));
#pragma unroll
    for (int oq = 0; oq < kQuads / NWH; ++oq) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int seq = 0;
        if (out_slot(oq, e, seq)) out[(size_t)seq * nd + doc] = get_pend(oq * 4 + e);
      }
    }
  };

  const float inv_h = 1.f / (float)H;
  // Each workgroup walks a contiguous range of tiles: the 4 scores a tile
  // writes per sequence are 16 bytes, and the 8 tiles of a 128-byte output
  // line then share one L2 (an XCD's), which merges them into whole lines.
  int tile = (int)((int64_t)blockIdx.x * n_tiles / gridDim.x), prev = -1;
  const int tile_hi = (int)(((int64_t)blockIdx.x + 1) * n_tiles / gridDim.x);
  if (tile < tile_hi) prefetch(tile);
  for (; tile < tile_hi; ++tile) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(ktile + lds_at(c / kSegs, c % kSegs)) = pf[i];
    }
    const bool col_ok = (int64_t)tile * 32 + cl < n_ch;
    const float ik0 = 1.f / fmaxf(pnorm[0], kEps), ik1 = 1.f / fmaxf(pnorm[1], kEps);
    const float ik_ratio = col_ok ? ik0 / ik1 : 0.f;
    const float ik_last = col_ok ? ik1 : 0.f;
    if (prev >= 0) flush(prev);
    // the registers are free again: start the next tile before the barrier
    const int next = tile + 1;
    if (next < tile_hi) prefetch(next);
    __syncthreads();

    f32x16 acc[QW];
#pragma unroll
    for (int qw = 0; qw < QW; ++qw) acc[qw] = f32x16{};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int h = 2 * hp + j;
      // key fragments in groups of KG (fewer live registers with two query blocks)
      constexpr int KG = QW == 1 ? 4 : 2;
#pragma unroll
      for (int k0 = 0; k0 < 8; k0 += KG) {
        bf16x8 kf[KG];
#pragma unroll
        for (int k = 0; k < KG; ++k) {
          const int kk = k0 + k;
          kf[k] = *reinterpret_cast<const bf16x8*>(ktile + lds_at(cl, h * 16 + 8 * (kk >> 2) + 4 * hf + (kk & 3)));
        }
#pragma unroll
        for (int qw = 0; qw < QW; ++qw) {
#pragma unroll
          for (int k = 0; k < KG; ++k) acc[qw] = mfma32(qf[qw][j][k0 + k], kf[k], acc[qw]);
        }
      }
      // x w0/w1 after the first head, x w1 after the second
      const float ikj = j == 0 ? ik_ratio : ik_last;
#pragma unroll
      for (int qw = 0; qw < QW; ++qw) {
        const float* tab = iqr + (((grp * QW + qw) * NWH + hp) * 2 + hf) * 32 + 16 * j;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(tab + i);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[qw][i + e] *= t4[e] * ikj;
        }
      }
    }
    // Head sum: wave hp of a group owns its accumulator quads Q = qw*4 + q with
    // Q % NWH == hp (query rows 32*qb + 8q + 4hf + 0..3) and adds the other
    // head pairs' partials of those quads.
#pragma unroll
    for (int Q = 0; Q < kQuads; ++Q)
      if (Q % NWH != hp)
        part[(wave * kSlotsAlloc + slot(hp, Q)) * 64 + lane] =
            f32x4{acc[Q >> 2][4 * (Q & 3)], acc[Q >> 2][4 * (Q & 3) + 1], acc[Q >> 2][4 * (Q & 3) + 2],
                  acc[Q >> 2][4 * (Q & 3) + 3]};
    __syncthreads();
#pragma unroll
    for (int Q = 0; Q < kQuads; ++Q) {
      const int qb = grp * QW + (Q >> 2), q = Q & 3;
      const int r0 = 32 * qb + 8 * q;            // first query row of the quad
      if (Q % NWH != hp || r0 >= t_tot) continue;
      float v[4] = {acc[Q >> 2][4 * q], acc[Q >> 2][4 * q + 1], acc[Q >> 2][4 * q + 2], acc[Q >> 2][4 * q + 3]};
#pragma unroll
      for (int w = 0; w < NWH; ++w) {
        if (w == hp) continue;
        const f32x4 pv = part[((grp * NWH + w) * kSlotsAlloc + slot(w, Q)) * 64 + lane];
        v[0] += pv[0];
        v[1] += pv[1];
        v[2] += pv[2];
        v[3] += pv[3];
      }
      // max over each sequence's rows, then over the document's chunks
      if constexpr (TLC == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e % t_len != 0) continue;
          float m = v[e];
          if (e + 1 < 4 && t_len >= 2) m = fmaxf(m, v[e + 1]);
          if (e + 3 < 4 && t_len >= 4) m = fmaxf(fmaxf(m, v[e + 2]), v[e + 3]);
          set_pend((Q / NWH) * 4 + e, doc_max_dpp(m, cpd) * inv_h);
        }
      } else {
        float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        m = fmaxf(m, __shfl_xor(m, 32));
        if constexpr (TLC == 1)
          set_pend((Q / NWH) * 4, doc_max_dpp(m, cpd) * inv_h);
        else
          qmax[(qb * 4 + q) * 64 + lane] = m;
      }
    }
    if constexpr (TLC == 2) {
      // a sequence spans t_len / 8 quads, possibly of several query blocks:
      // the owner of its first quad combines them
      __syncthreads();
      const int quads = t_len >> 3;
#pragma unroll
      for (int Q = 0; Q < kQuads; ++Q) {
        const int gq = grp * kQuads + Q;         // quad index over all query blocks
        if (Q % NWH != hp || gq % quads != 0 || 8 * gq >= t_tot) continue;
        float m = qmax[gq * 64 + lane];
        for (int qq = gq + 1; qq < gq + quads; ++qq) m = fmaxf(m, qmax[qq * 64 + lane]);
        set_pend((Q / NWH) * 4, doc_max_dpp(m, cpd) * inv_h);
      }
    }
    prev = tile;
  }
  if (prev >= 0) flush(prev);
}

// ---------------------------------------------------------------------------
// stream kernel: T_tot small, any T with T | 32 or 32 | T
// ---------------------------------------------------------------------------
template <int NW>
__global__ __launch_bounds__(NW * 64) void route_stream_kernel(
    const uint16_t* __restrict__ q_r, const uint16_t* __restrict__ kbar,
    const float* __restrict__ knorm, int t_tot, int t_len, int heads, int64_t n_ch, int64_t n_docs,
    int cpd, float* __restrict__ out) {
  __shared__ float part[NW][16][64];
  __shared__ float iq_s[NW][2][32];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int64_t col = (int64_t)blockIdx.x * 32 + cl;
  const bool col_ok = col < n_ch;
  const size_t row_elems = (size_t)heads * kDim;

  // Key fragments of this wave's two heads, straight from HBM (read once).
  bf16x8 kf[2][8];
  float ik[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int h = 2 * wave + j;
    const bool ok = col_ok && h < heads;
    const uint16_t* src = kbar + (ok ? (size_t)col * row_elems + (size_t)h * kDim : 0);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        kf[j][4 * g + s] = as_bf16x8(ok ? load16(src + 64 * g + 32 * hf + 8 * s) : z);
      }
    ik[j] = ok ? 1.f / fmaxf(knorm[(size_t)col * heads + h], kEps) : 0.f;
  }

  const int n_tiles = (t_tot + 31) / 32;
  const float inv_h = 1.f / (float)heads;
  float run = -INFINITY;  // running max across row tiles of one sequence (T > 32)
  for (int rt = 0; rt < n_tiles; ++rt) {
    const int row0 = rt * 32;
    const int row = row0 + cl;
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int h = 2 * wave + j;
      const bool ok = row < t_tot && h < heads;
      const uint16_t* src = q_r + (ok ? (size_t)row * row_elems + (size_t)h * kDim : 0);
      bf16x8 qf[8];
      float ss = 0.f;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 raw = ok ? load16(src + 64 * g + 32 * hf + 8 * st) : z;
          float f[8];
          Vec16<uint16_t>::widen(raw, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
          qf[4 * g + st] = as_bf16x8(raw);
        }
      ss += __shfl_xor(ss, 32);
      if (hf == 0) iq_s[wave][j][cl] = 1.f / fmaxf(sqrtf(ss), kEps);
      f32x16 acc = {};
#pragma unroll
      for (int k = 0; k < 8; ++k) acc = mfma32(qf[k], kf[j][k], acc);
      __syncthreads();  // iq_s visible to every lane of the wave
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] += acc[i] * (iq_s[wave][j][acc_row(i, hf)] * ik[j]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) part[wave][i][lane] = s[i];
    __syncthreads();
    if (wave == 0) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += part[w][i][lane];
        v[i] = doc_max(tot * inv_h, cpd);
      }
      const bool writer = (cl % cpd) == 0 && col_ok;
      const int64_t doc = col / cpd;
      if (t_len >= 32) {
        // the whole tile belongs to one sequence
        float m = v[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, v[i]);
        m = fmaxf(m, __shfl_xor(m, 32));
        run = fmaxf(run, m);
        if ((row0 + 32) % t_len == 0) {
          const int b = row0 / t_len;
          if (writer && hf == 0 && doc < n_docs) out[(size_t)b * n_docs + doc] = run;
          run = -INFINITY;
        }
      } else if (t_len >= 8) {
        // segments of t_len rows: groups of (t_len/8) register quads, both halves
        const int quads = t_len >> 3;
        for (int q0 = 0; q0 < 4; q0 += quads) {
          float m = -INFINITY;
          for (int q = q0; q < q0 + quads; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, v[4 * q + e]);
          m = fmaxf(m, __shfl_xor(m, 32));
          const int r = row0 + 8 * q0;
          if (writer && hf == 0 && r < t_tot && doc < n_docs) out[(size_t)(r / t_len) * n_docs + doc] = m;
        }
      } else {
        // t_len in {1, 2, 4}: segments inside one register quad of one half
        for (int i0 = 0; i0 < 16; i0 += t_len) {
          float m = -INFINITY;
          for (int e = 0; e < t_len; ++e) m = fmaxf(m, v[i0 + e]);
          const int r = row0 + acc_row(i0, hf);
          if (writer && r < t_tot && doc < n_docs) out[(size_t)(r / t_len) * n_docs + doc] = m;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// tiled kernel: many query rows, T % 32 == 0
// ---------------------------------------------------------------------------
constexpr int kTB = 256;             // rows per workgroup tile
constexpr int kNB = 256;             // columns (pooled chunks) per workgroup tile
constexpr int kTiledThreads = 512;   // 8 waves: 2 along rows x 4 along columns
constexpr int kStageK = 64;          // k elements per LDS stage (half a head)
constexpr int kMaxHeads = 8;         // scale tables sized for up to 8 heads (LDS budget)
constexpr int kStreamMaxHeads = 16;

struct TiledSmem {
  uint8_t q[2][kTB * kStageK * 2];   // [buf][row][128 B], XOR-swizzled 16 B segments
  uint8_t k[2][kNB * kStageK * 2];
  float rq[kMaxHeads + 1][kTB];      // rq[h]: scale applied before head h (h = H: final)
  float rk[kMaxHeads + 1][kNB];
  float red[8][kNB];                 // epilogue: per row block, per document of the tile
};

// 16 B segment seg of a 128 B row, XOR-swizzled by (row / 2) % 8.  A 256 B
// LDS bank line holds two rows; a 16-lane phase of a b128 read takes one
// segment of 16 consecutive rows, whose 8 even and 8 odd rows then fall on
// 8 distinct segments each, so the phase is conflict-free (with row % 8 the
// rows r and r + 8 collided, every operand read 2-way conflicted).  A
// 16-lane phase of the stores writes two whole rows: conflict-free too.
__device__ __forceinline__ int swz(int row, int seg) { return row * 128 + ((seg ^ ((row >> 1) & 7)) << 4); }

__global__ __launch_bounds__(kTiledThreads) void route_tiled_kernel(
    const uint16_t* __restrict__ q_r, const uint16_t* __restrict__ kbar,
    const float* __restrict__ knorm, const float* __restrict__ iq, int t_tot, int t_len, int heads,
    int64_t n_ch, int64_t n_docs, int cpd, int direct, int row_groups, int n_tiles,
    float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TiledSmem& sm = *reinterpret_cast<TiledSmem*>(smem_raw);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves
  // Tile order.  Launch index v runs on XCD v % 8 (workgroups reach the XCDs
  // round-robin); XCD c is given one contiguous run of a tile order in which
  // the row tiles are split into row_groups contiguous groups, each
  // enumerated column by column with its row tiles fastest.  An XCD's run
  // then stays inside one row group: it reads each of its column tiles of the
  // bank into its L2 once, for all of that group's row tiles, and keeps only
  // the group's queries resident.  The bank is read row_groups times, the
  // queries about 8 / row_groups times.  (Column tiles fastest streamed the
  // whole bank from HBM once per row tile.)  Any order is correct; this one
  // only places reuse.  The kernel is persistent: workgroup w takes the
  // virtual launch indices w, w + G, w + 2G, ... (G = gridDim.x, a multiple
  // of 8 when smaller than the tile count, so they stay on w's XCD).
  const int n_ty = (t_tot + kTB - 1) / kTB;
  const unsigned n_tx = (unsigned)n_tiles / (unsigned)n_ty;
  auto tile_at = [&](unsigned v, int* ty_out, int64_t* tx_out) {
    const unsigned xcd = v % 8u, per = (unsigned)n_tiles / 8u, extra = (unsigned)n_tiles % 8u;
    const unsigned tile = xcd * per + min(xcd, extra) + v / 8u;
    int grp = 0;
    while (grp + 1 < row_groups && n_tx * (unsigned)((grp + 1) * n_ty / row_groups) <= tile) ++grp;
    const int r_lo = grp * n_ty / row_groups, r_hi = (grp + 1) * n_ty / row_groups;
    const unsigned in_grp = tile - n_tx * (unsigned)r_lo;
    *ty_out = r_lo + (int)(in_grp % (unsigned)(r_hi - r_lo));
    *tx_out = in_grp / (unsigned)(r_hi - r_lo);
  };
  const size_t row_elems = (size_t)heads * kDim;
  const uint32_t row_bytes = (uint32_t)(row_elems * 2);
  const unsigned G = gridDim.x;

  // --- per-head scale tables -------------------------------------------------
  // Threads 0..255 own the tile's rows (inverse query norms), 256..511 its
  // columns (inverse key norms); every head's value is loaded at once, early
  // (for the next tile: during the current tile's last head), and turned into
  // the chained ratios when the tables are free.
  // (Head indices past `heads` reread the last head, so the loads need no
  // per-head predicate and stay inside the row.  The last head's value is
  // loaded on its own: selecting tv[heads - 1] would index the array
  // dynamically and move it to scratch memory.)
  float tv[kMaxHeads], tv_last;
  auto load_tables = [&](int row0, int64_t col0) {
    if (tid < kTB) {
      const int r = row0 + tid;
      const bool ok = r < t_tot;
      const float* src = iq + (size_t)(ok ? r : 0) * heads;
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) tv[h] = src[min(h, heads - 1)];
      tv_last = src[heads - 1];
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) tv[h] = ok ? tv[h] : 1.f;
      tv_last = ok ? tv_last : 1.f;
    } else {
      const int64_t n = col0 + (tid - kTB);
      const bool ok = n < n_ch;
      const float* src = knorm + (ok ? n : 0) * heads;
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) tv[h] = src[min(h, heads - 1)];
      tv_last = src[heads - 1];
#pragma unroll
      for (int h = 0; h < kMaxHeads; ++h) tv[h] = ok ? 1.f / fmaxf(tv[h], kEps) : 0.f;
      tv_last = ok ? 1.f / fmaxf(tv_last, kEps) : 0.f;
    }
  };
  auto store_tables = [&] {
    if (tid < kTB) {
#pragma unroll
      for (int h = 1; h < kMaxHeads; ++h)
        if (h < heads) sm.rq[h][tid] = tv[h - 1] / tv[h];
      sm.rq[heads][tid] = tv_last;
    } else {
      const int c = tid - kTB;
#pragma unroll
      for (int h = 1; h < kMaxHeads; ++h)
        if (h < heads) sm.rk[h][c] = tv[h] != 0.f ? tv[h - 1] / tv[h] : 0.f;
      sm.rk[heads][c] = tv_last / (float)heads;
    }
  };

  // --- staging: 4 x 16 B of q and 4 x 16 B of k per thread per stage ----------
  // Buffer loads: a per-lane offset fixed for the kernel plus the stage's
  // scalar offset; rows past t_tot / n_ch lie beyond the resources' records
  // and read as zeros, so the loads carry no branches and no address math.
  // (Base and size pass through readfirstlane: the compiler did not prove
  // them uniform and wrapped every load in a loop over the lanes' values.)
  auto uniform_rsrc = [](const uint16_t* p, size_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* u = reinterpret_cast<void*>((uintptr_t)(((uint64_t)hi << 32) | lo));
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes), 0x00020000);
  };
  auto q_rsrc = [&](int row0) {
    return uniform_rsrc(q_r + (size_t)row0 * row_elems, (size_t)max(0, min(kTB, t_tot - row0)) * row_bytes);
  };
  auto k_rsrc = [&](int64_t col0) {
    return uniform_rsrc(kbar + (size_t)col0 * row_elems,
                        (size_t)max<int64_t>(0, min<int64_t>(kNB, n_ch - col0)) * row_bytes);
  };
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kTiledThreads * i;
    voff[i] = (uint32_t)(c >> 3) * row_bytes + (c & 7) * 16;
  }
  // LDS byte addresses.  The key buffers start at 64 KiB, past the reach of a
  // DS instruction's 16-bit offset, so each lane's addresses carry their
  // buffer's base: every access is then (lane address) + (constant offset),
  // with no address arithmetic in the loop.  A 32-row block moves an
  // address by 32 * 128 B and leaves its swizzle ((row / 2) % 8) unchanged;
  // so does a staging piece (64 rows).
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t q_lds = (uint32_t)(uintptr_t)(lds_u8*)(&sm.q[0][0]);
  const uint32_t k_lds = (uint32_t)(uintptr_t)(lds_u8*)(&sm.k[0][0]);
  // (Each address is passed through an empty asm: the compiler otherwise
  // splits it into shared parts and adds them back before every access.)
  uint32_t q_rd[4], k_rd[4];   // operand reads of k step s: row block 0, buffer 0
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    q_rd[s] = q_lds + (uint32_t)swz(wm * 128 + cl, 4 * hf + s);
    k_rd[s] = k_lds + (uint32_t)swz(wn * 64 + cl, 4 * hf + s);
    asm("" : "+v"(q_rd[s]));
    asm("" : "+v"(k_rd[s]));
  }
  uint32_t q_st = q_lds + (uint32_t)swz(tid >> 3, tid & 7);   // staging piece 0, buffer 0
  uint32_t k_st = k_lds + (uint32_t)swz(tid >> 3, tid & 7);
  asm("" : "+v"(q_st));
  asm("" : "+v"(k_st));
  constexpr uint32_t kBufBytes = kTB * kStageK * 2;
  static_assert(kTB * kStageK * 2 == kNB * kStageK * 2, "q and k buffers have one size");
  static_assert(kBufBytes + 3 * 64 * 128 < 65536 && kBufBytes + 3 * 32 * 128 < 65536, "offsets must fit 16 bits");

  // first tile of this workgroup: its tables, stage 0 in buffer 0, stage 1 in registers
  unsigned v = blockIdx.x;
  int ty;
  int64_t tx;
  tile_at(v, &ty, &tx);
  // the tile the staging loads read: the current one, switched to the next
  // tile for the current tile's last head (whose loads are the next tile's
  // first two stages)
  __amdgpu_buffer_rsrc_t ld_q = q_rsrc(ty * kTB), ld_k = k_rsrc(tx * kNB);
  int ty_n = ty;
  int64_t tx_n = tx;
  bool has_next = false;
  const int n_stages = 2 * heads;
  u32x4 pq[4], pk[4];
  // one of the four 16 B pieces of q and of k per thread: load for a stage
  // (stages n_stages and n_stages + 1 are the next tile's first two), store
  // to an LDS buffer
  auto gload1 = [&](int stage, int i) {
    const int st = stage >= n_stages ? stage - n_stages : stage;
    const uint32_t soff = (uint32_t)((st >> 1) * kDim + (st & 1) * 64) * 2;
    pq[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ld_q, voff[i], soff, 0));
    pk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ld_k, voff[i], soff, 0));
  };
  auto lstore1 = [&](int buf, int i) {   // piece i: rows 64 i + tid / 8
    const uint32_t off = (uint32_t)buf * kBufBytes + (uint32_t)i * 64 * 128;
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((uintptr_t)(q_st + off)) = pq[i];
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((uintptr_t)(k_st + off)) = pk[i];
  };
  load_tables(ty * kTB, tx * kNB);
  store_tables();
#pragma unroll
  for (int i = 0; i < 4; ++i) gload1(0, i);
#pragma unroll
  for (int i = 0; i < 4; ++i) lstore1(0, i);
#pragma unroll
  for (int i = 0; i < 4; ++i) gload1(1, i);
  __syncthreads();

  f32x16 acc[4][2];
  // (the tables sit past 128 KiB: the lane's address of head 0, plus the head's row)
  uint32_t rq_lane = (uint32_t)(uintptr_t)(lds_u8*)(&sm.rq[0][wm * 128 + 4 * hf]);
  uint32_t rk_lane = (uint32_t)(uintptr_t)(lds_u8*)(&sm.rk[0][wn * 64 + cl]);
  asm("" : "+v"(rq_lane));
  asm("" : "+v"(rk_lane));
  // chain to head hn (or, with hn == heads, apply the final scale); the four
  // factor reads of a row block are issued together, so their LDS latencies
  // overlap.
  auto rescale = [&](int hn) {
    const uint32_t rqa = rq_lane + (uint32_t)hn * kTB * 4, rka = rk_lane + (uint32_t)hn * kNB * 4;
    float ck[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
      ck[b] = *reinterpret_cast<__attribute__((address_space(3))) const float*>((uintptr_t)(rka + (uint32_t)b * 32 * 4));
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 rq4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rq4[q] = *reinterpret_cast<__attribute__((address_space(3))) const f32x4*>(
            (uintptr_t)(rqa + (uint32_t)(a * 32 + 8 * q) * 4));
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[a][b][4 * q + e] *= rq4[q][e] * ck[b];
    }
  };
  // One stage's MFMAs from LDS buffer buf.  Between them the staged
  // registers go to buffer nbuf (no wave reads it in this stage: every wave
  // passed the barrier after its last reads of it) and are reloaded with
  // stage nstage, one piece per k step, so the stores and loads issue while
  // the matrix core is busy instead of after the stage, and each load has a
  // whole stage to land before its store.
  // The operand reads run one k step ahead (two register sets): step s + 1's
  // fragments are requested before step s's MFMAs issue.
  auto stage_mfma = [&](int buf, int nbuf, int nstage) {
    typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
    bf16x8 af[2][4], bfr[2][2];
    auto read = [&](int s) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[s & 1][a] = *reinterpret_cast<lds_frag*>((uintptr_t)(q_rd[s] + (uint32_t)buf * kBufBytes + (uint32_t)a * 32 * 128));
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bfr[s & 1][b] = *reinterpret_cast<lds_frag*>((uintptr_t)(k_rd[s] + (uint32_t)buf * kBufBytes + (uint32_t)b * 32 * 128));
    };
    read(0);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);    // step 0's reads
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) read(s + 1);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(af[s & 1][a], bfr[s & 1][b], acc[a][b]);
      lstore1(nbuf, s);
      gload1(nstage, s);
      if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads of the next step
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);  // LDS writes
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // global loads
    }
  };

  const int ndw = kNB / cpd;  // documents per workgroup tile
  const int n_blk = t_tot / 32;
  while (true) {
    const int row0 = ty * kTB;
    const int64_t col0 = tx * kNB;
    has_next = v + G < (unsigned)n_tiles;
    if (has_next) tile_at(v + G, &ty_n, &tx_n);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    // Two stages (the halves of one head) per iteration; the chained rescale
    // to the next head closes it.  The last head's stages load the next
    // tile's first two (or, on the last tile, a clamped copy), so its loop
    // starts from LDS.
    for (int h = 0; h < heads; ++h) {
      const bool last = h == heads - 1;
      if (last && has_next) {
        ld_q = q_rsrc(ty_n * kTB);
        ld_k = k_rsrc(tx_n * kNB);
      }
      // on the last tile the last head's loads are clamped copies of its last stage
      const int clamp = last && !has_next ? n_stages - 1 : 1 << 30;
      stage_mfma(0, 1, min(2 * h + 2, clamp));
      __syncthreads();
      stage_mfma(1, 0, min(2 * h + 3, last ? clamp : n_stages - 1));
      rescale(h + 1);                   // h + 1 == heads: the final scale
      __syncthreads();
    }
    // The next tile's scale factors are loaded now and go into the tables
    // (every wave is past its last read of them) behind the block maxima.
    if (has_next) load_tables(ty_n * kTB, tx_n * kNB);

    // --- epilogue: max over each row block's 32 rows, then each doc's chunks --
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float m = acc[a][b][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, acc[a][b][i]);
        m = fmaxf(m, __shfl_xor(m, 32));
        m = doc_max(m, cpd);
        const int c = wn * 64 + b * 32 + cl;
        if (hf == 0 && (cl % cpd) == 0) sm.red[wm * 4 + a][c / cpd] = m;
      }
    }
    if (has_next) store_tables();
    __syncthreads();
    for (int idx = tid; idx < 8 * ndw; idx += kTiledThreads) {
      const int rb = idx / ndw, dw = idx - rb * ndw;
      const int gblk = ty * 8 + rb;
      if (gblk >= n_blk) continue;
      const int b = gblk * 32 / t_len;
      const bool start = rb == 0 || ((gblk - 1) * 32 / t_len) != b;
      if (!start) continue;
      float m = sm.red[rb][dw];
      for (int r2 = rb + 1; r2 < 8 && ty * 8 + r2 < n_blk && (ty * 8 + r2) * 32 / t_len == b; ++r2)
        m = fmaxf(m, sm.red[r2][dw]);
      const int64_t doc = col0 / cpd + dw;
      if (doc >= n_docs) continue;
      if (direct)
        out[(size_t)b * n_docs + doc] = m;
      else
        atomic_max_float(out + (size_t)b * n_docs + doc, m);
    }
    (void)row0;
    if (!has_next) break;
    // (the next tile's epilogue writes red only after many barriers)
    v += G;
    ty = ty_n;
    tx = tx_n;
  }
}

enum class RoutePath { Generic, Scan, Stream, Tiled };

constexpr int kStreamMaxRows = 128;

RoutePath pick(int batch, int q_len, int heads, int dim, int cpd, msa_dtype dt) {
  if (dt != MSA_BF16 || dim != kDim || heads > kStreamMaxHeads) return RoutePath::Generic;
  if (cpd > 32 || (32 % cpd) != 0) return RoutePath::Generic;
  const int64_t t_tot = (int64_t)batch * q_len;
  const bool small_t = q_len <= 32 && (32 % q_len) == 0;
  const bool t32 = q_len % 32 == 0;
  if (t_tot <= 32 && small_t && (heads == 2 || heads == 4 || heads == 8)) return RoutePath::Scan;
  if (t_tot <= 128 && (small_t || t32) && heads == 8) return RoutePath::Scan;
  if (t_tot <= kStreamMaxRows && (small_t || t32)) return RoutePath::Stream;
  if (t32 && heads <= kMaxHeads) return RoutePath::Tiled;
  if (small_t) return RoutePath::Stream;
  return RoutePath::Generic;
}

// direct: every sequence's rows lie inside one 256-row tile
bool tiled_direct(int q_len) { return q_len <= kTB && (kTB % q_len) == 0; }

}  // namespace

hipError_t launch_route_generic(const void* q_r, const void* kbar_r, const float* knorm, int batch,
                                int q_len, int heads, int dim, int64_t n_docs, int cpd,
                                msa_dtype dt, float* doc_scores, hipStream_t s);

bool route_is_tiled(int batch, int q_len, int heads, int dim, int cpd, msa_dtype dt) {
  return pick(batch, q_len, heads, dim, cpd, dt) == RoutePath::Tiled;
}

size_t route_workspace_bytes(int batch, int q_len, int heads, int dim, int64_t n_docs, int cpd,
                             msa_dtype dt) {
  if (pick(batch, q_len, heads, dim, cpd, dt) != RoutePath::Tiled) return 0;
  const size_t t_tot = (size_t)batch * q_len;
  return t_tot * heads * sizeof(float);  // inverse query norms
}

hipError_t launch_route(const void* q_r, const void* kbar_r, const float* knorm, int batch,
                        int q_len, int heads, int dim, int64_t n_docs, int cpd, msa_dtype dt,
                        float* doc_scores, void* ws, hipStream_t s) {
  const RoutePath path = pick(batch, q_len, heads, dim, cpd, dt);
  const int64_t n_ch = n_docs * cpd;
  const int t_tot = batch * q_len;
  const uint16_t* q = static_cast<const uint16_t*>(q_r);
  const uint16_t* k = static_cast<const uint16_t*>(kbar_r);
  if (path == RoutePath::Generic)
    return launch_route_generic(q_r, kbar_r, knorm, batch, q_len, heads, dim, n_docs, cpd, dt,
                                doc_scores, s);
  if (path == RoutePath::Scan) {
    const int n_tiles = (int)((n_ch + 31) / 32);
    const int qb = (t_tot + 31) / 32 == 3 ? 4 : (t_tot + 31) / 32;
    const int n_cu = device_cu_count();
    auto go = [&](auto kern, int nwh, int qw, int g) {
      const int nw = nwh * g, quads = 4 * qw;
      const int slots = std::max(1, quads - quads / nwh);
      const int blocks = qw * g;
      const size_t pend = qw > 1 ? (size_t)nw * (4 * quads / nwh) * 64 * 4 : 0;
      const size_t smem = (size_t)32 * (heads * kDim * 2 + 16) + (size_t)nw * slots * 64 * 16 +
                          (size_t)blocks * 4 * 64 * 4 + (size_t)blocks * nwh * 2 * 32 * 4 + pend;
      static const hipError_t attr = hipFuncSetAttribute(
          reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (attr != hipSuccess) return attr;
      const int per_cu = (qw == 1 && g == 1) ? 2 : 1;
      const unsigned grid = (unsigned)std::min<int64_t>(n_tiles, (int64_t)n_cu * per_cu);
      hipLaunchKernelGGL(kern, dim3(grid), dim3(nw * 64), smem, s, q, k, knorm, t_tot, q_len, n_ch,
                         n_docs, cpd, n_tiles, doc_scores);
      return hipGetLastError();
    };
    const int tlc = q_len <= 4 ? 0 : q_len == 8 ? 1 : 2;
#define MSA_SCAN(H, QW, G, NWH)                                                  \
  switch (tlc) {                                                                 \
    case 0: return go(route_scan_kernel<H, QW, G, 0>, NWH, QW, G);              \
    case 1: return go(route_scan_kernel<H, QW, G, 1>, NWH, QW, G);              \
    default: return go(route_scan_kernel<H, QW, G, 2>, NWH, QW, G);             \
  }
    if (qb == 1) {
      if (heads == 2) MSA_SCAN(2, 1, 1, 1)
      if (heads == 4) MSA_SCAN(4, 1, 1, 2)
      MSA_SCAN(8, 1, 1, 4)
    }
    if (qb == 2) MSA_SCAN(8, 1, 2, 4)
    MSA_SCAN(8, 2, 2, 4)
#undef MSA_SCAN
  }
  if (path == RoutePath::Stream) {
    const unsigned grid = (unsigned)((n_ch + 31) / 32);
    const int nw = (heads + 1) / 2;
#define MSA_STREAM(NW)                                                                         \
  case NW:                                                                                     \
    hipLaunchKernelGGL(route_stream_kernel<NW>, dim3(grid), dim3(NW * 64), 0, s, q, k, knorm, \
                       t_tot, q_len, heads, n_ch, n_docs, cpd, doc_scores);                    \
    break;
    switch (nw) {
      MSA_STREAM(1)
      MSA_STREAM(2)
      MSA_STREAM(3)
      MSA_STREAM(4)
      MSA_STREAM(5)
      MSA_STREAM(6)
      MSA_STREAM(7)
      MSA_STREAM(8)
      default:
        return hipErrorInvalidValue;
    }
#undef MSA_STREAM
    return hipGetLastError();
  }
  // tiled: the inverse query norms (and, when a sequence spans several
  // 256-row tiles, the scores set to -inf for the tiles' atomic maxima), then
  // the tiled kernel
  float* iq = static_cast<float*>(ws);
  const int64_t items = (int64_t)t_tot * heads;
  const bool direct = tiled_direct(q_len);
  hipLaunchKernelGGL(route_qnorm_kernel, dim3((unsigned)((items * 16 + 255) / 256)), dim3(256), 0, s,
                     q, (int64_t)t_tot, heads, iq, doc_scores, direct ? (int64_t)0 : (int64_t)batch * n_docs);
  const int64_t n_tiles = ((n_ch + kNB - 1) / kNB) * ((t_tot + kTB - 1) / kTB);
  // persistent: one workgroup per CU (the LDS holds one), a multiple of 8 of
  // them so each keeps to its XCD's run of tiles
  const int n_cu = device_cu_count();
  const int64_t wgs = n_tiles <= n_cu ? n_tiles : std::max<int64_t>(8, (n_cu / 8) * 8);
  const dim3 grid((unsigned)wgs);
  const size_t smem = sizeof(TiledSmem);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(route_tiled_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)smem);
  if (attr != hipSuccess) return attr;
  // row groups: enough that one group's queries (heads * 256 B per token)
  // take at most about 2 MiB of an XCD's 4 MB L2; a divisor of 8, at most
  // the number of row tiles
  const int n_ty = (t_tot + kTB - 1) / kTB;
  int row_groups = 1;
  while (row_groups < 8 && 2 * row_groups <= n_ty &&
         (size_t)t_tot * heads * kDim * 2 > (size_t)row_groups * (2u << 20))
    row_groups *= 2;
  hipLaunchKernelGGL(route_tiled_kernel, grid, dim3(kTiledThreads), smem, s, q, k, knorm, iq, t_tot,
                     q_len, heads, n_ch, n_docs, cpd, direct ? 1 : 0, row_groups, (int)n_tiles, doc_scores);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Library-resident routing scratch, for callers that cannot allocate (code
// under graph capture, serving loops that forbid hipMalloc).  Each device the
// library runs on holds its own copy from the moment the module loads until
// the process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address reaches a kernel.
static __device__ __align__(256) uint8_t scratch[kRouteStaticScratchBytes];

hipError_t route_static_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace msa
