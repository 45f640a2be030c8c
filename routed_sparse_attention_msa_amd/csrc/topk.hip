// S3: exact top-k document selection.
//
// Method: MSA README (EverMind-AI/MSA), "Overall Design" and "Inference
// Pipeline" stage 2 -- the top-k documents by routing score are selected.
//
// Each (score, doc id) pair becomes one unique 64-bit key:
//     high 32 bits: the score's bits mapped so that unsigned order = float order
//     low  32 bits: 0xFFFFFFFF - id   (equal scores: the lower id is larger)
// so "k largest keys" is exactly "k best scores, ties to the lower id", a
// total order with a unique answer.
//
// A workgroup (256 threads x 16 keys = 4096 keys in registers) finds the k
// largest of its keys with an MSB-first radix select (8-bit digits, an LDS
// histogram per digit, a suffix scan across the 4 waves with cross-lane
// shuffles), stopping as soon as the remaining candidates are all selected.
// The k winners are appended to LDS and ordered with a bitonic network.
// Rows longer than one tile are reduced in rounds: every tile emits its k
// best keys to the workspace, and the next round selects among those.
//
// Exclusion (multi-round routing, MSA README "Inference Pipeline", Figure 3,
// and the page's FAQ on Memory Interleave: a later routing round skips the
// documents earlier rounds selected): each first-round tile marks the
// excluded ids that fall in its 4096-id range in an LDS bitmap and drops
// those keys before the select.
#include "internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;
constexpr int kTile = kThreads * kItems;
constexpr int kMaxK = 1024;

__device__ __forceinline__ uint32_t order_score(float s) {
  if (s == 0.f) s = 0.f;  // -0.0 and +0.0 compare equal: give them one key
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unorder_score(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
  return ((uint64_t)order_score(s) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

struct Smem {
  uint64_t list[kMaxK];
  uint32_t excl_bits[kTile / 32];
  uint32_t hist[256];
  uint32_t wave_sum[kThreads / 64];
  uint32_t count;
  uint32_t sel_digit, sel_gt, sel_cnt;
};

// Inclusive prefix sum of one value per thread over the block.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, Smem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sm.wave_sum[wave] = v;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += sm.wave_sum[w];
  __syncthreads();
  return v + base;
}

// The block holds kItems keys per thread (`valid` marks real ones; real keys
// are unique).  Leaves the min(k, #valid) largest keys sorted in descending
// order in sm.list[0 .. kp2), padded with 0 (below every real key).
__device__ void block_select(const uint64_t (&key)[kItems], const bool (&valid)[kItems], int k,
                             int kp2, Smem& sm) {
  const int tid = threadIdx.x;
  uint32_t my_valid = 0;
#pragma unroll
  for (int i = 0; i < kItems; ++i) my_valid += valid[i] ? 1u : 0u;
  const uint32_t n_valid = block_inclusive_scan(my_valid, sm);
  if (tid == kThreads - 1) sm.count = n_valid;  // total
  __syncthreads();
  const int k_eff = (int)min((uint32_t)k, sm.count);
  __syncthreads();

  uint64_t prefix = 0, mask = 0;
  int krem = k_eff;
  if (k_eff > 0) {
    for (int shift = 56; shift >= 0; shift -= 8) {
      sm.hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kItems; ++i)
        if (valid[i] && (key[i] & mask) == prefix) atomicAdd(&sm.hist[(key[i] >> shift) & 0xFF], 1u);
      __syncthreads();
      // Thread t looks at bin 255 - t: the inclusive scan is then the number
      // of candidates whose digit is >= that bin.
      const uint32_t bin = 255 - tid;
      const uint32_t h = sm.hist[bin];
      const uint32_t incl = block_inclusive_scan(h, sm);
      const uint32_t excl = incl - h;
      if (excl < (uint32_t)krem && (uint32_t)krem <= incl) {
        sm.sel_digit = bin;
        sm.sel_gt = excl;
        sm.sel_cnt = h;
      }
      __syncthreads();
      prefix |= (uint64_t)sm.sel_digit << shift;
      mask |= (uint64_t)0xFF << shift;
      krem -= (int)sm.sel_gt;
      const bool done = (int)sm.sel_cnt == krem;  // every key with this prefix is in
      __syncthreads();
      if (done) break;
    }
  }

  if (tid == 0) sm.count = 0;
  __syncthreads();
  if (k_eff > 0) {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      if (valid[i] && (key[i] & mask) >= prefix) {
        const uint32_t pos = atomicAdd(&sm.count, 1u);
        sm.list[pos] = key[i];
      }
    }
  }
  __syncthreads();
  for (int i = k_eff + tid; i < kp2; i += kThreads) sm.list[i] = 0;
  __syncthreads();

  // Bitonic sort of sm.list[0 .. kp2), descending.
  for (int size = 2; size <= kp2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < kp2 / 2; i += kThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = sm.list[lo], b = sm.list[hi];
        if ((a < b) == desc) {
          sm.list[lo] = b;
          sm.list[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// One tile of one row.  FROM_KEYS: the input is a previous round's keys
// (0 = padding); otherwise raw float scores whose ids are their positions.
// FINAL: write ids/scores; otherwise write the tile's k best keys.
// Exclusion (raw-score rounds only): excl[b * excl_stride + j], j < n_excl;
// ids outside [0, n) are ignored.  Outputs of FINAL go to row b * out_stride.
template <bool FROM_KEYS, bool FINAL>
__global__ __launch_bounds__(kThreads) void topk_tile_kernel(
    const float* __restrict__ scores, const uint64_t* __restrict__ keys_in, int64_t n, int k,
    int kp2, const int32_t* excl, int n_excl, int64_t excl_stride, uint64_t* __restrict__ keys_out,
    int32_t* ids_out, float* vals_out, int64_t out_stride) {
  __shared__ Smem sm;
  const int b = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * kTile;
  const bool any_excl = !FROM_KEYS && n_excl > 0;
  if (any_excl) {
    for (int i = threadIdx.x; i < kTile / 32; i += kThreads) sm.excl_bits[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n_excl; j += kThreads) {
      const int64_t id = excl[(size_t)b * excl_stride + j];
      const int64_t rel = id - base;
      if (id >= 0 && id < n && rel >= 0 && rel < kTile) atomicOr(&sm.excl_bits[rel >> 5], 1u << (rel & 31));
    }
    __syncthreads();
  }
  uint64_t key[kItems];
  bool valid[kItems];
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int rel = i * kThreads + threadIdx.x;
    const int64_t idx = base + rel;
    valid[i] = idx < n && !(any_excl && ((sm.excl_bits[rel >> 5] >> (rel & 31)) & 1u));
    key[i] = 0;
    if (valid[i]) {
      if (FROM_KEYS) {
        key[i] = keys_in[(size_t)b * n + idx];
        valid[i] = key[i] != 0;
      } else {
        key[i] = make_key(scores[(size_t)b * n + idx], (uint32_t)idx);
      }
    }
  }
  block_select(key, valid, k, kp2, sm);
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const uint64_t kk = sm.list[i];
    if (FINAL) {
      ids_out[(size_t)b * out_stride + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)kk);
      if (vals_out) vals_out[(size_t)b * out_stride + i] = unorder_score((uint32_t)(kk >> 32));
    } else {
      keys_out[((size_t)b * gridDim.x + blockIdx.x) * k + i] = kk;
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of at most one tile with k <= 64 (the routing and decode sizes): each
// lane sorts its few keys in registers, each wave takes out its k largest by
// repeated wave maxima (DPP reductions, the result broadcast through a
// scalar register), and wave 0 takes the final k out of the four waves'
// candidates.  One barrier instead of the radix passes' dozens; exact like
// them (the keys are unique).
constexpr int kSmallMaxK = 64;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  // quad xor 1, quad xor 2, row half-mirror, row mirror: every lane holds its
  // row's max; row broadcasts 15 and 31 carry the rows' maxima to lane 63
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Largest 64-bit key of the wave (the high words first, then the low words
// of the lanes that hold the largest high word; when one lane holds it, its
// low word is read directly).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint64_t holders = __ballot((uint32_t)(v >> 32) == hi);
  uint32_t lo;
  if (__popcll(holders) == 1)   // uniform
    lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, __ffsll((long long)holders) - 1);
  else
    lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// Descending bitonic sort of one key per lane across the wave: lane r ends
// with the r-th largest.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t xlo = (uint32_t)__shfl_xor((int)(uint32_t)v, stride);
      const uint32_t xhi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), stride);
      const uint64_t x = ((uint64_t)xhi << 32) | xlo;
      // blocks of `size` lanes alternate direction; the last block (all 64) runs descending
      const bool up = (lane & size) != 0 && size < 64;
      const bool lower = (lane & stride) == 0;
      const bool keep_max = lower != up;
      v = keep_max ? (x > v ? x : v) : (x < v ? x : v);
    }
  return v;
}

// Descending bitonic sort of a register array (constant indices throughout).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const uint64_t x = a[i], y = a[j];
          const bool swap = desc ? x < y : x > y;
          a[i] = swap ? y : x;
          a[j] = swap ? x : y;
        }
      }
}

// Take the k largest keys out of the wave's sorted per-lane lists; lane r
// receives the r-th largest (0 once the wave runs out).
template <int N>
__device__ __forceinline__ uint64_t wave_extract(uint64_t (&a)[N], int k, int lane) {
  uint64_t mine = 0;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(a[0]);
    if (m == 0) break;                           // uniform: every lane sees the same maximum
    if (lane == r) mine = m;
    const bool pop = a[0] == m;                  // exactly one lane: the keys are unique
#pragma unroll
    for (int j = 0; j < N - 1; ++j) a[j] = pop ? a[j + 1] : a[j];
    a[N - 1] = pop ? 0 : a[N - 1];
  }
  return mine;
}

template <int ITEMS>
__global__ __launch_bounds__(kThreads) void topk_small_kernel(
    const float* __restrict__ scores, int64_t n, int k, const int32_t* excl, int n_excl, int64_t excl_stride,
    int32_t* ids_out, float* vals_out, int64_t out_stride) {
  __shared__ uint32_t excl_bits[kTile / 32];
  __shared__ uint64_t cand[kThreads / 64][kSmallMaxK];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n_excl > 0) {
    for (int i = tid; i < kTile / 32; i += kThreads) excl_bits[i] = 0;
    __syncthreads();
    for (int j = tid; j < n_excl; j += kThreads) {
      const int64_t id = excl[(size_t)b * excl_stride + j];
      if (id >= 0 && id < n) atomicOr(&excl_bits[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
  }
  uint64_t a[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int idx = i * kThreads + tid;
    const bool ok = idx < n && !(n_excl > 0 && ((excl_bits[idx >> 5] >> (idx & 31)) & 1u));
    a[i] = ok ? make_key(scores[(size_t)b * n + idx], (uint32_t)idx) : 0;
  }
  if (k >= 12 && k <= 16) {
    // Threshold pass (for smaller k the extraction below, k wave maxima, is
    // the quicker).  The 16 largest lane maxima of the row are 16 distinct
    // keys, so the 16th largest lane maximum T is at most the row's 16th
    // largest key: the keys >= T hold the top k.  Each wave sorts its lanes'
    // maxima, the waves' 16 largest (64 values) are sorted again by every
    // wave, and the keys >= T (16-20 of 2048 on random and on tied rows) are
    // sorted once more; no one-at-a-time extraction (k = 16 of 2048: 7.2 ->
    // 6.8 us for one row, 8.6 -> 7.8 us for 32).  More than 64 of them (not
    // seen in practice) take the extraction below.
    __shared__ uint64_t tops[kThreads / 64 * 16];
    __shared__ int wtot[kThreads / 64];
    uint64_t lm = a[0];
#pragma unroll
    for (int i = 1; i < ITEMS; ++i) lm = a[i] > lm ? a[i] : lm;
    const uint64_t srt = wave_sort_desc(lm, lane);
    if (lane < 16) tops[wave * 16 + lane] = srt;
    __syncthreads();
    const uint64_t st2 = wave_sort_desc(tops[lane], lane);
    const uint64_t T = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(st2 >> 32), 15) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)st2, 15);
    int c = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) c += (a[i] != 0 && a[i] >= T) ? 1 : 0;
    int incl = c;                                 // inclusive prefix of the counts over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int t = wtot[w];
      base += w < wave ? t : 0;
      total += t;
    }
    if (total <= 64) {                            // uniform over the workgroup
      uint64_t* list = &cand[0][0];
      int pos = base + incl - c;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
        if (a[i] != 0 && a[i] >= T) list[pos++] = a[i];
      __syncthreads();
      if (wave != 0) return;
      const uint64_t best = wave_sort_desc(lane < total ? list[lane] : 0, lane);
      if (lane < k) {
        ids_out[(size_t)b * out_stride + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
        if (vals_out) vals_out[(size_t)b * out_stride + lane] = unorder_score((uint32_t)(best >> 32));
      }
      return;
    }
  }
  sort_desc(a);
  const uint64_t mine = wave_extract(a, k, lane);
  if (lane < k) cand[wave][lane] = mine;
  __syncthreads();
  if (wave != 0) return;
  uint64_t best;
  if (k * (kThreads / 64) <= 64) {
    // at most 64 candidates: one per lane (wave w's r-th at lane 16 w + r), then one cross-lane sort
    const int w = lane >> 4, r = lane & 15;
    best = wave_sort_desc(r < k ? cand[w][r] : 0, lane);
  } else {
    uint64_t c[kThreads / 64];
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) c[w] = lane < k ? cand[w][lane] : 0;
    sort_desc(c);
    best = wave_extract(c, k, lane);
  }
  if (lane < k) {
    ids_out[(size_t)b * out_stride + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
    if (vals_out) vals_out[(size_t)b * out_stride + lane] = unorder_score((uint32_t)(best >> 32));
  }
}

inline int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace

size_t topk_workspace_bytes(int batch, int64_t n_docs, int k) {
  const int64_t tiles = (n_docs + kTile - 1) / kTile;
  if (tiles <= 1) return 0;
  return 2 * (size_t)batch * (size_t)tiles * (size_t)k * sizeof(uint64_t);
}

hipError_t launch_topk(const float* scores, int batch, int64_t n_docs, int k, int32_t* ids,
                       float* vals, void* ws, hipStream_t s) {
  return launch_topk_excl(scores, batch, n_docs, k, nullptr, 0, 0, ids, vals, k, ws, s);
}

hipError_t launch_topk_excl(const float* scores, int batch, int64_t n_docs, int k, const int32_t* excl,
                            int n_excl, int64_t excl_stride, int32_t* ids, float* vals,
                            int64_t out_stride, void* ws, hipStream_t s) {
  const int kp2 = next_pow2(k);
  int64_t tiles = (n_docs + kTile - 1) / kTile;
  if (tiles <= 1 && k <= kSmallMaxK) {
    if (n_docs <= kTile / 2)
      hipLaunchKernelGGL(topk_small_kernel<kItems / 2>, dim3(1, batch), dim3(kThreads), 0, s, scores, n_docs, k,
                         excl, n_excl, excl_stride, ids, vals, out_stride);
    else
      hipLaunchKernelGGL(topk_small_kernel<kItems>, dim3(1, batch), dim3(kThreads), 0, s, scores, n_docs, k, excl,
                         n_excl, excl_stride, ids, vals, out_stride);
    return hipGetLastError();
  }
  if (tiles <= 1) {
    hipLaunchKernelGGL((topk_tile_kernel<false, true>), dim3(1, batch), dim3(kThreads), 0, s,
                       scores, nullptr, n_docs, k, kp2, excl, n_excl, excl_stride, nullptr, ids, vals,
                       out_stride);
    return hipGetLastError();
  }
  uint64_t* buf[2];
  buf[0] = static_cast<uint64_t*>(ws);
  buf[1] = buf[0] + (size_t)batch * (size_t)tiles * (size_t)k;
  hipLaunchKernelGGL((topk_tile_kernel<false, false>), dim3((unsigned)tiles, batch), dim3(kThreads),
                     0, s, scores, nullptr, n_docs, k, kp2, excl, n_excl, excl_stride, buf[0], nullptr,
                     nullptr, 0);
  int cur = 0;
  int64_t n = tiles * k;
  for (;;) {
    tiles = (n + kTile - 1) / kTile;
    if (tiles == 1) {
      hipLaunchKernelGGL((topk_tile_kernel<true, true>), dim3(1, batch), dim3(kThreads), 0, s,
                         nullptr, buf[cur], n, k, kp2, nullptr, 0, 0, nullptr, ids, vals, out_stride);
      break;
    }
    hipLaunchKernelGGL((topk_tile_kernel<true, false>), dim3((unsigned)tiles, batch),
                       dim3(kThreads), 0, s, nullptr, buf[cur], n, k, kp2, nullptr, 0, 0, buf[cur ^ 1],
                       nullptr, nullptr, 0);
    cur ^= 1;
    n = tiles * k;
  }
  return hipGetLastError();
}

}  // namespace msa
