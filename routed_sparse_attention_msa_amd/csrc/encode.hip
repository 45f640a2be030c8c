// Offline encoder: chunk means of variable-length documents, with the
// document-wise rotary position embedding of K fused in front of the mean.
//
// Method: MSA README (EverMind-AI/MSA), "Overall Design" -- document K, V and
// router keys K_r are compressed by the mean over fixed-size chunks, K having
// been rotated by document-wise RoPE; "Inference Pipeline" stage 1 encodes the
// memory offline.  Documents are row ranges [doc_off[n], doc_off[n+1]) of one
// tensor; the last chunk of a document may be short, and its mean is over the
// rows present.  RoPE is the rotate-half form: for k < d/2 the pair
// (x_k, x_{k+d/2}) turns by position * base^(-2k/d), the position counting
// from 0 at the document's first row.
//
// Same streaming design as the pool kernel (one round of workgroups over
// contiguous chunk ranges, 16-byte column slots, row groups merged through
// LDS, pooled rows staged in LDS and written together, non-temporal
// accesses).  Per chunk a workgroup reads its document's offsets with scalar
// loads: one binary search for its first chunk, then a forward walk.  The
// rotation: a lane reads 8 bytes from each half of one head, so it holds the
// rotation partners (x_k, x_{k+d/2}) itself and one (cos, sin) pair serves
// two elements.  Each chunk restarts the angles exactly (position * theta in
// float64, reduced modulo 2 pi, then sincos), and the rows inside a chunk
// advance them by a fixed float32 rotation, so the angle error stays at a
// few 1e-6 rad whatever the document length.
#include <algorithm>
#include <map>
#include <mutex>

#include "internal.h"

namespace msa {
namespace {

constexpr int kEncThreads = 256;
constexpr int kEncMaxStage = 32;
constexpr size_t kEncStageBytes = 64 * 1024;
constexpr double kTwoPi = 6.283185307179586476925286766559;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 load8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// ---------------------------------------------------------------------------
// chunk offsets: chunk_off[0] = 0, chunk_off[n+1] = chunk_off[n] + ceil(L_n / chunk)
// One workgroup: tiles of 1024 documents, a block scan, and a running carry.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int64_t* __restrict__ doc_off,
                                                            int64_t n_docs, int chunk,
                                                            int64_t* __restrict__ chunk_off) {
  __shared__ long long wsum[16];
  __shared__ long long carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    carry_s = 0;
    chunk_off[0] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < n_docs; base += 1024) {
    const int64_t n = base + tid;
    int64_t c = 0;
    if (n < n_docs) {
      const int64_t len = doc_off[n + 1] - doc_off[n];
      c = len > 0 ? (len + chunk - 1) / chunk : 0;
    }
    // inclusive scan inside the wave, then across waves
    long long v = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long o = __shfl_up(v, off);
      if (lane >= off) v += o;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    long long before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (n < n_docs) chunk_off[n + 1] = before + v;
    __syncthreads();
    if (tid == 1023) carry_s = before + v;   // the tile's last document (or past the end: sum unchanged)
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// encoder
// ---------------------------------------------------------------------------
template <typename T, bool ROPE>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(
    const T* __restrict__ x, T* __restrict__ xbar, float* __restrict__ norm,
    const int64_t* __restrict__ doc_off, const int64_t* __restrict__ chunk_off, int64_t n_docs,
    int64_t total_rows, int64_t total_chunks, int chunk, int row_lanes, int seg_lanes,
    int row_groups, int lanes_per_head, int heads, int dim, float log2_base, int stage_cap) {
  constexpr int N = Vec16<T>::N;
  extern __shared__ u32x4 stage[];   // rows [cap][seg_lanes], norms [cap][heads_seg], partial sums x2

  const int tid = threadIdx.x;
  const int rg = tid / seg_lanes;
  const int lane = tid - rg * seg_lanes;
  const int col_lane = blockIdx.y * seg_lanes + lane;
  const bool in_row = col_lane < row_lanes;
  const size_t row_bytes = (size_t)row_lanes * 16;
  const int64_t lo = (int64_t)blockIdx.x * total_chunks / gridDim.x;
  const int64_t hi = ((int64_t)blockIdx.x + 1) * total_chunks / gridDim.x;
  const int heads_seg = norm != nullptr ? seg_lanes / lanes_per_head : 0;
  const int seg_valid = min(seg_lanes, row_lanes - (int)blockIdx.y * seg_lanes);
  const int h0 = (int)blockIdx.y * heads_seg;
  const int hv = min(heads_seg, heads - h0);
  float* snorm = reinterpret_cast<float*>(stage + (size_t)stage_cap * seg_lanes);
  float* red0 = snorm + (size_t)stage_cap * heads_seg;
  const int red_len = (kEncThreads - seg_lanes) * N;
  char* out = reinterpret_cast<char*>(xbar);

  // With RoPE a lane holds N/2 elements of each half of its head (8 bytes at
  // in_head * 8 in the low half, the same in the high half), so it holds its
  // own rotation partners: element e < N/2 of acc is frequency f0 + e of the
  // low half, element N/2 + e its partner.  Without RoPE a lane holds 16
  // consecutive bytes.
  constexpr int H2 = ROPE ? N / 2 : 1;
  const int in_head = col_lane % lanes_per_head;
  const int f0 = in_head * (N / 2);
  double theta[H2];
  float cstep[H2], sstep[H2];
  if constexpr (ROPE) {
#pragma unroll
    for (int e = 0; e < H2; ++e) {
      theta[e] = exp2(-2.0 * (double)(f0 + e) / (double)dim * (double)log2_base);
      sincosf((float)fmod((double)row_groups * theta[e], kTwoPi), &sstep[e], &cstep[e]);
    }
  }
  // byte offsets of this lane's data inside a row (lanes past the row: slot 0)
  const size_t lo_off = !in_row ? 0
                        : ROPE ? (size_t)(col_lane - in_head) * 16 + (size_t)in_head * 8
                               : (size_t)col_lane * 16;
  const size_t hi_off = lo_off + (in_row ? (size_t)lanes_per_head * 8 : 0);
  const int st_lo = ROPE ? (lane - in_head) * 16 + in_head * 8 : lane * 16;
  const int st_hi = st_lo + lanes_per_head * 8;

  if (lo >= hi) return;
  // document of the first chunk: the last n with chunk_off[n] <= lo
  int64_t n = 0;
  {
    int64_t a = 0, b = n_docs - 1;
    while (a < b) {
      const int64_t mid = (a + b + 1) >> 1;
      if (chunk_off[mid] <= lo) a = mid; else b = mid - 1;
    }
    n = a;
  }

  int parity = 0;
  for (int64_t c0 = lo; c0 < hi; c0 += stage_cap) {
    const int n_here = (int)(hi - c0 < stage_cap ? hi - c0 : stage_cap);
    for (int m = 0; m < n_here; ++m, parity ^= 1) {
      const int64_t ci = c0 + m;
      while (n + 1 < n_docs && chunk_off[n + 1] <= ci) ++n;
      const int64_t j = ci - chunk_off[n];
      const int64_t r0 = doc_off[n] + j * chunk;
      // malformed offsets read nothing out of bounds (the chunk comes out empty)
      int64_t left = (r0 >= 0 && r0 < total_rows) ? min(doc_off[n + 1], total_rows) - r0 : 0;
      const int cnt = (int)(left < chunk ? (left > 0 ? left : 0) : chunk);

      float acc[N];
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] = 0.f;
      float cs[H2], sn[H2];
      if constexpr (ROPE) {
        const double p0 = (double)(j * chunk + rg);
#pragma unroll
        for (int e = 0; e < H2; ++e) sincosf((float)fmod(p0 * theta[e], kTwoPi), &sn[e], &cs[e]);
      }
      auto add_row = [&](const u32x4& raw) {
        float f[N];
        Vec16<T>::widen(raw, f);
        if constexpr (ROPE) {
#pragma unroll
          for (int e = 0; e < H2; ++e) {
            acc[e] += f[e] * cs[e] - f[H2 + e] * sn[e];
            acc[H2 + e] += f[H2 + e] * cs[e] + f[e] * sn[e];
            const float c2 = cs[e] * cstep[e] - sn[e] * sstep[e];
            sn[e] = sn[e] * cstep[e] + cs[e] * sstep[e];
            cs[e] = c2;
          }
        } else {
#pragma unroll
          for (int e = 0; e < N; ++e) acc[e] += f[e];
        }
      };
      auto load_row = [&](const char* row) -> u32x4 {
        if constexpr (ROPE) {
          const u32x2 a = load8_stream(row + lo_off);
          const u32x2 b = load8_stream(row + hi_off);
          return u32x4{a[0], a[1], b[0], b[1]};
        } else {
          return load16_stream(row + lo_off);
        }
      };

      // every lane of a row group walks the same rows; loads are
      // unconditional (lanes past the row read slot 0 of the same row and
      // drop it): a branch per load would make the compiler wait for every
      // load in flight at each join
      if (rg < row_groups) {
        const char* base = reinterpret_cast<const char*>(x) + (size_t)r0 * row_bytes;
        int r = rg;
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (; r + 7 * row_groups < cnt; r += 8 * row_groups) {
          u32x4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = load_row(base + (size_t)(r + u * row_groups) * row_bytes);
#pragma unroll
          for (int u = 0; u < 8; ++u) add_row(in_row ? v[u] : z);
        }
        for (; r < cnt; r += row_groups) {
          const u32x4 v = load_row(base + (size_t)r * row_bytes);
          add_row(in_row ? v : z);
        }
      }

      if (row_groups > 1) {
        float* rb = red0 + parity * red_len;
        if (rg > 0) {
#pragma unroll
          for (int i = 0; i < N; ++i) rb[(tid - seg_lanes) * N + i] = acc[i];
        }
        __syncthreads();
        if (rg == 0) {
          for (int g = 1; g < row_groups; ++g) {
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] += rb[((g - 1) * seg_lanes + lane) * N + i];
          }
        }
      }

      float sq = 0.f;
      if (rg == 0 && in_row) {
        const float div = (float)(cnt > 0 ? cnt : 1);
        float mean[N];
#pragma unroll
        for (int i = 0; i < N; ++i) mean[i] = acc[i] / div;
        const u32x4 packed = Vec16<T>::narrow(mean);
        char* srow = reinterpret_cast<char*>(stage + (size_t)m * seg_lanes);
        if constexpr (ROPE) {
          *reinterpret_cast<u32x2*>(srow + st_lo) = u32x2{packed[0], packed[1]};
          *reinterpret_cast<u32x2*>(srow + st_hi) = u32x2{packed[2], packed[3]};
        } else {
          *reinterpret_cast<u32x4*>(srow + st_lo) = packed;
        }
        if (norm != nullptr) {
          float stored[N];
          Vec16<T>::widen(packed, stored);
#pragma unroll
          for (int i = 0; i < N; ++i) sq += stored[i] * stored[i];
        }
      }
      if (norm != nullptr) {
        for (int off = lanes_per_head >> 1; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
        if (rg == 0 && in_row && (lane % lanes_per_head) == 0)
          snorm[m * heads_seg + lane / lanes_per_head] = sqrtf(sq);
      }
    }
    __syncthreads();
    for (int i = tid; i < n_here * seg_lanes; i += kEncThreads) {
      const int m = i / seg_lanes;
      const int l = i - m * seg_lanes;
      if (l < seg_valid)
        store16_stream(out + (size_t)(c0 + m) * row_bytes + (size_t)(blockIdx.y * seg_lanes + l) * 16,
                       stage[i]);
    }
    if (norm != nullptr) {
      for (int i = tid; i < n_here * heads_seg; i += kEncThreads) {
        const int m = i / heads_seg;
        const int hh = i - m * heads_seg;
        if (hh < hv) norm[(size_t)(c0 + m) * heads + h0 + hh] = snorm[i];
      }
    }
    __syncthreads();
  }
}

template <typename T, bool ROPE>
int enc_occupancy(size_t smem) {
  static std::mutex mu;
  static std::map<size_t, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(smem);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(encode_kernel<T, ROPE>),
                                                   kEncThreads, smem) != hipSuccess)
    nb = 0;
  cache[smem] = nb;
  return nb;
}

template <typename T, bool ROPE>
hipError_t launch_encode_t(const void* x, void* xbar, float* norm, const int64_t* doc_off,
                           const int64_t* chunk_off, int64_t n_docs, int64_t total_rows,
                           int64_t total_chunks, int chunk, int heads, int dim, float rope_base,
                           hipStream_t s) {
  const int row_lanes = (int)((size_t)heads * dim * sizeof(T) / 16);
  const int seg_lanes = row_lanes < kEncThreads ? row_lanes : kEncThreads;
  const int segments = (row_lanes + seg_lanes - 1) / seg_lanes;
  const int row_groups = kEncThreads / seg_lanes;
  const bool head_lanes = norm != nullptr || ROPE;
  const int lanes_per_head = head_lanes ? (int)(dim * sizeof(T) / 16) : seg_lanes;
  const int heads_seg = norm != nullptr ? seg_lanes / lanes_per_head : 0;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(encode_kernel<T, ROPE>), hipFuncAttributeMaxDynamicSharedMemorySize,
      96 * 1024);
  if (attr != hipSuccess) return attr;
  const size_t per_chunk_stage = (size_t)seg_lanes * 16 + (size_t)heads_seg * 4;
  const size_t red_bytes = (size_t)2 * (kEncThreads - seg_lanes) * Vec16<T>::N * sizeof(float);
  int cap = (int)std::min<size_t>(kEncMaxStage, kEncStageBytes / per_chunk_stage);
  int occ = 0;
  for (;;) {
    occ = enc_occupancy<T, ROPE>(cap * per_chunk_stage + red_bytes);
    if (occ >= 2 || cap == 1) break;
    cap = std::max(1, cap * 3 / 4);
  }
  occ = std::max(occ, 1);
  const int64_t slots = (int64_t)occ * device_cu_count() / segments;
  const int64_t blocks_x = std::max<int64_t>(1, std::min<int64_t>(total_chunks, slots));
  const int64_t per_block = (total_chunks + blocks_x - 1) / blocks_x;
  if (per_block < cap) cap = (int)per_block;
  const size_t smem = (size_t)cap * per_chunk_stage + red_bytes;
  const float log2_base = ROPE ? log2f(rope_base) : 0.f;
  hipLaunchKernelGGL((encode_kernel<T, ROPE>), dim3((unsigned)blocks_x, (unsigned)segments),
                     dim3(kEncThreads), smem, s, static_cast<const T*>(x), static_cast<T*>(xbar), norm,
                     doc_off, chunk_off, n_docs, total_rows, total_chunks, chunk, row_lanes, seg_lanes,
                     row_groups, lanes_per_head, heads, dim, log2_base, cap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_offsets(const int64_t* doc_off, int64_t n_docs, int chunk, int64_t* chunk_off,
                                hipStream_t s) {
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, s, doc_off, n_docs, chunk, chunk_off);
  return hipGetLastError();
}

hipError_t launch_encode(const void* x, void* xbar, float* norm, const int64_t* doc_off,
                         const int64_t* chunk_off, int64_t n_docs, int64_t total_rows,
                         int64_t total_chunks, int chunk, int heads, int dim, float rope_base,
                         msa_dtype dt, hipStream_t s) {
  if (total_chunks == 0 || n_docs == 0) return hipSuccess;
  const bool rope = rope_base > 0.f;
#define MSA_ENC(T, R)                                                                                \
  launch_encode_t<T, R>(x, xbar, norm, doc_off, chunk_off, n_docs, total_rows, total_chunks, chunk, \
                        heads, dim, rope_base, s)
  if (dt == MSA_F32) return rope ? MSA_ENC(float, true) : MSA_ENC(float, false);
  return rope ? MSA_ENC(uint16_t, true) : MSA_ENC(uint16_t, false);
#undef MSA_ENC
}

}  // namespace msa
