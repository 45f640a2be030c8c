// S1: chunk-mean pooling of document rows into the memory bank.
//
// Method: MSA README (EverMind-AI/MSA), "Overall Design" -- document K, V and
// router keys K_r are compressed by the mean over fixed-size chunks; "Inference
// Pipeline" stage 1 caches these pooled tensors offline.
//
// HBM-bound streaming kernel.  One round of workgroups; each pools a
// contiguous range of chunks (all `chunk` rows of each) for one <= 4 KiB
// column segment of the row.  Each thread owns 16 contiguous bytes of the
// row and walks a chunk's rows with a stride of `row_groups`; the row groups
// are combined through LDS.  Loads are 16 B per lane and consecutive lanes
// read consecutive addresses, so every wave instruction touches whole 64 B
// segments.  Accumulation is float32; the mean is rounded once (RNE) to the
// storage dtype, and the norm of the *stored* row is reduced across the
// lanes of each head with cross-lane shuffles.
//
// The pooled rows and norms are held in LDS and written out together, up to
// 32 chunks at a time.  Writes scattered between the reads (2 KiB after
// every 128 KiB at the 1M-token bank) cost ~15% of the read bandwidth;
// grouped, they cost about their own size.  Input and output are touched
// once, so both use non-temporal accesses.
#include <algorithm>
#include <map>
#include <mutex>

#include "internal.h"

namespace msa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kPoolMaxStage = 32;               // chunks held in LDS before a write-out
constexpr size_t kPoolStageBytes = 64 * 1024;  // bound on the LDS holding pooled rows

// Workgroup b (of gridDim.x) pools the contiguous chunk range
// [b*n/G, (b+1)*n/G), `stage_cap` chunks at a time.
template <typename T>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const T* __restrict__ x, T* __restrict__ xbar, float* __restrict__ norm, int64_t n_chunks,
    int chunk, int row_lanes, int seg_lanes, int row_groups, int lanes_per_head, int heads,
    int stage_cap) {
  constexpr int N = Vec16<T>::N;
  // LDS: pooled rows [stage_cap][seg_lanes], norms [stage_cap][heads_seg],
  // then two buffers of the partial sums of row groups 1.. [threads - seg_lanes][N].
  extern __shared__ u32x4 stage[];

  const int tid = threadIdx.x;
  const int rg = tid / seg_lanes;
  const int lane = tid - rg * seg_lanes;
  const int col_lane = blockIdx.y * seg_lanes + lane;  // 16-byte slot within the row
  const bool in_row = col_lane < row_lanes;
  const bool active = rg < row_groups && in_row;
  const size_t row_bytes = (size_t)row_lanes * 16;
  const int64_t lo = (int64_t)blockIdx.x * n_chunks / gridDim.x;
  const int64_t hi = ((int64_t)blockIdx.x + 1) * n_chunks / gridDim.x;
  const int heads_seg = norm != nullptr ? seg_lanes / lanes_per_head : 0;
  const int seg_valid = min(seg_lanes, row_lanes - (int)blockIdx.y * seg_lanes);
  const int h0 = (int)blockIdx.y * heads_seg;
  const int hv = min(heads_seg, heads - h0);
  float* snorm = reinterpret_cast<float*>(stage + (size_t)stage_cap * seg_lanes);
  float* red0 = snorm + (size_t)stage_cap * heads_seg;
  const int red_len = (kPoolThreads - seg_lanes) * N;
  char* out = reinterpret_cast<char*>(xbar);

  int parity = 0;
  for (int64_t c0 = lo; c0 < hi; c0 += stage_cap) {
    const int n_here = (int)(hi - c0 < stage_cap ? hi - c0 : stage_cap);
    for (int m = 0; m < n_here; ++m, parity ^= 1) {
      const size_t chunk_idx = (size_t)(c0 + m);
      float acc[N];
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] = 0.f;

      if (active) {
        const char* base = reinterpret_cast<const char*>(x) +
                           chunk_idx * (size_t)chunk * row_bytes + (size_t)col_lane * 16;
        int r = rg;
        // 8 independent 16-byte loads in flight per thread per iteration.
        for (; r + 7 * row_groups < chunk; r += 8 * row_groups) {
          u32x4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            v[u] = load16_stream(base + (size_t)(r + u * row_groups) * row_bytes);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            float f[N];
            Vec16<T>::widen(v[u], f);
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] += f[i];
          }
        }
        for (; r < chunk; r += row_groups) {
          float f[N];
          Vec16<T>::widen(load16_stream(base + (size_t)r * row_bytes), f);
#pragma unroll
          for (int i = 0; i < N; ++i) acc[i] += f[i];
        }
      }

      if (row_groups > 1) {
        // Double-buffered: a thread can write this buffer again only after
        // the next chunk's barrier, which row group 0 reaches after reading it.
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
        const float div = (float)chunk;
        float mean[N];
#pragma unroll
        for (int i = 0; i < N; ++i) mean[i] = acc[i] / div;
        const u32x4 packed = Vec16<T>::narrow(mean);
        stage[(size_t)m * seg_lanes + lane] = packed;
        if (norm != nullptr) {
          float stored[N];
          Vec16<T>::widen(packed, stored);
#pragma unroll
          for (int i = 0; i < N; ++i) sq += stored[i] * stored[i];
        }
      }
      if (norm != nullptr) {
        // Sum of squares across the lanes of one head (lanes_per_head is a
        // power of two <= 64 and heads start at multiples of it, so a head
        // never straddles a wave).  Every lane of the wave takes part.
        for (int off = lanes_per_head >> 1; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
        if (rg == 0 && in_row && (lane % lanes_per_head) == 0)
          snorm[m * heads_seg + lane / lanes_per_head] = sqrtf(sq);
      }
    }
    __syncthreads();

    // Write out the staged rows (and norms) of these chunks.
    for (int i = tid; i < n_here * seg_lanes; i += kPoolThreads) {
      const int m = i / seg_lanes;
      const int l = i - m * seg_lanes;
      if (l < seg_valid)
        store16_stream(out + (size_t)(c0 + m) * row_bytes + (size_t)(blockIdx.y * seg_lanes + l) * 16,
                       stage[i]);
    }
    if (norm != nullptr) {
      for (int i = tid; i < n_here * heads_seg; i += kPoolThreads) {
        const int m = i / heads_seg;
        const int h = i - m * heads_seg;
        if (h < hv) norm[(size_t)(c0 + m) * heads + h0 + h] = snorm[i];
      }
    }
    __syncthreads();  // the stage is reused by the next group of chunks
  }
}

// Resident workgroups per CU for a given dynamic LDS size (cached).
template <typename T>
int pool_occupancy(size_t smem) {
  static std::mutex mu;
  static std::map<size_t, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(smem);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(pool_kernel<T>),
                                                   kPoolThreads, smem) != hipSuccess)
    n = 0;
  cache[smem] = n;
  return n;
}

template <typename T>
hipError_t launch_pool_t(const void* x, void* xbar, float* norm, int64_t n_chunks, int chunk,
                         int heads, int dim, hipStream_t s) {
  const int row_lanes = (int)((size_t)heads * dim * sizeof(T) / 16);
  const int seg_lanes = row_lanes < kPoolThreads ? row_lanes : kPoolThreads;
  const int segments = (row_lanes + seg_lanes - 1) / seg_lanes;
  const int row_groups = kPoolThreads / seg_lanes;
  // Norms need whole heads of a power-of-two number of 16-byte lanes (the
  // entry point checks this); without norms the head split is not used.
  const int lanes_per_head = norm != nullptr ? (int)(dim * sizeof(T) / 16) : seg_lanes;
  const int heads_seg = norm != nullptr ? seg_lanes / lanes_per_head : 0;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(pool_kernel<T>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     96 * 1024);
  if (attr != hipSuccess) return attr;

  // One round of workgroups, each over a contiguous, balanced range of
  // chunks.  The stage holds up to 32 chunks (the whole range at the 1M-token
  // bank, so all writes come at the end); it shrinks until at least two
  // workgroups fit on a CU.
  const size_t per_chunk_stage = (size_t)seg_lanes * 16 + (size_t)heads_seg * 4;
  const size_t red_bytes = (size_t)2 * (kPoolThreads - seg_lanes) * Vec16<T>::N * sizeof(float);
  int cap = (int)std::min<size_t>(kPoolMaxStage, kPoolStageBytes / per_chunk_stage);
  int occ = 0;
  for (;;) {
    occ = pool_occupancy<T>(cap * per_chunk_stage + red_bytes);
    if (occ >= 2 || cap == 1) break;
    cap = std::max(1, cap * 3 / 4);
  }
  occ = std::max(occ, 1);
  const int64_t slots = (int64_t)occ * device_cu_count() / segments;
  const int64_t blocks_x = std::max<int64_t>(1, std::min<int64_t>(n_chunks, slots));
  const int64_t per_block = (n_chunks + blocks_x - 1) / blocks_x;
  if (per_block < cap) cap = (int)per_block;
  const size_t smem = (size_t)cap * per_chunk_stage + red_bytes;
  dim3 grid((unsigned)blocks_x, (unsigned)segments);
  hipLaunchKernelGGL(pool_kernel<T>, grid, dim3(kPoolThreads), smem, s, static_cast<const T*>(x),
                     static_cast<T*>(xbar), norm, n_chunks, chunk, row_lanes, seg_lanes, row_groups,
                     lanes_per_head, heads, cap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const void* x, void* xbar, float* norm, int64_t n_chunks, int chunk,
                       int heads, int dim, msa_dtype dt, hipStream_t s) {
  if (n_chunks == 0) return hipSuccess;
  if (dt == MSA_F32) return launch_pool_t<float>(x, xbar, norm, n_chunks, chunk, heads, dim, s);
  return launch_pool_t<uint16_t>(x, xbar, norm, n_chunks, chunk, heads, dim, s);
}

}  // namespace msa
