// S1: chunk-mean pooling of document rows into the memory bank.
//
// Method: MSA README (EverMind-AI/MSA), "Overall Design" -- document K, V and
// router keys K_r are compressed by the mean over fixed-size chunks; "Inference
// Pipeline" stage 1 caches these pooled tensors offline.
//
// HBM-bound streaming kernel.  One workgroup reduces one chunk (all `chunk`
// rows of one document chunk) for one <= 4 KiB column segment of the row.
// Each thread owns 16 contiguous bytes of the row and walks the chunk's rows
// with a stride of `row_groups`; the row groups are then combined through
// LDS.  Loads are 16 B per lane and consecutive lanes read consecutive
// addresses, so every wave instruction touches whole 64 B segments.
// Accumulation is float32; the mean is rounded once (RNE) to the storage
// dtype, and the norm of the *stored* row is reduced across the lanes of
// each head with cross-lane shuffles.
#include "internal.h"

namespace msa {
namespace {

constexpr int kPoolThreads = 256;

template <typename T>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const T* __restrict__ x, T* __restrict__ xbar, float* __restrict__ norm, int chunk,
    int row_lanes, int seg_lanes, int row_groups, int lanes_per_head, int heads) {
  constexpr int N = Vec16<T>::N;
  __shared__ float red[kPoolThreads * N];

  const int tid = threadIdx.x;
  const int rg = tid / seg_lanes;
  const int lane = tid - rg * seg_lanes;
  const int col_lane = blockIdx.y * seg_lanes + lane;  // 16-byte slot within the row
  const bool active = rg < row_groups && col_lane < row_lanes;
  const size_t row_bytes = (size_t)row_lanes * 16;
  const size_t chunk_idx = blockIdx.x;

  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.f;

  if (active) {
    const char* base = reinterpret_cast<const char*>(x) + chunk_idx * (size_t)chunk * row_bytes +
                       (size_t)col_lane * 16;
    int r = rg;
    // 8 independent 16-byte loads in flight per thread per iteration.
    for (; r + 7 * row_groups < chunk; r += 8 * row_groups) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = load16(base + (size_t)(r + u * row_groups) * row_bytes);
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
      Vec16<T>::widen(load16(base + (size_t)r * row_bytes), f);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += f[i];
    }
  }

  if (row_groups > 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) red[tid * N + i] = acc[i];
    __syncthreads();
    if (rg == 0) {
      for (int g = 1; g < row_groups; ++g) {
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] += red[(g * seg_lanes + lane) * N + i];
      }
    }
  }

  float sq = 0.f;
  if (rg == 0 && col_lane < row_lanes) {
    const float inv_div = (float)chunk;
    float mean[N];
#pragma unroll
    for (int i = 0; i < N; ++i) mean[i] = acc[i] / inv_div;
    u32x4 packed = Vec16<T>::narrow(mean);
    store16(reinterpret_cast<char*>(xbar) + chunk_idx * row_bytes + (size_t)col_lane * 16, packed);
    if (norm != nullptr) {
      float stored[N];
      Vec16<T>::widen(packed, stored);
#pragma unroll
      for (int i = 0; i < N; ++i) sq += stored[i] * stored[i];
    }
  }
  if (norm != nullptr) {
    // Sum of squares across the lanes of one head (lanes_per_head is a power
    // of two <= 64 and heads start at multiples of it, so a head never
    // straddles a wave).  Every lane of the wave takes part in the shuffles.
    for (int off = lanes_per_head >> 1; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if (rg == 0 && col_lane < row_lanes && (col_lane % lanes_per_head) == 0) {
      const int h = col_lane / lanes_per_head;
      norm[chunk_idx * (size_t)heads + h] = sqrtf(sq);
    }
  }
}

template <typename T>
hipError_t launch_pool_t(const void* x, void* xbar, float* norm, int64_t n_chunks, int chunk,
                         int heads, int dim, hipStream_t s) {
  const int row_lanes = (int)((size_t)heads * dim * sizeof(T) / 16);
  const int seg_lanes = row_lanes < kPoolThreads ? row_lanes : kPoolThreads;
  const int segments = (row_lanes + seg_lanes - 1) / seg_lanes;
  const int row_groups = kPoolThreads / seg_lanes;
  const int lanes_per_head = (int)(dim * sizeof(T) / 16);
  dim3 grid((unsigned)n_chunks, (unsigned)segments);
  hipLaunchKernelGGL(pool_kernel<T>, grid, dim3(kPoolThreads), 0, s, static_cast<const T*>(x),
                     static_cast<T*>(xbar), norm, chunk, row_lanes, seg_lanes, row_groups,
                     lanes_per_head, heads);
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
