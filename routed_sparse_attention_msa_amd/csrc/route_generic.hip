// S2 (any shape, float32 or bf16): cosine routing with plain vector ALU code.
//
// Method: MSA README (EverMind-AI/MSA), "Overall Design" -- cosine similarity
// per head, averaged over heads, maximised over the query tokens; this
// implementation also maximises over the document's chunks.
//
// This is the shape-general path (any head count, head dim and chunks per
// document).  One workgroup scores one document for one sequence: each
// thread takes query tokens t = tid, tid+256, ..., evaluates the head-mean
// cosine against each of the document's chunks, keeps the running maximum,
// and the block reduces the maxima.  The bf16 MFMA path in route.hip serves
// the production shapes.
#include "internal.h"

namespace msa {

namespace {
constexpr int kThreads = 256;
constexpr float kEps = 1e-12f;
}  // namespace

template <typename T>
__global__ __launch_bounds__(kThreads) void route_generic_kernel(
    const T* __restrict__ q_r, const T* __restrict__ kbar, const float* __restrict__ knorm,
    int q_len, int heads, int dim, int64_t n_docs, int cpd, float* __restrict__ out) {
  __shared__ float red[kThreads / 64];
  const int64_t doc = blockIdx.x;
  const int b = blockIdx.y;
  const size_t row = (size_t)heads * dim;
  float best = -INFINITY;
  for (int t = threadIdx.x; t < q_len; t += kThreads) {
    const T* q = q_r + ((size_t)b * q_len + t) * row;
    for (int j = 0; j < cpd; ++j) {
      const size_t n = (size_t)doc * cpd + j;
      const T* kr = kbar + n * row;
      float s = 0.f;
      for (int h = 0; h < heads; ++h) {
        float dot = 0.f, qq = 0.f;
        for (int e = 0; e < dim; ++e) {
          const float qv = Elem<T>::to_f32(q[h * dim + e]);
          const float kv = Elem<T>::to_f32(kr[h * dim + e]);
          dot += qv * kv;
          qq += qv * qv;
        }
        s += dot / (fmaxf(sqrtf(qq), kEps) * fmaxf(knorm[n * heads + h], kEps));
      }
      best = fmaxf(best, s / (float)heads);
    }
  }
  for (int off = 32; off > 0; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
    out[(size_t)b * n_docs + doc] = m;
  }
}

hipError_t launch_route_generic(const void* q_r, const void* kbar_r, const float* knorm, int batch,
                                int q_len, int heads, int dim, int64_t n_docs, int cpd,
                                msa_dtype dt, float* doc_scores, hipStream_t s) {
  dim3 grid((unsigned)n_docs, batch);
  if (dt == MSA_F32) {
    hipLaunchKernelGGL(route_generic_kernel<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(q_r), static_cast<const float*>(kbar_r), knorm,
                       q_len, heads, dim, n_docs, cpd, doc_scores);
  } else {
    hipLaunchKernelGGL(route_generic_kernel<uint16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(q_r), static_cast<const uint16_t*>(kbar_r),
                       knorm, q_len, heads, dim, n_docs, cpd, doc_scores);
  }
  return hipGetLastError();
}

}  // namespace msa
