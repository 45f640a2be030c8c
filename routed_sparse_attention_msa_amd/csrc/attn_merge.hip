// Merge of two partial attentions over disjoint key sets.
//
// Method: the attention of the MSA layer runs over the gathered memory rows
// followed by the local rows (MSA README (EverMind-AI/MSA), "Inference
// Pipeline" stage 3; william-0g/MSA-Qwen3.5 model card, "Architecture
// summary").  A softmax over the union of two disjoint key sets K1, K2 is a
// weighted sum of the softmaxes over each: with lse_i = log sum_{j in K_i}
// exp(l_j) and o_i the attention output over K_i,
//
//   lse = log(exp(lse_1) + exp(lse_2)),
//   o   = exp(lse_1 - lse) o_1 + exp(lse_2 - lse) o_2.
//
// A part whose lse is -inf (no visible key) gets weight 0; with both at -inf
// the output is 0 and lse stays -inf.  The local rows of a decode step do not
// depend on routing, so their attention can run beside route, top-k and
// gather, and only the memory rows' attention and this merge wait for the
// gather.
//
// One wave per (sequence, token, query head) row; lane i takes the row's i-th
// 16 bytes.  Each lane reads its own bytes before writing them, and the lse
// word is written after every lane of the wave has read it, so the output
// may alias either input.
#include <cmath>

#include "internal.h"

namespace msa {
namespace {

constexpr int kWavesPerBlock = 4;

template <typename T>
__global__ __launch_bounds__(kWavesPerBlock * 64) void attn_merge_kernel(
    const T* o_a, const float* lse_a, const T* o_b, const float* lse_b, int64_t rows, int q_len,
    int heads_q, int dim, T* o, float* lse) {   // (no __restrict__: the output may alias an input)
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  // row = (b * q_len + t) * heads_q + h; the lse arrays are [batch, heads_q, q_len]
  const int h = (int)(row % heads_q);
  const int64_t bt = row / heads_q;
  const int t = (int)(bt % q_len);
  const int64_t b = bt / q_len;
  const int64_t li = (b * heads_q + h) * q_len + t;
  const float la = lse_a[li], lb = lse_b[li];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(la - m), eb = expf(lb - m);
    const float s = ea + eb;
    wa = ea / s;
    wb = eb / s;
    l = m + logf(s);
  }
  constexpr int N = Vec16<T>::N;
  if (lane < dim / N) {
    const size_t off = (size_t)row * dim + (size_t)lane * N;
    float a[N], c[N], r[N];
    Vec16<T>::widen(load16(o_a + off), a);
    Vec16<T>::widen(load16(o_b + off), c);
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = wa * a[i] + wb * c[i];
    store16(o + off, Vec16<T>::narrow(r));
  }
  if (lse != nullptr && lane == 0) lse[li] = l;
}

}  // namespace

hipError_t launch_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                             int batch, int q_len, int heads_q, int dim, msa_dtype dt, void* o, float* lse,
                             hipStream_t s) {
  const int64_t rows = (int64_t)batch * q_len * heads_q;
  const dim3 grid((unsigned)((rows + kWavesPerBlock - 1) / kWavesPerBlock));
  if (dt == MSA_BF16)
    hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, grid, dim3(kWavesPerBlock * 64), 0, s,
                       static_cast<const uint16_t*>(o_a), lse_a, static_cast<const uint16_t*>(o_b), lse_b, rows,
                       q_len, heads_q, dim, static_cast<uint16_t*>(o), lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<float>, grid, dim3(kWavesPerBlock * 64), 0, s,
                       static_cast<const float*>(o_a), lse_a, static_cast<const float*>(o_b), lse_b, rows, q_len,
                       heads_q, dim, static_cast<float*>(o), lse);
  return hipGetLastError();
}

}  // namespace msa
