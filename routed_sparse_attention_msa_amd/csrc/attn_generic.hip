// S5/S6 (any shape, float32 or bf16): sparse GQA attention with plain vector
// ALU code.
//
// Method: william-0g/MSA-Qwen3.5 model card, "Architecture summary" -- in the
// softmax layers the selected chunks' K/V are concatenated with the local KV;
// MSA README, "Inference Pipeline" stage 3 -- generation runs over that
// sparse context.  Causal alignment is bottom-right: query token t sees the
// M memory rows and local rows 0 .. L_loc - T + t.
//
// Shape-general path (any head dim <= 256, any group size).  One wavefront
// owns one (sequence, token, query head) row; each lane holds up to four
// elements of the head dim.  Per key: a wave-wide dot product (xor-shuffle
// reduction), an online-softmax update, and the value accumulation.  The
// bf16 MFMA kernels in attn_prefill.hip / attn_decode.hip serve the
// production shapes.
#include "internal.h"

namespace msa {

namespace {
constexpr int kThreads = 256;
constexpr int kMaxPerLane = 4;  // head dim <= 256
}  // namespace

template <typename T>
__global__ __launch_bounds__(kThreads) void attn_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k_sel, const T* __restrict__ v_sel, int mem_len,
    const T* __restrict__ k_loc, const T* __restrict__ v_loc, int loc_len, int batch, int q_len,
    int heads_q, int heads_kv, int dim, float scale, T* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t n_rows = (int64_t)batch * q_len * heads_q;
  if (row >= n_rows) return;  // whole wave exits together
  const int h = (int)(row % heads_q);
  const int t = (int)((row / heads_q) % q_len);
  const int b = (int)(row / ((int64_t)heads_q * q_len));
  const int g = h / (heads_q / heads_kv);

  float qv[kMaxPerLane], acc[kMaxPerLane];
  const T* qrow = q + (((size_t)b * q_len + t) * heads_q + h) * dim;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    qv[i] = e < dim ? Elem<T>::to_f32(qrow[e]) : 0.f;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int n_vis = mem_len + loc_len - q_len + t + 1;
  for (int j = 0; j < n_vis; ++j) {
    const T *kr, *vr;
    if (j < mem_len) {
      const size_t off = (((size_t)b * mem_len + j) * heads_kv + g) * dim;
      kr = k_sel + off;
      vr = v_sel + off;
    } else {
      const size_t off = (((size_t)b * loc_len + (j - mem_len)) * heads_kv + g) * dim;
      kr = k_loc + off;
      vr = v_loc + off;
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < dim) dot += qv[i] * Elem<T>::to_f32(kr[e]);
    }
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
    const float logit = dot * scale;
    const float m_new = fmaxf(m, logit);
    const float alpha = expf(m - m_new);
    const float p = expf(logit - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      const float vv = e < dim ? Elem<T>::to_f32(vr[e]) : 0.f;
      acc[i] = acc[i] * alpha + p * vv;
    }
    m = m_new;
  }
  T* orow = out + (((size_t)b * q_len + t) * heads_q + h) * dim;
  const float inv_l = 1.f / l;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    if (e < dim) orow[e] = Elem<T>::from_f32(acc[i] * inv_l);
  }
  if (lse != nullptr && lane == 0) lse[((size_t)b * heads_q + h) * q_len + t] = m + logf(l);
}

hipError_t launch_attn_generic(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                               const void* k_loc, const void* v_loc, int loc_len, int batch,
                               int q_len, int heads_q, int heads_kv, int dim, float scale,
                               msa_dtype dt, void* out, float* lse, hipStream_t s) {
  const int64_t rows = (int64_t)batch * q_len * heads_q;
  const unsigned blocks = (unsigned)((rows + (kThreads / 64) - 1) / (kThreads / 64));
  if (dt == MSA_F32) {
    hipLaunchKernelGGL(attn_generic_kernel<float>, dim3(blocks), dim3(kThreads), 0, s,
                       static_cast<const float*>(q), static_cast<const float*>(k_sel),
                       static_cast<const float*>(v_sel), mem_len, static_cast<const float*>(k_loc),
                       static_cast<const float*>(v_loc), loc_len, batch, q_len, heads_q, heads_kv,
                       dim, scale, static_cast<float*>(out), lse);
  } else {
    hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, dim3(blocks), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_sel),
                       static_cast<const uint16_t*>(v_sel), mem_len,
                       static_cast<const uint16_t*>(k_loc), static_cast<const uint16_t*>(v_loc),
                       loc_len, batch, q_len, heads_q, heads_kv, dim, scale,
                       static_cast<uint16_t*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace msa
