// Linear-layer variant: injection of the selected documents' states and the
// gated delta rule over a sequence from that initial state.
//
// Method: william-0g/MSA-Qwen3.5 model card, "Architecture summary" -- in the
// linear (gated-delta) layers each document is encoded through the layer's
// recurrence, the top-k documents (routed on the chunk-pooled router keys as
// in the softmax layers) have their recurrent states summed into S_ext, and
// the query path runs the gated delta rule with S_ext as its initial state.
// The rule is the published gated delta rule, per (sequence, head), with the
// state h[dk][dv]:
//     h <- alpha_t h;   u = h^T k_t;   h <- h + k_t (beta_t (v_t - u))^T;   o_t = scale h^T q_t
// with alpha_t = exp(g_t).
//
// State sum: one thread per 4 floats of a sequence's [H, dk, dv] state,
// summing the k documents in rank order (deterministic), HBM-bound.
//
// Recurrence: the state's value columns evolve independently (they share
// only k_t, q_t, alpha_t, beta_t), so a lane owns one value column and holds
// its dk entries in registers; a wave covers 64 columns and needs no
// cross-lane reduction at all.  Tokens are staged 32 at a time in LDS as
// float32 (q and k broadcast to every lane).  The decay is kept as a lazy
// scalar: the registers hold h / sigma with sigma the product of the decays
// since the last renormalisation, so a token costs one FMA per entry for the
// prediction, one for the write and (when outputs are wanted) one for the
// output, instead of an extra multiply per entry for the decay.
#include "internal.h"

namespace msa {
namespace {

constexpr int kTC = 32;                 // tokens per LDS stage
// h / sigma is renormalised once sigma drops below this, so a write (delta /
// sigma) stays far from float32 overflow; a decay that underflows sigma to 0
// zeroes the state, as the true decay would to float32 precision.
constexpr float kRenorm = 1.0e-18f;

__global__ __launch_bounds__(256) void gdn_state_sum_kernel(const float* __restrict__ states,
                                                            const int32_t* __restrict__ ids, int batch, int k,
                                                            int64_t n_docs, int64_t per_doc,
                                                            float* __restrict__ out) {
  const int64_t n4 = per_doc / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (i >= n4) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int32_t d = ids[(size_t)b * k + j];
    if (d < 0 || d >= n_docs) continue;          // out-of-range ids contribute nothing
    acc += *reinterpret_cast<const f32x4*>(states + (size_t)d * per_doc + 4 * i);
  }
  *reinterpret_cast<f32x4*>(out + (size_t)b * per_doc + 4 * i) = acc;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return Elem<T>::to_f32(*p); }

// One wave per (sequence, head, 64 value columns).  WITH_OUT: write o_t.
template <typename T, int DK, bool WITH_OUT>
__global__ __launch_bounds__(64) void gdn_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v, const float* __restrict__ g,
                                                 const float* __restrict__ beta, float scale,
                                                 const float* __restrict__ init, int seq_len, int heads, int dv,
                                                 T* __restrict__ out, float* __restrict__ final_state) {
  __shared__ __align__(16) float sq[kTC][DK];
  __shared__ __align__(16) float sk[kTC][DK];
  __shared__ float sa[kTC], sb[kTC];
  const int lane = threadIdx.x;
  const int c = blockIdx.x * 64 + lane;          // this lane's value column
  const bool c_ok = c < dv;
  const int hh = blockIdx.y;
  const int b = blockIdx.z;
  const size_t state_off = ((size_t)b * heads + hh) * DK * dv;

  float hs[DK];                                   // h / sigma, column c
#pragma unroll
  for (int r = 0; r < DK; ++r) hs[r] = (init != nullptr && c_ok) ? init[state_off + (size_t)r * dv + c] : 0.f;
  float sigma = 1.f;

  for (int t0 = 0; t0 < seq_len; t0 += kTC) {
    const int n = min(kTC, seq_len - t0);
    // stage q, k (float32) and the gates of tokens t0 .. t0+n-1
    for (int e = lane; e < n * DK; e += 64) {
      const int tt = e / DK, r = e - tt * DK;
      const size_t off = (((size_t)b * seq_len + t0 + tt) * heads + hh) * DK + r;
      sk[tt][r] = ld(k + off);
      if (WITH_OUT) sq[tt][r] = ld(q + off);
    }
    if (lane < n) {
      const size_t gi = ((size_t)b * seq_len + t0 + lane) * heads + hh;
      sa[lane] = __expf(g[gi]);
      sb[lane] = beta[gi];
    }
    __syncthreads();
    for (int tt = 0; tt < n; ++tt) {
      const size_t row = ((size_t)b * seq_len + t0 + tt) * heads + hh;
      const float vt = c_ok ? ld(v + row * dv + c) : 0.f;
      sigma *= sa[tt];
      if (sigma < kRenorm) {                      // uniform across the wave (same gates)
#pragma unroll
        for (int r = 0; r < DK; ++r) hs[r] *= sigma;
        sigma = 1.f;
      }
      float u = 0.f;
#pragma unroll
      for (int r = 0; r < DK; r += 4) {
        const f32x4 kk = *reinterpret_cast<const f32x4*>(&sk[tt][r]);
        u = fmaf(hs[r], kk[0], u);
        u = fmaf(hs[r + 1], kk[1], u);
        u = fmaf(hs[r + 2], kk[2], u);
        u = fmaf(hs[r + 3], kk[3], u);
        if (r % 32 == 28) __builtin_amdgcn_sched_barrier(0);   // bounds the operands kept in flight
      }
      const float delta = sb[tt] * (vt - sigma * u);
      const float w = delta / sigma;             // the write, in units of h / sigma
      float o = 0.f;
#pragma unroll
      for (int r = 0; r < DK; r += 4) {
        const f32x4 kk = *reinterpret_cast<const f32x4*>(&sk[tt][r]);
        hs[r] = fmaf(kk[0], w, hs[r]);
        hs[r + 1] = fmaf(kk[1], w, hs[r + 1]);
        hs[r + 2] = fmaf(kk[2], w, hs[r + 2]);
        hs[r + 3] = fmaf(kk[3], w, hs[r + 3]);
        if (WITH_OUT) {
          const f32x4 qq = *reinterpret_cast<const f32x4*>(&sq[tt][r]);
          o = fmaf(hs[r], qq[0], o);
          o = fmaf(hs[r + 1], qq[1], o);
          o = fmaf(hs[r + 2], qq[2], o);
          o = fmaf(hs[r + 3], qq[3], o);
        }
        if (r % 32 == 28) __builtin_amdgcn_sched_barrier(0);
      }
      if (WITH_OUT && c_ok) out[row * dv + c] = Elem<T>::from_f32(scale * sigma * o);
    }
    __syncthreads();
  }
  if (final_state != nullptr && c_ok) {
#pragma unroll
    for (int r = 0; r < DK; ++r) final_state[state_off + (size_t)r * dv + c] = sigma * hs[r];
  }
}

template <typename T, int DK>
hipError_t launch_gdn_t(const void* q, const void* k, const void* v, const float* g, const float* beta, float scale,
                        const float* init, int batch, int seq_len, int heads, int dv, void* out, float* final_state,
                        hipStream_t s) {
  const dim3 grid((unsigned)((dv + 63) / 64), (unsigned)heads, (unsigned)batch);
  if (out != nullptr)
    hipLaunchKernelGGL((gdn_kernel<T, DK, true>), grid, dim3(64), 0, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), g, beta, scale, init, seq_len, heads,
                       dv, static_cast<T*>(out), final_state);
  else
    hipLaunchKernelGGL((gdn_kernel<T, DK, false>), grid, dim3(64), 0, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), g, beta, scale, init, seq_len, heads,
                       dv, static_cast<T*>(nullptr), final_state);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_state_sum(const float* states, const int32_t* ids, int batch, int k, int64_t n_docs,
                                int64_t per_doc, float* out, hipStream_t s) {
  const int64_t n4 = per_doc / 4;
  hipLaunchKernelGGL(gdn_state_sum_kernel, dim3((unsigned)((n4 + 255) / 256), (unsigned)batch), dim3(256), 0, s,
                     states, ids, batch, k, n_docs, per_doc, out);
  return hipGetLastError();
}

hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* g, const float* beta, float scale,
                      const float* init, int batch, int seq_len, int heads, int dk, int dv, msa_dtype dt,
                      void* out, float* final_state, hipStream_t s) {
  if (dt == MSA_F32)
    return dk == 64 ? launch_gdn_t<float, 64>(q, k, v, g, beta, scale, init, batch, seq_len, heads, dv, out,
                                              final_state, s)
                    : launch_gdn_t<float, 128>(q, k, v, g, beta, scale, init, batch, seq_len, heads, dv, out,
                                               final_state, s);
  return dk == 64 ? launch_gdn_t<uint16_t, 64>(q, k, v, g, beta, scale, init, batch, seq_len, heads, dv, out,
                                               final_state, s)
                  : launch_gdn_t<uint16_t, 128>(q, k, v, g, beta, scale, init, batch, seq_len, heads, dv, out,
                                                final_state, s);
}

}  // namespace msa
