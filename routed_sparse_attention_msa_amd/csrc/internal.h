// Internal declarations shared by the libmsa sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/msa.h"

namespace msa {

// ---------------------------------------------------------------------------
// vector types for gfx950 MFMA operands and 16-byte memory traffic
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 <-> f32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float32 -> bf16 bits: add 0x7FFF plus the lowest kept
// bit, then truncate.  Exact RNE for every finite input (overflow goes to inf).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element traits for the two storage dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
};

// 16 bytes of elements, widened to float32.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void widen(const u32x4& raw, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(raw[i]);
  }
  static __device__ __forceinline__ u32x4 narrow(const float* in) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(in[i]);
    return r;
  }
};
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void widen(const u32x4& raw, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(raw[i] << 16);
      out[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ u32x4 narrow(const float* in) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = (uint32_t)f32_to_bf16(in[2 * i]) | ((uint32_t)f32_to_bf16(in[2 * i + 1]) << 16);
    return r;
  }
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming variants for data touched once (no reuse through L2 / MALL).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16_stream(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Compute units of the current device (256 on MI355X).
inline int device_cu_count() {
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  return n_cu;
}

// ---------------------------------------------------------------------------
// launchers (each returns hipGetLastError() of its launches)
// ---------------------------------------------------------------------------
hipError_t launch_pool(const void* x, void* xbar, float* norm, int64_t n_chunks, int chunk,
                       int heads, int dim, msa_dtype dt, hipStream_t s);

hipError_t launch_chunk_offsets(const int64_t* doc_off, int64_t n_docs, int chunk, int64_t* chunk_off,
                                hipStream_t s);
hipError_t launch_encode(const void* x, void* xbar, float* norm, const int64_t* doc_off,
                         const int64_t* chunk_off, int64_t n_docs, int64_t total_rows,
                         int64_t total_chunks, int chunk, int heads, int dim, float rope_base,
                         msa_dtype dt, hipStream_t s);

// Whether routing this shape takes the tiled MFMA kernel (whose scores for a
// sequence do not depend on the other sequences of the launch).
bool route_is_tiled(int batch, int q_len, int heads, int dim, int cpd, msa_dtype dt);
size_t route_workspace_bytes(int batch, int q_len, int heads, int dim, int64_t n_docs, int cpd,
                             msa_dtype dt);
hipError_t launch_route(const void* q_r, const void* kbar_r, const float* knorm, int batch,
                        int q_len, int heads, int dim, int64_t n_docs, int cpd, msa_dtype dt,
                        float* doc_scores, void* ws, hipStream_t s);
// Device address of the library-resident routing scratch of the current
// device (kRouteStaticScratchBytes, looked up once per device).
constexpr size_t kRouteStaticScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
hipError_t route_static_scratch(void** ptr);

size_t topk_workspace_bytes(int batch, int64_t n_docs, int k);
hipError_t launch_topk(const float* scores, int batch, int64_t n_docs, int k, int32_t* ids,
                       float* vals, void* ws, hipStream_t s);
// As launch_topk over the documents not in excl[b*excl_stride + 0..n_excl-1]
// (ids outside [0, n_docs) ignored); outputs at row b*out_stride.
hipError_t launch_topk_excl(const float* scores, int batch, int64_t n_docs, int k, const int32_t* excl,
                            int n_excl, int64_t excl_stride, int32_t* ids, float* vals,
                            int64_t out_stride, void* ws, hipStream_t s);

hipError_t launch_gather(const void* kbar, const void* vbar, const int32_t* ids, int batch, int k,
                         int64_t n_docs, int cpd, size_t row_bytes, bool host_src, void* k_sel, void* v_sel,
                         int* err_flag, hipStream_t s);

size_t attn_workspace_bytes(int batch, int q_len, int heads_q, int heads_kv, int dim, int mem_len,
                            int loc_len, msa_dtype dt);
hipError_t launch_attn(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                       const void* k_loc, const void* v_loc, int loc_len, int batch, int q_len,
                       int heads_q, int heads_kv, int dim, float scale, msa_dtype dt, void* out,
                       float* lse, void* ws, hipStream_t s);

// Log-sum-exp merge of two partial attentions over disjoint key sets.
hipError_t launch_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                             int batch, int q_len, int heads_q, int dim, msa_dtype dt, void* o, float* lse,
                             hipStream_t s);

size_t attn_backward_workspace_bytes(int batch, int q_len, int heads_q, int heads_kv, int dim, int mem_len,
                                     int loc_len, msa_dtype dt);
hipError_t launch_attn_backward(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                                const void* k_loc, const void* v_loc, int loc_len, const void* out,
                                const void* d_out, const float* lse, int batch, int q_len, int heads_q,
                                int heads_kv, int dim, float scale, msa_dtype dt, void* dq, void* dk_sel,
                                void* dv_sel, void* dk_loc, void* dv_loc, void* ws, hipStream_t s);

hipError_t launch_gdn_state_sum(const float* states, const int32_t* ids, int batch, int k, int64_t n_docs,
                                int64_t per_doc, float* out, hipStream_t s);
hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* g, const float* beta, float scale,
                      const float* init, int batch, int seq_len, int heads, int dk, int dv, msa_dtype dt,
                      void* out, float* final_state, hipStream_t s);
hipError_t launch_gdn_chunked(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              float scale, const float* init, int batch, int seq_len, int heads, void* out,
                              float* final_state, hipStream_t s);

}  // namespace msa
