// Kernel selection for attention.  bf16 with head dim 128 runs on MFMA:
// the split-KV decode kernel when one KV group has at most 32 query columns
// (tokens x query heads), the flash prefill kernel otherwise.  Every other
// shape (float32, other head dims, odd group sizes) runs on the vector-ALU
// kernel.  All are HIP; there is no CPU path.
#include "internal.h"

namespace msa {

hipError_t launch_attn_generic(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                               const void* k_loc, const void* v_loc, int loc_len, int batch,
                               int q_len, int heads_q, int heads_kv, int dim, float scale,
                               msa_dtype dt, void* out, float* lse, hipStream_t s);
bool attn_prefill_supported(int q_len, int heads_q, int heads_kv, int dim, msa_dtype dt);
hipError_t launch_attn_prefill(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                               const void* k_loc, const void* v_loc, int loc_len, int batch,
                               int q_len, int heads_q, int heads_kv, float scale, void* out,
                               float* lse, hipStream_t s);
bool attn_decode_supported(int q_len, int heads_q, int heads_kv, int dim, msa_dtype dt);
size_t attn_decode_workspace(int batch, int q_len, int heads_q, int heads_kv, int mem_len,
                             int loc_len);
hipError_t launch_attn_decode(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                              const void* k_loc, const void* v_loc, int loc_len, int batch,
                              int q_len, int heads_q, int heads_kv, float scale, void* out,
                              float* lse, void* ws, hipStream_t s);

size_t attn_workspace_bytes(int batch, int q_len, int heads_q, int heads_kv, int dim, int mem_len,
                            int loc_len, msa_dtype dt) {
  if (attn_decode_supported(q_len, heads_q, heads_kv, dim, dt))
    return attn_decode_workspace(batch, q_len, heads_q, heads_kv, mem_len, loc_len);
  return 0;
}

hipError_t launch_attn(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                       const void* k_loc, const void* v_loc, int loc_len, int batch, int q_len,
                       int heads_q, int heads_kv, int dim, float scale, msa_dtype dt, void* out,
                       float* lse, void* ws, hipStream_t s) {
  if (attn_decode_supported(q_len, heads_q, heads_kv, dim, dt))
    return launch_attn_decode(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, batch, q_len,
                              heads_q, heads_kv, scale, out, lse, ws, s);
  if (attn_prefill_supported(q_len, heads_q, heads_kv, dim, dt))
    return launch_attn_prefill(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, batch, q_len,
                               heads_q, heads_kv, scale, out, lse, s);
  return launch_attn_generic(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, batch, q_len, heads_q,
                             heads_kv, dim, scale, dt, out, lse, s);
}

}  // namespace msa
