// Kernel selection for attention: the bf16 MFMA kernels serve
// the shapes they are built for, the vector-ALU kernels serve every other
// shape (float32, odd head dims).  Both are HIP; there is no CPU path.
#include "internal.h"

namespace msa {

hipError_t launch_attn_generic(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                               const void* k_loc, const void* v_loc, int loc_len, int batch,
                               int q_len, int heads_q, int heads_kv, int dim, float scale,
                               msa_dtype dt, void* out, float* lse, hipStream_t s);

size_t attn_workspace_bytes(int batch, int q_len, int heads_q, int heads_kv, int dim, int mem_len,
                            int loc_len, msa_dtype dt) {
  (void)batch; (void)q_len; (void)heads_q; (void)heads_kv; (void)dim; (void)mem_len;
  (void)loc_len; (void)dt;
  return 0;
}

hipError_t launch_attn(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                       const void* k_loc, const void* v_loc, int loc_len, int batch, int q_len,
                       int heads_q, int heads_kv, int dim, float scale, msa_dtype dt, void* out,
                       float* lse, void* ws, hipStream_t s) {
  (void)ws;
  return launch_attn_generic(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, batch, q_len, heads_q,
                             heads_kv, dim, scale, dt, out, lse, s);
}

}  // namespace msa
