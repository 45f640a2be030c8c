// S6: sparse GQA attention for decode (few query tokens), split over keys.
//
// Method: MSA README (EverMind-AI/MSA), "Inference Pipeline" stage 3 --
// autoregressive generation over the sparse context [selected pooled memory ;
// local KV]; william-0g/MSA-Qwen3.5 model card, "Architecture summary".
//
// HBM-bound: every key and value row is read once.  The query columns are
// the (token, head) pairs of one KV group (T * group <= 32), so each K/V row
// is read once for all query heads that share it.  The keys of a sequence
// are cut into splits of 128; a workgroup (4 waves) owns one split and each
// wave 32 keys of it:
//   * K rows go straight from HBM into MFMA operands (16-byte loads, one
//     64-byte run per lane per half head),
//   * V rows are staged in the wave's own LDS region as interleaved key pairs
//     (see attn_prefill.hip) to form the V^T operand,
//   * S^T = K . Q^T and O^T = V^T . P^T run on bf16 MFMA in the same
//     lane-owns-a-query orientation as the prefill kernel.
// The four waves' (max, sum, O) partials merge through LDS, the workgroup
// writes one float32 partial per split, and attn_decode_combine merges the
// splits (the standard log-sum-exp merge) into bf16 output and the LSE.
#include "internal.h"

namespace msa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kSplitKeys = kWaves * 32;
constexpr int kVStride = 144;  // words per key-pair row (128 + pad)
constexpr int kVRegionWords = 16 * kVStride;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

struct Rows {
  const uint16_t* sel;
  const uint16_t* loc;
  int mem_len, loc_len, heads_kv, b, g;
  __device__ __forceinline__ const uint16_t* row(int kappa) const {
    if (kappa < mem_len) return sel + (((size_t)b * mem_len + kappa) * heads_kv + g) * kD;
    return loc + (((size_t)b * loc_len + (kappa - mem_len)) * heads_kv + g) * kD;
  }
};

__global__ __launch_bounds__(kWaves * 64) void attn_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_sel,
    const uint16_t* __restrict__ v_sel, int mem_len, const uint16_t* __restrict__ k_loc,
    const uint16_t* __restrict__ v_loc, int loc_len, int batch, int q_len, int heads_q, int heads_kv,
    float scale_log2, int n_split, float* __restrict__ part_o, float* __restrict__ part_ml) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  uint32_t* vsm = reinterpret_cast<uint32_t*>(smem_raw);     // [wave][16 pairs][kVStride]
  float* cb = reinterpret_cast<float*>(smem_raw);            // reused: [wave][nq][kD]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int group = heads_q / heads_kv;
  const int nq = q_len * group;

  int bid = blockIdx.x;
  const int split = bid % n_split;
  bid /= n_split;
  const int g = bid % heads_kv;
  const int b = bid / heads_kv;

  const int kend = mem_len + loc_len;
  const int causal0 = kend - q_len;  // token tt sees kappa < causal0 + tt + 1
  const int k0 = split * kSplitKeys + wave * 32;
  const Rows kr{k_sel, k_loc, mem_len, loc_len, heads_kv, b, g};
  const Rows vr{v_sel, v_loc, mem_len, loc_len, heads_kv, b, g};
  const u32x4 z = {0u, 0u, 0u, 0u};

  // issue all global loads first: V pairs (staging), K operand, Q^T operand
  u32x4 va[4], vb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int task = lane + 64 * i;
    const int p = task >> 4, seg = task & 15;
    const int ka = k0 + 2 * p;
    va[i] = ka < kend ? load16(vr.row(ka) + seg * 8) : z;
    vb[i] = ka + 1 < kend ? load16(vr.row(ka + 1) + seg * 8) : z;
  }
  bf16x8 kf[8];
  {
    const int key = k0 + cl;
    const bool ok = key < kend;
    const uint16_t* src = ok ? kr.row(key) : k_loc;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      kf[s] = as_bf16x8(ok ? load16(src + 64 * (s >> 2) + 32 * hf + 8 * (s & 3)) : z);
  }
  const bool col_ok = cl < nq;
  const int tt = col_ok ? cl / group : 0;
  const int h = g * group + (col_ok ? cl % group : 0);
  bf16x8 qf[8];
  {
    const uint16_t* src = q + (((size_t)b * q_len + tt) * heads_q + h) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = as_bf16x8(col_ok ? load16(src + 64 * (s >> 2) + 32 * hf + 8 * (s & 3)) : z);
  }

  // S^T = K . Q^T  (32 keys x 32 query columns)
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < 8; ++st) s = mfma32(kf[st], qf[st], s);

  // stage V as key pairs in this wave's LDS region
  uint32_t* vreg = vsm + wave * kVRegionWords;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int task = lane + 64 * i;
    const int p = task >> 4, seg = task & 15;
    u32x4 w0, w1;
    w0[0] = pair_lo(va[i][0], vb[i][0]);
    w0[1] = pair_hi(va[i][0], vb[i][0]);
    w0[2] = pair_lo(va[i][1], vb[i][1]);
    w0[3] = pair_hi(va[i][1], vb[i][1]);
    w1[0] = pair_lo(va[i][2], vb[i][2]);
    w1[1] = pair_hi(va[i][2], vb[i][2]);
    w1[2] = pair_lo(va[i][3], vb[i][3]);
    w1[3] = pair_hi(va[i][3], vb[i][3]);
    *reinterpret_cast<u32x4*>(&vreg[p * kVStride + seg * 8]) = w0;
    *reinterpret_cast<u32x4*>(&vreg[p * kVStride + seg * 8 + 4]) = w1;
  }

  // mask, max, probabilities
  const int lim = min(kend, causal0 + tt + 1);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = s[i] * scale_log2;
    if (k0 + acc_row(i, hf) >= lim) v = -INFINITY;
    s[i] = v;
    m = fmaxf(m, v);
  }
  m = fmaxf(m, __shfl_xor(m, 32));
  const float mref = m == -INFINITY ? 0.f : m;
  float lsum = 0.f;
  bf16x8 pf[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(s[8 * s2 + 2 * e] - mref);
      const float p1 = fast_exp2(s[8 * s2 + 2 * e + 1] - mref);
      lsum += p0 + p1;
      w[e] = pack_bf16x2(p0, p1);
    }
    pf[s2] = as_bf16x8(w);
  }
  const float l = lsum + __shfl_xor(lsum, 32);
  __syncthreads();

  // O^T = V^T . P^T  (128 d x 32 query columns)
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const uint32_t* vrow = &vreg[(8 * s2 + 2 * hf) * kVStride];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + cl;
      u32x4 w;
      w[0] = vrow[d];
      w[1] = vrow[kVStride + d];
      w[2] = vrow[4 * kVStride + d];
      w[3] = vrow[5 * kVStride + d];
      o[db] = mfma32(as_bf16x8(w), pf[s2], o[db]);
    }
  }
  __syncthreads();  // every wave is done with its V region before it is reused

  // merge the four waves: cb[wave][n][d], then (m, l) after it
  float* cbw = cb + (size_t)wave * nq * kD;
  float* mls = cb + (size_t)kWaves * nq * kD;  // [wave][n][2]
  if (col_ok) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) cbw[cl * kD + db * 32 + acc_row(i, hf)] = o[db][i];
    if (hf == 0) {
      mls[(wave * nq + cl) * 2] = m;
      mls[(wave * nq + cl) * 2 + 1] = l;
    }
  }
  __syncthreads();
  const size_t pbase = (((size_t)b * heads_kv + g) * n_split + split) * nq;
  for (int idx = tid; idx < nq * kD; idx += kWaves * 64) {
    const int n = idx / kD, d = idx - n * kD;
    float mw[kWaves];
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = mls[(w * nq + n) * 2];
      mx = fmaxf(mx, mw[w]);
    }
    float acc = 0.f, lt = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - mx);
        acc += cb[((size_t)w * nq + n) * kD + d] * f;
        lt += mls[(w * nq + n) * 2 + 1] * f;
      }
    }
    part_o[(pbase + n) * kD + d] = acc;
    if (d == 0) {
      part_ml[(pbase + n) * 2] = mx;
      part_ml[(pbase + n) * 2 + 1] = lt;
    }
  }
}

// Merge the splits of one (sequence, token, query head): one wave, 2 d per lane.
__global__ __launch_bounds__(256) void attn_decode_combine(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int batch, int q_len,
    int heads_q, int heads_kv, int n_split, uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n_rows = (int64_t)batch * q_len * heads_q;
  if (row >= n_rows) return;
  const int h = (int)(row % heads_q);
  const int t = (int)((row / heads_q) % q_len);
  const int b = (int)(row / ((int64_t)heads_q * q_len));
  const int group = heads_q / heads_kv;
  const int g = h / group;
  const int nq = q_len * group;
  const int n = t * group + (h - g * group);
  const size_t base = ((size_t)b * heads_kv + g) * n_split;
  float mx = -INFINITY;
  for (int sp = 0; sp < n_split; ++sp) mx = fmaxf(mx, part_ml[((base + sp) * nq + n) * 2]);
  float o0 = 0.f, o1 = 0.f, lt = 0.f;
  for (int sp = 0; sp < n_split; ++sp) {
    const size_t pi = (base + sp) * nq + n;
    const float ms = part_ml[pi * 2];
    if (ms == -INFINITY) continue;
    const float f = fast_exp2(ms - mx);
    lt += part_ml[pi * 2 + 1] * f;
    const float2 v = *reinterpret_cast<const float2*>(&part_o[pi * kD + 2 * lane]);
    o0 += v.x * f;
    o1 += v.y * f;
  }
  const float inv = 1.f / lt;
  uint16_t* orow = out + (((size_t)b * q_len + t) * heads_q + h) * kD;
  *reinterpret_cast<uint32_t*>(orow + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
  if (lse != nullptr && lane == 0) lse[((size_t)b * heads_q + h) * q_len + t] = (mx + __log2f(lt)) * kLn2;
}

}  // namespace

bool attn_decode_supported(int q_len, int heads_q, int heads_kv, int dim, msa_dtype dt) {
  return dt == MSA_BF16 && dim == kD && q_len * (heads_q / heads_kv) <= 32;
}

static int decode_splits(int mem_len, int loc_len) {
  return (mem_len + loc_len + kSplitKeys - 1) / kSplitKeys;
}

size_t attn_decode_workspace(int batch, int q_len, int heads_q, int heads_kv, int mem_len,
                             int loc_len) {
  const size_t nq = (size_t)q_len * (heads_q / heads_kv);
  const size_t parts = (size_t)batch * heads_kv * decode_splits(mem_len, loc_len) * nq;
  return parts * (kD + 2) * sizeof(float) + 256;
}

hipError_t launch_attn_decode(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                              const void* k_loc, const void* v_loc, int loc_len, int batch,
                              int q_len, int heads_q, int heads_kv, float scale, void* out,
                              float* lse, void* ws, hipStream_t s) {
  const int n_split = decode_splits(mem_len, loc_len);
  const int nq = q_len * (heads_q / heads_kv);
  const size_t parts = (size_t)batch * heads_kv * n_split * nq;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + parts * kD;
  const size_t smem_v = (size_t)kWaves * kVRegionWords * 4;
  const size_t smem_c = ((size_t)kWaves * nq * kD + (size_t)kWaves * nq * 2) * 4;
  const size_t smem = smem_v > smem_c ? smem_v : smem_c;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(attn_decode_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(kWaves * (32 * kD + 64) * 4 > (int)smem_v ? kWaves * (32 * kD + 64) * 4 : (int)smem_v));
  if (attr != hipSuccess) return attr;
  const unsigned grid = (unsigned)((size_t)batch * heads_kv * n_split);
  hipLaunchKernelGGL(attn_decode_kernel, dim3(grid), dim3(kWaves * 64), smem, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_sel),
                     static_cast<const uint16_t*>(v_sel), mem_len, static_cast<const uint16_t*>(k_loc),
                     static_cast<const uint16_t*>(v_loc), loc_len, batch, q_len, heads_q, heads_kv,
                     scale * kLog2e, n_split, part_o, part_ml);
  const int64_t rows = (int64_t)batch * q_len * heads_q;
  hipLaunchKernelGGL(attn_decode_combine, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, part_o,
                     part_ml, batch, q_len, heads_q, heads_kv, n_split, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace msa
