// S5: sparse GQA attention for prefill on bf16 MFMA (gfx950, head dim 128).
//
// Method: william-0g/MSA-Qwen3.5 model card, "Architecture summary" -- in the
// softmax layers the selected chunks' K/V are concatenated with the local KV
// inside attention; MSA README, "Overall Design" and "Inference Pipeline"
// stage 3.  Query token t of a sequence sees the M gathered memory rows and
// the local rows 0 .. L_loc - T + t (bottom-right causal alignment).
//
// Flash-style online softmax, written in the "transposed" orientation so a
// lane owns one query:
//     S^T[key, query] = K . Q^T      (A = K tile from LDS, B = Q^T in registers)
//     O^T[d,   query] += V^T . P^T   (A = V^T from LDS,    B = P^T in registers)
// On a 32x32 MFMA accumulator lane (n, hf) holds column n (one query) and 16
// rows, so the running max / sum of a query are lane scalars (the other lane
// half adds one xor-32 shuffle), the O^T rescale is a scalar multiply, and the
// P^T operand of the second product is the lane's own S^T values converted to
// bf16 -- no cross-lane traffic.  The key order inside each 32-key block is
// chosen so that holds; V is staged in LDS as interleaved key pairs (one
// 32-bit word = the same d of two consecutive keys), so each V^T operand is
// four 32-bit LDS reads.
//
// Work split: one workgroup = (sequence, KV head, 32-token block); its waves
// are the query heads of that KV group (GQA packing: each K/V tile is staged
// once for all of them).  K/V tiles of 64 keys are double-buffered in LDS,
// the next tile's global loads in flight during the current tile's math.
// Keys are a virtual sequence [memory rows ; local rows]; blocks fully below
// every query's causal limit skip the mask, blocks beyond the last query's
// limit are never loaded.  Workgroups are issued longest-first.
#include "internal.h"

namespace msa {
namespace {

constexpr int kD = 128;
constexpr int kKT = 64;          // keys per LDS tile
constexpr int kVStride = 144;    // 32-bit words per key-pair row of the V tile (128 + pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct PrefillSmem {
  uint8_t k[2][kKT * kD * 2];             // [key][256 B], XOR-swizzled 16 B segments
  uint32_t v[2][(kKT / 2) * kVStride];    // [key pair][d]: V[2p][d] | V[2p+1][d] << 16
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }
__device__ __forceinline__ int kswz(int key, int seg) { return key * 256 + ((seg ^ (key & 7)) << 4); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two bf16 of one key and two of the next key -> the (key pair) words for two d's.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

struct KeySrc {
  const uint16_t* sel;
  const uint16_t* loc;
  int mem_len, loc_len, heads_kv, b, g;
  __device__ __forceinline__ const uint16_t* row(int kappa) const {
    if (kappa < mem_len) return sel + (((size_t)b * mem_len + kappa) * heads_kv + g) * kD;
    return loc + (((size_t)b * loc_len + (kappa - mem_len)) * heads_kv + g) * kD;
  }
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_sel,
    const uint16_t* __restrict__ v_sel, int mem_len, const uint16_t* __restrict__ k_loc,
    const uint16_t* __restrict__ v_loc, int loc_len, int batch, int q_len, int heads_q, int heads_kv,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int kThreads = NW * 64;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  PrefillSmem& sm = *reinterpret_cast<PrefillSmem*>(smem_raw);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int group = heads_q / heads_kv;
  const int hsub = group / NW;                  // head sub-groups per KV head
  const int n_tblk = (q_len + 31) / 32;

  // blockIdx -> (token block, sequence, kv head, head sub-group); longest first
  int bid = blockIdx.x;
  const int hs = bid % hsub;
  bid /= hsub;
  const int g = bid % heads_kv;
  bid /= heads_kv;
  const int b = bid % batch;
  const int tb = n_tblk - 1 - bid / batch;
  const int h = g * group + hs * NW + wave;
  const int t0 = tb * 32;
  const int t = t0 + cl;                        // this lane's query token
  const bool t_ok = t < q_len;

  const KeySrc ks{k_sel, k_loc, mem_len, loc_len, heads_kv, b, g};
  const int causal0 = mem_len + loc_len - q_len;          // token t sees kappa < causal0 + t + 1
  const int kend = causal0 + min(t0 + 32, q_len);          // keys needed by the block
  const int n_tiles = (kend + kKT - 1) / kKT;
  const int full_below = causal0 + t0 + 1;                 // keys < this are visible to all

  // Q^T operand: lane (query cl, half hf), d-slots 64*(s/4) + 32*hf + 8*(s%4) .. +8
  bf16x8 qf[8];
  {
    const uint16_t* qrow = q + (((size_t)b * q_len + (t_ok ? t : 0)) * heads_q + h) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[s] = as_bf16x8(t_ok ? load16(qrow + 64 * (s >> 2) + 32 * hf + 8 * (s & 3)) : z);
    }
  }

  // staging: K 64 rows x 16 segments; V 32 key pairs x 16 segments (two rows each)
  constexpr int kKChunks = kKT * 16 / kThreads;
  constexpr int kVChunks = (kKT / 2) * 16 / kThreads;
  u32x4 pk[kKChunks], pv0[kVChunks], pv1[kVChunks];
  auto gload = [&](int tile) {
    const int kappa0 = tile * kKT;
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) {
      const int c = tid + kThreads * i;
      const int r = c >> 4, seg = c & 15;
      const int kappa = kappa0 + r;
      const u32x4 z = {0u, 0u, 0u, 0u};
      pk[i] = kappa < kend ? load16(ks.row(kappa) + seg * 8) : z;
    }
#pragma unroll
    for (int i = 0; i < kVChunks; ++i) {
      const int c = tid + kThreads * i;
      const int p = c >> 4, seg = c & 15;
      const int k0 = kappa0 + 2 * p;
      const u32x4 z = {0u, 0u, 0u, 0u};
      const KeySrc vs{v_sel, v_loc, mem_len, loc_len, heads_kv, b, g};
      pv0[i] = k0 < kend ? load16(vs.row(k0) + seg * 8) : z;
      pv1[i] = k0 + 1 < kend ? load16(vs.row(k0 + 1) + seg * 8) : z;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) {
      const int c = tid + kThreads * i;
      const int r = c >> 4, seg = c & 15;
      *reinterpret_cast<u32x4*>(&sm.k[buf][kswz(r, seg)]) = pk[i];
    }
#pragma unroll
    for (int i = 0; i < kVChunks; ++i) {
      const int c = tid + kThreads * i;
      const int p = c >> 4, seg = c & 15;
      const u32x4 a = pv0[i], bb = pv1[i];
      u32x4 w0, w1;  // d = seg*8 + 0..3 and + 4..7
      w0[0] = pair_lo(a[0], bb[0]);
      w0[1] = pair_hi(a[0], bb[0]);
      w0[2] = pair_lo(a[1], bb[1]);
      w0[3] = pair_hi(a[1], bb[1]);
      w1[0] = pair_lo(a[2], bb[2]);
      w1[1] = pair_hi(a[2], bb[2]);
      w1[2] = pair_lo(a[3], bb[3]);
      w1[3] = pair_hi(a[3], bb[3]);
      uint32_t* dst = &sm.v[buf][p * kVStride + seg * 8];
      *reinterpret_cast<u32x4*>(dst) = w0;
      *reinterpret_cast<u32x4*>(dst + 4) = w1;
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;  // running max (log2 domain) and this half's running sum

  gload(0);
  lstore(0);
  if (n_tiles > 1) gload(1);
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    const int kappa0 = tile * kKT;
    // S^T for the tile's two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int seg = 8 * (st >> 2) + 4 * hf + (st & 3);
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sm.k[buf][kswz(kb * 32 + cl, seg)]);
        s[kb] = mfma32(kf, qf[st], s[kb]);
      }
    }
    // scale, mask, tile max
    const bool full = kappa0 + kKT <= full_below;
    const int lim = causal0 + t + 1;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[kb][i] * scale_log2;
        if (!full && kappa0 + kb * 32 + acc_row(i, hf) >= lim) v = -INFINITY;
        s[kb][i] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float lsum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(s[kb][8 * s2 + 2 * e] - m_new);
          const float p1 = fast_exp2(s[kb][8 * s2 + 2 * e + 1] - m_new);
          lsum += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[kb][s2] = as_bf16x8(w);
      }
    l = l * alpha + lsum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int p = kb * 16 + 8 * s2 + 2 * hf;
        const uint32_t* vrow = &sm.v[buf][p * kVStride];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = db * 32 + cl;
          u32x4 w;
          w[0] = vrow[d];
          w[1] = vrow[kVStride + d];
          w[2] = vrow[4 * kVStride + d];
          w[3] = vrow[5 * kVStride + d];
          o[db] = mfma32(as_bf16x8(w), pf[kb][s2], o[db]);
        }
      }
    if (tile + 1 < n_tiles) lstore(buf ^ 1);
    if (tile + 2 < n_tiles) gload(tile + 2);
    __syncthreads();
  }

  const float l_tot = l + __shfl_xor(l, 32);
  if (!t_ok) return;
  const float inv_l = 1.f / l_tot;
  uint16_t* orow = out + (((size_t)b * q_len + t) * heads_q + h) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = db * 32 + 8 * qd + 4 * hf;
      uint2 w;
      w.x = pack_bf16x2(o[db][4 * qd] * inv_l, o[db][4 * qd + 1] * inv_l);
      w.y = pack_bf16x2(o[db][4 * qd + 2] * inv_l, o[db][4 * qd + 3] * inv_l);
      *reinterpret_cast<uint2*>(orow + d0) = w;
    }
  if (lse != nullptr && hf == 0) lse[((size_t)b * heads_q + h) * q_len + t] = (m + __log2f(l_tot)) * kLn2;
}

}  // namespace

bool attn_prefill_supported(int q_len, int heads_q, int heads_kv, int dim, msa_dtype dt) {
  (void)q_len;
  if (dt != MSA_BF16 || dim != kD) return false;
  const int group = heads_q / heads_kv;
  return group % 4 == 0 || group == 2 || group == 1;
}

hipError_t launch_attn_prefill(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                               const void* k_loc, const void* v_loc, int loc_len, int batch,
                               int q_len, int heads_q, int heads_kv, float scale, void* out,
                               float* lse, hipStream_t s) {
  const int group = heads_q / heads_kv;
  const int nw = group % 4 == 0 ? 4 : group;
  const int n_tblk = (q_len + 31) / 32;
  const unsigned grid = (unsigned)(n_tblk * batch * heads_kv * (group / nw));
  const size_t smem = sizeof(PrefillSmem);
  const float sl2 = scale * kLog2e;
  auto args = [&](auto kern) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * nw), smem, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k_sel), static_cast<const uint16_t*>(v_sel),
                       mem_len, static_cast<const uint16_t*>(k_loc),
                       static_cast<const uint16_t*>(v_loc), loc_len, batch, q_len, heads_q, heads_kv,
                       sl2, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
  };
  if (nw == 4) return args(attn_prefill_kernel<4>);
  if (nw == 2) return args(attn_prefill_kernel<2>);
  return args(attn_prefill_kernel<1>);
}

}  // namespace msa
