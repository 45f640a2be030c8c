// S6: sparse GQA attention for decode (few query tokens), split over keys.
//
// Method: MSA README (EverMind-AI/MSA), "Inference Pipeline" stage 3 --
// autoregressive generation over the sparse context [selected pooled memory ;
// local KV]; william-0g/MSA-Qwen3.5 model card, "Architecture summary".
//
// HBM-bound: every key and value row is read once.  The query columns are
// the (token, head) pairs of one KV group (T * group <= 32), so each K/V row
// is read once for all query heads that share it.  Keys are cut into splits
// of 128, and wave w of a workgroup takes keys 32w .. 32w+31 of each split:
//   * K and V rows are read whole (16 lanes x 16 bytes per 256-byte row, so a
//     wave instruction covers 4 rows): reading a K row as MFMA operand pieces
//     straight from HBM (32 rows x 32 bytes per instruction) costs ~30% of
//     the bandwidth,
//   * K rows go through the wave's own LDS region (row pitch padded to 272
//     bytes for conflict-free operand reads) into the K operand; V rows are
//     staged there as interleaved key pairs to form the V^T operand,
//   * S^T = K . Q^T and O^T = V^T . P^T run on bf16 MFMA in the same
//     lane-owns-a-query orientation as the prefill kernel.
// A workgroup owns one (sequence, KV head) and a contiguous run of splits.
// Each wave keeps an online softmax over its slices of those splits and has
// two register sets of K/V rows: the loads of the next split are in flight
// while the current one is computed, so HBM sees a steady stream instead of
// a burst per short workgroup.  The four waves merge through LDS at the end.
// With at least one (sequence, KV head) per CU a workgroup takes all splits
// and writes the bf16 output directly; with fewer, each pair is cut into P
// runs that write float32 partials and attn_decode_combine merges them (the
// log-sum-exp merge).
#include <algorithm>

#include "internal.h"

namespace msa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kSplitKeys = kWaves * 32;
constexpr int kVStride = 144;  // words per key-pair row (128 + pad)
constexpr int kVRegionWords = 16 * kVStride;
constexpr int kKPitch = 272;   // bytes per K row in LDS (256 + pad)
constexpr int kKRegionBytes = 32 * kKPitch;
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
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v v = {(__bf16)lo, (__bf16)hi};   // one v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// (aux 2: the non-temporal policy, as for the streamed rows of the other path)
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2));
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

struct KVRegs {
  u32x4 kw[8];         // K rows of the wave's 32 keys, 16 bytes at a time
  u32x4 va[4], vb[4];  // V rows of its 16 key pairs, 16 bytes at a time
};
// K piece st of a lane: row 8*(st & 3) + 2*(lane >> 4) + (st >> 2) of the wave's
// 32 keys, 16-byte segment lane & 15.
__device__ __forceinline__ int krow_of(int st, int lane) { return 8 * (st & 3) + 2 * (lane >> 4) + (st >> 2); }

// BLOCKS: the memory length is a multiple of 32, so each wave's 32 keys of a
// split are all memory rows or all local rows: the loads go through one
// buffer resource (chosen per wave and split) with 32-bit offsets, the row
// part of every offset a scalar.  Otherwise each row's address is formed on
// its own (64-bit, per lane).
template <bool BLOCKS>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_sel,
    const uint16_t* __restrict__ v_sel, int mem_len, const uint16_t* __restrict__ k_loc,
    const uint16_t* __restrict__ v_loc, int loc_len, int batch, int q_len, int heads_q, int heads_kv,
    float scale_log2, int n_split, int n_part, int per_part, float* __restrict__ part_o,
    float* __restrict__ part_ml, uint16_t* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  uint32_t* vsm = reinterpret_cast<uint32_t*>(smem_raw);     // [wave][16 pairs][kVStride]
  float* cb = reinterpret_cast<float*>(smem_raw);            // reused: [wave][nq][kD]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int group = heads_q / heads_kv;
  const int nq = q_len * group;

  int bid = blockIdx.x;
  const int part = bid % n_part;
  bid /= n_part;
  const int g = bid % heads_kv;
  const int b = bid / heads_kv;
  const int s_lo = part * per_part;
  const int s_hi = min(n_split, s_lo + per_part);

  const int kend = mem_len + loc_len;
  const int causal0 = kend - q_len;  // token tt sees kappa < causal0 + tt + 1
  const Rows kr{k_sel, k_loc, mem_len, loc_len, heads_kv, b, g};
  const Rows vr{v_sel, v_loc, mem_len, loc_len, heads_kv, b, g};
  const u32x4 z = {0u, 0u, 0u, 0u};

  // Loads are unconditional (a branch per load would leave the compiler unable
  // to count them and make it wait for all of them): keys past the end read
  // the last key's row, whose scores are masked to -inf, so its V rows get
  // weight 0.
  // per (sequence, KV head): memory and local rows behind buffer resources
  // sized to them (rows past the end read as zeros; such keys are masked)
  const uint32_t rs = (uint32_t)heads_kv * kD * 2;
  const size_t sel0 = ((size_t)b * mem_len * heads_kv + g) * kD, loc0 = ((size_t)b * loc_len * heads_kv + g) * kD;
  const uint32_t sel_bytes = (uint32_t)mem_len * rs - (uint32_t)g * kD * 2;
  const uint32_t loc_bytes = (uint32_t)loc_len * rs - (uint32_t)g * kD * 2;
  const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc((void*)(k_sel + (mem_len ? sel0 : 0)), (short)0, (int)(mem_len ? sel_bytes : 0u), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc((void*)(v_sel + (mem_len ? sel0 : 0)), (short)0, (int)(mem_len ? sel_bytes : 0u), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rkl = __builtin_amdgcn_make_buffer_rsrc((void*)(k_loc + loc0), (short)0, (int)loc_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rvl = __builtin_amdgcn_make_buffer_rsrc((void*)(v_loc + loc0), (short)0, (int)loc_bytes, kRsrcWord3);
  // the lane's part of every offset: rows 2 (lane / 16) + ..., 16-byte segment lane % 16
  const uint32_t lane_off = (uint32_t)(2 * (lane >> 4)) * rs + (lane & 15) * 16;

  auto load = [&](KVRegs& r, int sp) {
    const int k0 = sp * kSplitKeys + wave * 32;
    if (BLOCKS) {
      const bool in_mem = k0 < mem_len;           // uniform: the wave's 32 keys lie on one side
      const __amdgpu_buffer_rsrc_t rk = in_mem ? rks : rkl, rv = in_mem ? rvs : rvl;
      const int r0 = in_mem ? k0 : k0 - mem_len;
#pragma unroll
      for (int i = 0; i < 4; ++i) {               // V rows 2 (lane / 16) + 8 i and the next one
        r.va[i] = bload(rv, lane_off + (uint32_t)(r0 + 8 * i) * rs);
        r.vb[i] = bload(rv, lane_off + (uint32_t)(r0 + 8 * i + 1) * rs);
      }
#pragma unroll
      for (int st = 0; st < 8; ++st)              // K row krow_of(st, lane)
        r.kw[st] = bload(rk, lane_off + (uint32_t)(r0 + 8 * (st & 3) + (st >> 2)) * rs);
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int task = lane + 64 * i;
      const int pr = task >> 4, seg = task & 15;
      const int ka = min(k0 + 2 * pr, kend - 1), kb = min(k0 + 2 * pr + 1, kend - 1);
      r.va[i] = load16_stream(vr.row(ka) + seg * 8);
      r.vb[i] = load16_stream(vr.row(kb) + seg * 8);
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
      r.kw[st] = load16_stream(kr.row(min(k0 + krow_of(st, lane), kend - 1)) + (lane & 15) * 8);
  };

  const bool col_ok = cl < nq;
  const int tt = col_ok ? cl / group : 0;
  const int h = g * group + (col_ok ? cl % group : 0);
  bf16x8 qf[8];
  {
    const uint16_t* src = q + (((size_t)b * q_len + tt) * heads_q + h) * kD;
#pragma unroll
    for (int st = 0; st < 8; ++st)
      qf[st] = as_bf16x8(col_ok ? load16(src + 64 * (st >> 2) + 32 * hf + 8 * (st & 3)) : z);
  }
  const int lim = min(kend, causal0 + tt + 1);

  uint32_t* vreg = vsm + wave * kVRegionWords;
  uint8_t* kreg = smem_raw + (size_t)kWaves * kVRegionWords * 4 + (size_t)wave * kKRegionBytes;
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m = -INFINITY;   // running max of the scaled scores (log2 units)
  float lh = 0.f;        // this lane half's running sum

  auto process = [&](const KVRegs& r, int sp) {
    const int k0 = sp * kSplitKeys + wave * 32;
    // K rows into this wave's LDS region, then the K operand: lane (key cl,
    // half hf) takes d-slots 64*(st/4) + 32*hf + 8*(st%4) .. +8 (the order of Q^T)
#pragma unroll
    for (int st = 0; st < 8; ++st)
      *reinterpret_cast<u32x4*>(kreg + krow_of(st, lane) * kKPitch + (lane & 15) * 16) = r.kw[st];
    bf16x8 kf[8];
#pragma unroll
    for (int st = 0; st < 8; ++st)
      kf[st] = *reinterpret_cast<const bf16x8*>(kreg + cl * kKPitch + (8 * (st >> 2) + 4 * hf + (st & 3)) * 16);
    // S^T = K . Q^T  (32 keys x 32 query columns)
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) s = mfma32(kf[st], qf[st], s);
    // V key pairs into this wave's LDS region (read back by the same wave only)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int task = lane + 64 * i;
      const int pr = task >> 4, seg = task & 15;
      u32x4 w0, w1;
      w0[0] = pair_lo(r.va[i][0], r.vb[i][0]);
      w0[1] = pair_hi(r.va[i][0], r.vb[i][0]);
      w0[2] = pair_lo(r.va[i][1], r.vb[i][1]);
      w0[3] = pair_hi(r.va[i][1], r.vb[i][1]);
      w1[0] = pair_lo(r.va[i][2], r.vb[i][2]);
      w1[1] = pair_hi(r.va[i][2], r.vb[i][2]);
      w1[2] = pair_lo(r.va[i][3], r.vb[i][3]);
      w1[3] = pair_hi(r.va[i][3], r.vb[i][3]);
      // A lane's 32 B are two stores.  A 16-lane phase of one store covers
      // a 256 B bank line with 16 B units: with every lane storing its
      // first half first, lanes seg and seg + 8 would hit one unit (2-way
      // conflict); lanes seg >= 8 store their second half first instead.
      const bool swap = seg >= 8;
      const int x = swap ? 4 : 0;
      *reinterpret_cast<u32x4*>(&vreg[pr * kVStride + seg * 8 + x]) = swap ? w1 : w0;
      *reinterpret_cast<u32x4*>(&vreg[pr * kVStride + seg * 8 + (4 - x)]) = swap ? w0 : w1;
    }
    // mask, online max, probabilities
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = s[i] * scale_log2;
      if (k0 + acc_row(i, hf) >= lim) v = -INFINITY;
      s[i] = v;
      mt = fmaxf(mt, v);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m, mt);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - mref);   // 0 while nothing was visible
    m = m_new;
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
    lh = lh * alpha + lsum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    // O^T += V^T . P^T  (128 d x 32 query columns)
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
  };

  // Two register sets: the next split's rows load while the current is
  // computed.  The steady-state body loads unconditionally, so the compiler
  // can wait for exactly the older set; the last one or two splits are peeled.
  KVRegs ra, rb;
  int sp = s_lo;
  if (sp < s_hi) load(ra, sp);
  for (; sp + 2 < s_hi; sp += 2) {
    load(rb, sp + 1);
    process(ra, sp);
    load(ra, sp + 2);
    process(rb, sp + 1);
  }
  if (sp + 1 < s_hi) {
    load(rb, sp + 1);
    process(ra, sp);
    process(rb, sp + 1);
  } else if (sp < s_hi) {
    process(ra, sp);
  }
  const float l = lh + __shfl_xor(lh, 32);
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
  const size_t pbase = (((size_t)b * heads_kv + g) * n_part + part) * nq;
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
    if (n_part == 1) {
      // every key of the pair was seen here: normalise and write the output
      const int tq = n / group, hq = g * group + n % group;
      out[(((size_t)b * q_len + tq) * heads_q + hq) * kD + d] = f32_to_bf16(acc / lt);
      if (d == 0 && lse != nullptr)
        lse[((size_t)b * heads_q + hq) * q_len + tq] = (mx + __log2f(lt)) * kLn2;
    } else {
      part_o[(pbase + n) * kD + d] = acc;
      if (d == 0) {
        part_ml[(pbase + n) * 2] = mx;
        part_ml[(pbase + n) * 2 + 1] = lt;
      }
    }
  }
}

// Merge the P partials of one (sequence, token, query head): one wave; lanes
// read the partials' (max, sum) in parallel, then each lane sums 2 d over the
// partials with the weights broadcast from the lane that read them.
__global__ __launch_bounds__(256) void attn_decode_combine(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int batch, int q_len,
    int heads_q, int heads_kv, int n_part, uint16_t* __restrict__ out, float* __restrict__ lse) {
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
  const size_t base = ((size_t)b * heads_kv + g) * n_part;
  // n_part <= 64: lane p holds partial p
  const bool has = lane < n_part;
  const float mp = has ? part_ml[((base + lane) * nq + n) * 2] : -INFINITY;
  const float lp = has ? part_ml[((base + lane) * nq + n) * 2 + 1] : 0.f;
  float mx = mp;
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float f = (mp == -INFINITY) ? 0.f : fast_exp2(mp - mx);
  float lt = lp * f;
  for (int off = 32; off > 0; off >>= 1) lt += __shfl_xor(lt, off);
  float o0 = 0.f, o1 = 0.f;
  for (int p0 = 0; p0 < n_part; p0 += 4) {
    float2 v[4];
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pp = min(p0 + j, n_part - 1);
      w[j] = p0 + j < n_part ? __shfl(f, pp) : 0.f;
      v[j] = *reinterpret_cast<const float2*>(&part_o[((base + pp) * nq + n) * kD + 2 * lane]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o0 += v[j].x * w[j];
      o1 += v[j].y * w[j];
    }
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

namespace {
constexpr int kMaxParts = 64;

int decode_splits(int mem_len, int loc_len) {
  return (mem_len + loc_len + kSplitKeys - 1) / kSplitKeys;
}

// Runs per (sequence, KV head): enough workgroups for one per CU, never more
// runs than splits, at most kMaxParts.
int decode_parts(int batch, int heads_kv, int n_split) {
  const int pairs = batch * heads_kv;
  int p = device_cu_count() / (pairs > 0 ? pairs : 1);
  p = std::max(1, std::min({p, n_split, kMaxParts}));
  return p;
}
}  // namespace

size_t attn_decode_workspace(int batch, int q_len, int heads_q, int heads_kv, int mem_len,
                             int loc_len) {
  const int n_split = decode_splits(mem_len, loc_len);
  const int n_part = decode_parts(batch, heads_kv, n_split);
  if (n_part == 1) return 0;
  const size_t nq = (size_t)q_len * (heads_q / heads_kv);
  const size_t parts = (size_t)batch * heads_kv * n_part * nq;
  return parts * (kD + 2) * sizeof(float) + 256;
}

hipError_t launch_attn_decode(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                              const void* k_loc, const void* v_loc, int loc_len, int batch,
                              int q_len, int heads_q, int heads_kv, float scale, void* out,
                              float* lse, void* ws, hipStream_t s) {
  const int n_split = decode_splits(mem_len, loc_len);
  int n_part = decode_parts(batch, heads_kv, n_split);
  const int per_part = (n_split + n_part - 1) / n_part;
  n_part = (n_split + per_part - 1) / per_part;   // no empty runs
  const int nq = q_len * (heads_q / heads_kv);
  const size_t parts = (size_t)batch * heads_kv * n_part * nq;
  if (n_part > 1 && ws == nullptr) return hipErrorInvalidValue;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = n_part > 1 ? part_o + parts * kD : nullptr;
  const size_t smem_v = (size_t)kWaves * (kVRegionWords * 4 + kKRegionBytes);
  const size_t smem_c = ((size_t)kWaves * nq * kD + (size_t)kWaves * nq * 2) * 4;
  const size_t smem = smem_v > smem_c ? smem_v : smem_c;
  static const hipError_t attr = [] {
    const int bytes = kWaves * (32 * kD + 64) * 4 > (int)((size_t)kWaves * (kVRegionWords * 4 + kKRegionBytes))
                          ? kWaves * (32 * kD + 64) * 4
                          : (int)((size_t)kWaves * (kVRegionWords * 4 + kKRegionBytes));
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_decode_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_decode_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  const unsigned grid = (unsigned)((size_t)batch * heads_kv * n_part);
  auto kern = mem_len % 32 == 0 ? attn_decode_kernel<true> : attn_decode_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWaves * 64), smem, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_sel),
                     static_cast<const uint16_t*>(v_sel), mem_len, static_cast<const uint16_t*>(k_loc),
                     static_cast<const uint16_t*>(v_loc), loc_len, batch, q_len, heads_q, heads_kv,
                     scale * kLog2e, n_split, n_part, per_part, part_o, part_ml,
                     static_cast<uint16_t*>(out), lse);
  if (n_part > 1) {
    const int64_t rows = (int64_t)batch * q_len * heads_q;
    hipLaunchKernelGGL(attn_decode_combine, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, part_o,
                       part_ml, batch, q_len, heads_q, heads_kv, n_part, static_cast<uint16_t*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace msa
