// Chunked form of the gated delta rule (linear-layer variant: the offline
// document encoding and the query-side prefill from an injected state).
//
// Method: william-0g/MSA-Qwen3.5 model card, "Architecture summary" -- the
// linear layers run the chunked gated delta rule, with the summed states of
// the routed documents injected as the initial state.  The recurrence is the
// one msa_gated_delta_rule runs token by token:
//     S <- a_t S;   d_t = beta_t (v_t - S^T k_t);   S <- S + k_t d_t^T;   o_t = scale S^T q_t
// Over a chunk of C tokens starting from S0, with G_t the running sum of the
// log decays inside the chunk and gamma_t = exp(G_t), unrolling gives
//     d_t + sum_{j<t} beta_t exp(G_t - G_j) (k_t . k_j) d_j = beta_t (v_t - gamma_t S0^T k_t)
// i.e. (I + A) D = R with A strictly lower triangular, so D = T R with
// T = (I + A)^-1, and then
//     S_C = gamma_C S0 + K^T (exp(G_C - G) o D)
//     O   = scale (gamma o (Q S0) + (M o Q K^T) D),   M[t][j] = exp(G_t - G_j) for j <= t.
// T depends only on the chunk's keys and gates, never on S, so the T of 8
// chunks are built together ahead of the state's chain.
//
// Layout (one workgroup of 4 waves per (sequence, head); dk = dv = 128):
//  * the state lives in MFMA accumulators: wave w owns value columns
//    [32w, 32w+32) and all 128 key rows, as four 32x32 blocks;
//  * every contraction over rows of the state or of a chunk is done in the
//    accumulator's own row order (a lane half's k-slots are the rows its
//    accumulator registers hold), so accumulators feed the next MFMA as B
//    operands without moving through LDS;
//  * float32 x float32 products run on the bf16 MFMA as hi + lo splits
//    (x = hi + lo, both bf16, |x - hi - lo| <= 2^-18 |x|): two passes where
//    one side is an exact bf16 input (K, Q), three (hi.hi + hi.lo + lo.hi)
//    where both are float32 (T R and the masked Q K^T times D).
#include "attn_common.h"

namespace msa {
namespace {

using attn::acc_row;
using attn::as_bf16x8;
using attn::fast_exp2;
using attn::kLog2e;
using attn::mfma32;
using attn::kRsrcWord3;
using attn::pack_bf16x2;

constexpr int kC = 32;          // tokens per chunk
constexpr int kGroup = 8;       // chunks whose T matrices are built together
constexpr int kRowB = 272;      // bytes per K / Q row in LDS: 256 + 16 (rows land 16 B apart in the banks)
constexpr int kTP = 36;         // floats per row of a chunk's A / T in LDS (144 B: 16 rows, 16 distinct units)
constexpr int kKBytes = kC * kRowB;                  // one staged chunk of K, V or Q
constexpr int kTBytes = kGroup * kC * kTP * 4;       // the group's T matrices

// hi + lo bf16 split of 8 float32 values, packed as two MFMA operands.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t hp = pack_bf16x2(x[2 * w], x[2 * w + 1]);
    h[w] = hp;
    l[w] = pack_bf16x2(x[2 * w] - __uint_as_float(hp << 16), x[2 * w + 1] - __uint_as_float(hp & 0xFFFF0000u));
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}
__device__ __forceinline__ void split_acc(const f32x16& a, int s, bf16x8& hi, bf16x8& lo) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = a[8 * s + e];
  split8(x, hi, lo);
}
// Row of accumulator element i within its lane half's rows (acc_row(i, hf) = 4 hf + arow(i)); the
// addresses below are a per-lane base plus arow(i) times a constant, so they fold into offsets.
__device__ constexpr int arow(int i) { return 8 * (i >> 2) + (i & 3); }
__device__ __forceinline__ uint32_t u16pair(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }
// Buffer resource over `bytes` bytes at p: loads past the end read zero and
// stores past the end are dropped (the ragged last chunk needs no branches).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

template <bool WITH_OUT>
__global__ __launch_bounds__(256, WITH_OUT ? 1 : 2) void gdn_chunked_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float scale, const float* __restrict__ init,
    int seq_len, int heads, uint16_t* __restrict__ out, float* __restrict__ final_state) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* sK = smem;                                          // [kC rows][kRowB] the chunk's keys
  uint8_t* sV = sK + kKBytes;                                  // [kC][kRowB] values
  uint8_t* sQ = sV + kKBytes;                                  // [kC][kRowB] queries (outputs only)
  float* sT = reinterpret_cast<float*>(sQ + (WITH_OUT ? kKBytes : 0));   // [kGroup][kC][kTP]
  float* sG = sT + kTBytes / 4;                                // [kGroup * kC] running log2-decay per chunk
  float* sB = sG + kGroup * kC;                                // [kGroup * kC] beta

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = 32 * wave + cl;                                // this lane's value column
  const int r4 = 4 * hf;                                       // first accumulator row of this lane half
  const int dlt = cl - r4;                                     // row 4 hf + a is above column cl iff a > dlt
  const uint32_t tb2 = (uint32_t)heads * 256u;                 // bytes between tokens of q / k / v
  const size_t base = ((size_t)b * seq_len * heads + h) * 128; // token 0 of (b, h)
  const size_t gbase = (size_t)b * seq_len * heads + h;        // g / beta of token 0
  const size_t sbase = ((size_t)b * heads + h) * 128 * 128;    // state of (b, h)
  const int n_chunks = (seq_len + kC - 1) / kC;
  // the rows of (b, h): tokens past seq_len fall outside
  const uint32_t span = (uint32_t)seq_len * tb2 - (uint32_t)h * 256u;
  const __amdgpu_buffer_rsrc_t rk = rsrc(k + base, span);
  const __amdgpu_buffer_rsrc_t rq = rsrc(WITH_OUT ? q + base : k + base, span);
  const __amdgpu_buffer_rsrc_t rv = rsrc(v + base, span);
  // this lane's rows acc_row(i, hf) sit at row0 + (8 (i / 4) + i % 4) tokens
  const uint32_t row0 = (uint32_t)(4 * hf) * tb2 + 2u * n;

  // state: S[db][i] = S[32 db + acc_row(i, hf)][n]  (no initial state: zeros).  The lane's part
  // of the offset is per lane, the row's part a constant (never out of range here)
  const uint32_t s_lane = (uint32_t)(4 * hf * 128 + n) * 4u;
  f32x16 S[4];
  {
    const __amdgpu_buffer_rsrc_t ri = rsrc(init != nullptr ? init + sbase : init, init != nullptr ? 65536u : 0u);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        S[db][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ri, s_lane, (32 * db + 8 * (i >> 2) + (i & 3)) * 512, 0));
  }

  // staging of one chunk's K, V (and Q) rows: two 16 B pieces per thread each
  u32x4 pk[2], pv[2], pq[2];
  auto fetch_kq = [&](int cg) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int piece = tid + 256 * p, row = piece >> 4, seg = piece & 15;
      const uint32_t off = (uint32_t)(cg * kC + row) * tb2 + seg * 16u;
      pk[p] = attn::bload(rk, off, 0);
      pv[p] = attn::bload(rv, off, 0);
      if (WITH_OUT) pq[p] = attn::bload(rq, off, 0);
    }
  };
  auto stash_kq = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int piece = tid + 256 * p, row = piece >> 4, seg = piece & 15;
      *reinterpret_cast<u32x4*>(sK + row * kRowB + seg * 16) = pk[p];
      *reinterpret_cast<u32x4*>(sV + row * kRowB + seg * 16) = pv[p];
      if (WITH_OUT) *reinterpret_cast<u32x4*>(sQ + row * kRowB + seg * 16) = pq[p];
    }
  };

  // T matrices of the group starting at chunk cg0 (wave w builds chunks 2w and 2w + 1)
  auto build_group = [&](int cg0) __attribute__((always_inline)) {
    // running log2-decay and beta of the group's 256 tokens: lane half = one chunk
    {
      const int t = cg0 * kC + tid;
      float gv = 0.f, bv = 0.f;
      if (t < seq_len) {
        gv = g[gbase + (size_t)t * heads];
        bv = beta[gbase + (size_t)t * heads];
      }
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) {
        const float o = __shfl_up(gv, d, 32);
        if (cl >= d) gv += o;
      }
      sG[tid] = gv * kLog2e;
      sB[tid] = bv;
    }
    // A = beta_i exp(G_i - G_l) (k_i . k_l) for l < i, both chunks of this wave
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = 2 * wave + cc;
      const uint32_t off = (uint32_t)((cg0 + c) * kC + cl) * tb2 + 16u * hf;
      f32x16 X = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = as_bf16x8(attn::bload(rk, off + 32u * ks, 0));
        X = mfma32(a, a, X);
      }
      const float* gcl = sG + c * kC + r4;
      const float* bcl = sB + c * kC + r4;
      const float gl = sG[c * kC + cl];
      float* Tl = sT + c * kC * kTP + r4 * kTP + cl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a = bcl[arow(r)] * fast_exp2(gcl[arow(r)] - gl) * X[r];
        Tl[arow(r) * kTP] = dlt < arow(r) ? a : 0.f;
      }
    }
    // T = (I + A)^-1, column cl of chunk 2w + hf: T e_cl = e_cl + z with (I + A) z = -A e_cl,
    // by forward substitution (z is zero down to row cl).  Row i of A is read before row i
    // of T is written, so the matrix is replaced in place.
    {
      float* Tc = sT + (2 * wave + hf) * kC * kTP;
      float z[kC];
#pragma unroll
      for (int i = 0; i < kC; ++i) {
        float s0 = Tc[i * kTP + cl], s1 = 0.f;
#pragma unroll
        for (int m4 = 0; m4 < kC; m4 += 4) {
          if (m4 < i) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(Tc + i * kTP + m4);
            s0 = fmaf(a[0], z[m4], s0);
            if (m4 + 1 < i) s1 = fmaf(a[1], z[m4 + 1], s1);
            if (m4 + 2 < i) s0 = fmaf(a[2], z[m4 + 2], s0);
            if (m4 + 3 < i) s1 = fmaf(a[3], z[m4 + 3], s1);
          }
        }
        z[i] = -(s0 + s1);
        asm volatile("" ::: "memory");   // the next row's loads wait here: one row in flight
      }
#pragma unroll
      for (int i = 0; i < kC; ++i) Tc[i * kTP + cl] = z[i];
      Tc[cl * kTP + cl] = 1.f;
    }
  };

  if (n_chunks > 0) {
    fetch_kq(0);
    stash_kq();
  }

  for (int cg = 0; cg < n_chunks; ++cg) {
    const int c = cg % kGroup;
    const int t0 = cg * kC;
    const bool more = cg + 1 < n_chunks;
    if (c == 0) build_group(cg);
    __syncthreads();   // the chunk's rows and the group's T are in place
    if (more) fetch_kq(cg + 1);
    const uint8_t* kc = sK;
    const uint8_t* qc = sQ;
    const uint8_t* kl = kc + cl * kRowB + r4 * 2;   // row cl, columns from 4 hf
    const uint8_t* ql = qc + cl * kRowB + r4 * 2;
    const float* gc = sG + c * kC;
    const float* bc = sB + c * kC;

    // P = K S0 (and Q S0): contraction over the state's rows in its accumulator order
    f32x16 P = {}, QS = {};
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 sh, sl;
        split_acc(S[db], s, sh, sl);
        const int col = 32 * db + 16 * s;       // + 4 hf in the lane's base
        u32x4 a;
        {
          const uint2 a0 = *reinterpret_cast<const uint2*>(kl + col * 2);
          const uint2 a1 = *reinterpret_cast<const uint2*>(kl + (col + 8) * 2);
          a = u32x4{a0.x, a0.y, a1.x, a1.y};
        }
        P = mfma32(as_bf16x8(a), sh, P);
        P = mfma32(as_bf16x8(a), sl, P);
        if (WITH_OUT) {
          const uint2 b0 = *reinterpret_cast<const uint2*>(ql + col * 2);
          const uint2 b1 = *reinterpret_cast<const uint2*>(ql + (col + 8) * 2);
          const u32x4 qa = {b0.x, b0.y, b1.x, b1.y};
          QS = mfma32(as_bf16x8(qa), sh, QS);
          QS = mfma32(as_bf16x8(qa), sl, QS);
        }
        __builtin_amdgcn_sched_barrier(0);   // one step's split and operands live at a time
      }
    // X = K Q^T (keys j = rows, queries t = columns)
    f32x16 X = {};
    if (WITH_OUT) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(kl + r4 * 2 + 32 * ks);   // columns 16 ks + 8 hf
        const u32x4 qb = *reinterpret_cast<const u32x4*>(ql + r4 * 2 + 32 * ks);
        X = mfma32(as_bf16x8(ka), as_bf16x8(qb), X);
      }
    }
    // R = beta (V - gamma P), rows acc_row(i, hf)
    float gr[16];
    f32x16 R;
    {
      const float* gcl = gc + r4;
      const float* bcl = bc + r4;
      const uint8_t* vl = sV + r4 * kRowB + n * 2;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        gr[i] = gcl[arow(i)];
        const uint32_t vt = *reinterpret_cast<const uint16_t*>(vl + arow(i) * kRowB);
        R[i] = bcl[arow(i)] * (__uint_as_float(vt << 16) - fast_exp2(gr[i]) * P[i]);
      }
    }
    // D = T R (three passes)
    f32x16 D = {};
    {
      const float* Tc = sT + c * kC * kTP + cl * kTP;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4 t0v = *reinterpret_cast<const f32x4*>(Tc + 16 * s + 4 * hf);
        const f32x4 t1v = *reinterpret_cast<const f32x4*>(Tc + 16 * s + 8 + 4 * hf);
        const float tx[8] = {t0v[0], t0v[1], t0v[2], t0v[3], t1v[0], t1v[1], t1v[2], t1v[3]};
        bf16x8 th, tl, rh, rl;
        split8(tx, th, tl);
        split_acc(R, s, rh, rl);
        D = mfma32(th, rh, D);
        D = mfma32(th, rl, D);
        D = mfma32(tl, rh, D);
      }
    }
    if (WITH_OUT) {
      // O = scale (gamma o (Q S0) + (M o Q K^T) D): the masked scores are the A operand as they lie
      const float gq = gc[cl];
      f32x16 Xm;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Xm[i] = arow(i) <= dlt ? fast_exp2(gq - gr[i]) * X[i] : 0.f;   // key row <= query column
      }
      f32x16 O = {};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 xh, xl, dh, dl;
        split_acc(Xm, s, xh, xl);
        split_acc(D, s, dh, dl);
        O = mfma32(xh, dh, O);
        O = mfma32(xh, dl, O);
        O = mfma32(xl, dh, O);
      }
      const __amdgpu_buffer_rsrc_t ro = rsrc(out + base, span);
      const uint32_t off = (uint32_t)t0 * tb2 + row0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(scale * (fast_exp2(gr[i]) * QS[i] + O[i])), ro,
                                              off + (uint32_t)(8 * (i >> 2) + (i & 3)) * tb2, 0, 0);
    }
    // S <- gamma_C S + K^T (exp(G_C - G) o D)
    {
      const float gC = gc[kC - 1];
      const float decay = fast_exp2(gC);
      f32x16 Dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) Dp[i] = fast_exp2(gC - gr[i]) * D[i];
      bf16x8 dh[2], dl[2];
      split_acc(Dp, 0, dh[0], dl[0]);
      split_acc(Dp, 1, dh[1], dl[1]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) S[db][i] *= decay;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          // K^T operand: rows 16s + 4hf + {0..3} and 16s + 8 + 4hf + {0..3}, key column 32 db + cl
          const uint8_t* kcol = kc + r4 * kRowB + (32 * db + cl) * 2;
          uint16_t e[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[r] = *reinterpret_cast<const uint16_t*>(kcol + (16 * s + r) * kRowB);
            e[4 + r] = *reinterpret_cast<const uint16_t*>(kcol + (16 * s + 8 + r) * kRowB);
          }
          const u32x4 kt = {u16pair(e[0], e[1]), u16pair(e[2], e[3]), u16pair(e[4], e[5]), u16pair(e[6], e[7])};
          S[db] = mfma32(as_bf16x8(kt), dh[s], S[db]);
          S[db] = mfma32(as_bf16x8(kt), dl[s], S[db]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // every wave is done with this chunk's rows (and the group's T) before they are replaced
    __syncthreads();
    if (more) stash_kq();
  }

  if (final_state != nullptr) {
    const __amdgpu_buffer_rsrc_t rf = rsrc(final_state + sbase, 65536u);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[db][i]), rf, s_lane,
                                              (32 * db + 8 * (i >> 2) + (i & 3)) * 512, 0);
  }
}

template <bool WITH_OUT>
hipError_t launch_t(const void* q, const void* k, const void* v, const float* g, const float* beta, float scale,
                    const float* init, int batch, int seq_len, int heads, void* out, float* final_state,
                    hipStream_t s) {
  const size_t lds = (WITH_OUT ? 3 : 2) * (size_t)kKBytes + kTBytes + 2 * kGroup * kC * 4;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(gdn_chunked_kernel<WITH_OUT>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(gdn_chunked_kernel<WITH_OUT>, dim3((unsigned)heads, (unsigned)batch), dim3(256), lds, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), g, beta, scale, init, seq_len, heads,
                     static_cast<uint16_t*>(out), final_state);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_chunked(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              float scale, const float* init, int batch, int seq_len, int heads, void* out,
                              float* final_state, hipStream_t s) {
  if (out != nullptr)
    return launch_t<true>(q, k, v, g, beta, scale, init, batch, seq_len, heads, out, final_state, s);
  return launch_t<false>(q, k, v, g, beta, scale, init, batch, seq_len, heads, nullptr, final_state, s);
}

}  // namespace msa
