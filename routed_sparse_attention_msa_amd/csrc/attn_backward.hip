// Backward of the sparse GQA attention, for training through the routed layer.
//
// Method: MSA README, "Abstract" and the Figure 1 caption -- top-k selection
// is fused with a sparse attention that stays end-to-end differentiable;
// william-0g/MSA-Qwen3.5 model card, "Architecture summary" and "Training
// (CPT)" -- the router and adapters train through the routed layers.  The
// forward is the attention of attn_prefill.hip: query token t sees the M
// gathered memory rows and the local rows 0 .. L_loc - T + t.
//
// With P = softmax(scale * Q K^T) over the visible keys, recomputed from the
// forward's log-sum-exp, and D_t = sum_d dO[t,d] O[t,d] (= sum_j P_tj dP_tj):
//     dP = dO V^T,   dS = P o (dP - D),   dQ = scale dS K,
//     dK = scale dS^T Q,   dV = P^T dO,
// and a KV head's dK, dV sum over the query heads of its group.
//
// bf16, head dim 128, on MFMA, in two kernels without atomics (deterministic):
//  * dq kernel -- one workgroup per (sequence, KV head, 32 tokens), one wave
//    per query head of the group, as in the forward: S^T = K Q^T and
//    dP^T = V dO^T with a lane owning one query, so lse and D are lane
//    scalars; dS^T, converted to bf16 in registers, is the B operand of
//    dQ^T += K^T dS^T (K^T staged in the transposed operand groups).  It
//    also writes D for the second kernel.
//  * dk/dv kernel -- one workgroup per (sequence, KV head, 128 keys), one wave
//    per 32 keys: S = Q K^T and dP = dO V^T with a lane owning one key (K and
//    V rows held in registers for the whole kernel); P and dS in bf16 are the
//    B operands of dV^T += dO^T P and dK^T += Q^T dS.  The loop runs over the
//    group's query heads and over the query tiles that see the keys; each
//    tile (Q and dO rows, both again transposed, lse, D) is staged once in
//    LDS for the workgroup's four waves (two of them stage it).
// Every other shape (float32, other head dims, group size 1) runs on the
// vector-ALU kernels at the end of the file.
#include <algorithm>

#include "attn_common.h"

namespace msa {
namespace {

using namespace attn;

constexpr int kKT = 64;   // keys per tile of the dq kernel

// ---------------------------------------------------------------------------
// dq kernel (MFMA)
// ---------------------------------------------------------------------------
struct DqTile {
  uint8_t k[kKT * kKPitch];          // K rows: A operand of S^T
  uint8_t v[kKT * kKPitch];          // V rows: A operand of dP^T
  uint8_t kt[8 * kVGStride * 16];    // K^T groups: A operand of dQ^T
};
struct DqSmem {
  DqTile buf[2];                     // double-buffered: the next tile is stored while this one is read
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_sel,
    const uint16_t* __restrict__ v_sel, int mem_len, const uint16_t* __restrict__ k_loc,
    const uint16_t* __restrict__ v_loc, int loc_len, const uint16_t* __restrict__ out,
    const uint16_t* __restrict__ d_out, const float* __restrict__ lse, int batch, int q_len,
    int heads_q, int heads_kv, float scale, float scale_log2, uint16_t* __restrict__ dq,
    float* __restrict__ dsum) {
  constexpr int kThreads = NW * 64;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  DqSmem& sm = *reinterpret_cast<DqSmem*>(smem_raw);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int group = heads_q / heads_kv;
  const int hsub = group / NW;
  const int n_tblk = (q_len + 31) / 32;

  int bid = blockIdx.x;
  const int hs = bid % hsub;
  bid /= hsub;
  const int g = bid % heads_kv;
  bid /= heads_kv;
  const int b = bid % batch;
  const int tb = n_tblk - 1 - bid / batch;       // longest blocks first
  const int h = g * group + hs * NW + wave;
  const int t0 = tb * 32;
  const int t = t0 + cl;
  const bool t_ok = t < q_len;

  const uint32_t rs = (uint32_t)heads_kv * kD * 2;
  const size_t sel_rows = (size_t)b * mem_len * heads_kv * kD;
  const size_t loc_rows = (size_t)b * loc_len * heads_kv * kD;
  const uint32_t sel_bytes = (uint32_t)((size_t)mem_len * rs);
  const uint32_t loc_bytes = (uint32_t)((size_t)loc_len * rs);
  const KVRows kr{__builtin_amdgcn_make_buffer_rsrc((void*)(k_sel + (mem_len ? sel_rows : 0)), (short)0, sel_bytes, kRsrcWord3),
                  __builtin_amdgcn_make_buffer_rsrc((void*)(k_loc + loc_rows), (short)0, loc_bytes, kRsrcWord3),
                  rs};
  const KVRows vr{__builtin_amdgcn_make_buffer_rsrc((void*)(v_sel + (mem_len ? sel_rows : 0)), (short)0, sel_bytes, kRsrcWord3),
                  __builtin_amdgcn_make_buffer_rsrc((void*)(v_loc + loc_rows), (short)0, loc_bytes, kRsrcWord3),
                  rs};

  const int causal0 = mem_len + loc_len - q_len;
  const int n_mt = (mem_len + kKT - 1) / kKT;
  const int loc_need = loc_len - q_len + min(t0 + 32, q_len);
  const int n_tiles = n_mt + (loc_need + kKT - 1) / kKT;
  const int full_below = causal0 + t0 + 1;
  auto tile_mem = [&](int tile) { return tile < n_mt; };
  auto tile_row0 = [&](int tile) { return tile < n_mt ? tile * kKT : (tile - n_mt) * kKT; };
  auto tile_kappa0 = [&](int tile) { return tile < n_mt ? tile * kKT : mem_len + (tile - n_mt) * kKT; };

  // this lane's query: Q^T and dO^T slices (d-slots 64*(s/4) + 32*hf + 8*(s%4)),
  // D = dO . O over the stored output, lse in log2 units
  bf16x8 qf[8], df[8];
  float dpart = 0.f;
  {
    const size_t row = (((size_t)b * q_len + (t_ok ? t : 0)) * heads_q + h) * kD;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int off = 64 * (s >> 2) + 32 * hf + 8 * (s & 3);
      const u32x4 qv = load16(q + row + off);
      const u32x4 dv = load16(d_out + row + off);
      const u32x4 ov = load16(out + row + off);
      qf[s] = as_bf16x8(t_ok ? qv : z);
      df[s] = as_bf16x8(t_ok ? dv : z);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dpart = fmaf(__uint_as_float(dv[e] << 16), __uint_as_float(ov[e] << 16), dpart);
        dpart = fmaf(__uint_as_float(dv[e] & 0xFFFF0000u), __uint_as_float(ov[e] & 0xFFFF0000u), dpart);
      }
    }
  }
  const float d_t = t_ok ? dpart + __shfl_xor(dpart, 32) : 0.f;
  const float lse2 = t_ok ? lse[((size_t)b * heads_q + h) * q_len + t] * kLog2e : 0.f;
  if (t_ok && hf == 0) dsum[((size_t)b * heads_q + h) * q_len + t] = d_t;

  // staging through buffer loads: V rows in 16-byte chunks (16 rows per
  // pass); K in tasks of four rows x one 8-d block -- the tasks cover every
  // chunk of the tile once, so each K chunk is loaded once and written both
  // as a row (A of S^T) and into the transposed groups (A of dQ^T)
  constexpr int kRowChunks = kKT * 16 / kThreads;
  constexpr int kRowStep = kThreads / 16;
  constexpr int kTTasks = 256 / kThreads;
  const uint32_t goff = (uint32_t)g * kD * 2;
  const uint32_t row_voff = (uint32_t)(tid >> 4) * rs + goff + (tid & 15) * 16;
  u32x4 pv[kRowChunks], pt[kTTasks][4];
  auto gload = [&](int tile) {
    const bool mem = tile_mem(tile);
    const int row0 = tile_row0(tile);
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) pv[i] = vr.load(mem, row0 + kRowStep * i, row_voff);
#pragma unroll
    for (int i = 0; i < kTTasks; ++i) {
      const uint32_t voff = (uint32_t)vtask_row0(tid + kThreads * i) * rs + goff + (tid & 15) * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) pt[i][j] = kr.load(mem, row0 + j, voff);
    }
  };
  auto lstore = [&](DqTile& tl) {
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(&tl.v[(c >> 4) * kKPitch + (c & 15) * 16]) = pv[i];
    }
#pragma unroll
    for (int i = 0; i < kTTasks; ++i) {
      const int c = tid + kThreads * i;
      const int r0 = vtask_row0(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&tl.k[(r0 + j) * kKPitch + (c & 15) * 16]) = pt[i][j];
      store_transposed(tl.kt, c >> 5, (c >> 4) & 1, c & 15, pt[i]);
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};

  // the next tile's loads are in flight while this one is computed (clamped
  // to the last tile, so the loads are unconditional)
  gload(0);
  lstore(sm.buf[0]);
  __syncthreads();
  gload(min(1, n_tiles - 1));
  for (int tile = 0; tile < n_tiles; ++tile) {
    const DqTile& tl = sm.buf[tile & 1];
    const int kappa0 = tile_kappa0(tile);
    const uint8_t* kbase = &tl.k[cl * kKPitch + hf * 64];
    const uint8_t* vbase = &tl.v[cl * kKPitch + hf * 64];
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kf[8], vf[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int o = kb * 32 * kKPitch + (8 * (st >> 2) + (st & 3)) * 16;
        kf[st] = *reinterpret_cast<const bf16x8*>(kbase + o);
        vf[st] = *reinterpret_cast<const bf16x8*>(vbase + o);
      }
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        s[kb] = mfma32(kf[st], qf[st], s[kb]);
        dp[kb] = mfma32(vf[st], df[st], dp[kb]);
      }
      // all sixteen operand reads before the MFMAs (otherwise each MFMA
      // waited for its own read, issued into one reused register quad)
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
    const bool mem = tile_mem(tile);
    if (mem ? kappa0 + kKT > mem_len : kappa0 + kKT > full_below) {
      const int lim = mem ? mem_len : causal0 + t + 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kappa0 + kb * 32 + acc_row(i, hf) >= lim) s[kb][i] = -INFINITY;
    }
    // dS^T = P^T o (dP^T - D), to bf16 in the B-operand order of dQ^T
    bf16x8 dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i0 = 8 * s2 + 2 * e;
          const float p0 = fast_exp2(fmaf(s[kb][i0], scale_log2, -lse2));
          const float p1 = fast_exp2(fmaf(s[kb][i0 + 1], scale_log2, -lse2));
          w[e] = pack_bf16x2(p0 * (dp[kb][i0] - d_t), p1 * (dp[kb][i0 + 1] - d_t));
        }
        dsf[kb][s2] = as_bf16x8(w);
      }
    // dQ^T += K^T dS^T
    const uint8_t* tbase = &tl.kt[(hf * kVGStride + vg_lane(cl)) * 16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 kt[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          kt[db] = *reinterpret_cast<const bf16x8*>(tbase + ((4 * kb + 2 * s2) * kVGStride + kVGBlock * db) * 16);
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = mfma32(kt[db], dsf[kb][s2], acc[db]);
      }
    lstore(sm.buf[(tile + 1) & 1]);
    __syncthreads();
    gload(min(tile + 2, n_tiles - 1));
  }

  if (!t_ok) return;
  uint16_t* qrow = dq + (((size_t)b * q_len + t) * heads_q + h) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = db * 32 + 8 * qd + 4 * hf;
      uint2 w;
      w.x = pack_bf16x2(acc[db][4 * qd] * scale, acc[db][4 * qd + 1] * scale);
      w.y = pack_bf16x2(acc[db][4 * qd + 2] * scale, acc[db][4 * qd + 3] * scale);
      *reinterpret_cast<uint2*>(qrow + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// dk/dv kernel (MFMA)
// ---------------------------------------------------------------------------
constexpr int kQT = 32;   // query rows per staged tile

struct DkvTile {
  uint8_t q[kQT * kKPitch];          // Q rows: A operand of S
  uint8_t o[kQT * kKPitch];          // dO rows: A operand of dP
  uint8_t qt[4 * kVGStride * 16];    // Q^T groups: A operand of dK^T
  uint8_t ot[4 * kVGStride * 16];    // dO^T groups: A operand of dV^T
  float lse2[kQT];                   // log2-unit lse (+inf past the last token)
  float dsum[kQT];
};
struct DkvSmem {
  DkvTile buf[2];
};

// Work unit = (sequence, KV head, NWK key blocks of 32, part).  The unit's
// items are (query head of the group, query tile) pairs that see its keys,
// head-major; the items are split evenly over n_parts units, whose float32
// partial dK, dV a second kernel sums in part order (with one part the unit
// writes bf16 directly).
template <int NWK>
__global__ __launch_bounds__(NWK * 64) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_sel,
    const uint16_t* __restrict__ v_sel, int mem_len, const uint16_t* __restrict__ k_loc,
    const uint16_t* __restrict__ v_loc, int loc_len, const uint16_t* __restrict__ d_out,
    const float* __restrict__ lse, const float* __restrict__ dsum, int batch, int q_len,
    int heads_q, int heads_kv, float scale, float scale_log2, int n_parts,
    uint16_t* __restrict__ dk_sel, uint16_t* __restrict__ dv_sel, uint16_t* __restrict__ dk_loc,
    uint16_t* __restrict__ dv_loc, float* __restrict__ part_dk, float* __restrict__ part_dv) {
  constexpr int kThreads = NWK * 64;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  DkvSmem& sm = *reinterpret_cast<DkvSmem*>(smem_raw);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int group = heads_q / heads_kv;
  const int n_mb = (mem_len + 31) / 32;
  const int n_kb = n_mb + (loc_len + 31) / 32;
  const int n_keys = mem_len + loc_len;

  int bid = blockIdx.x;
  const int g = bid % heads_kv;
  bid /= heads_kv;
  const int b = bid % batch;
  bid /= batch;
  const int part = bid % n_parts;
  const int wg = bid / n_parts;                   // memory blocks and early local rows first
  const int kb_first = wg * NWK;

  // this wave's 32 keys: memory rows or local rows (never both)
  const int kbi = kb_first + wave;
  const bool active = kbi < n_kb;
  const bool mem = kbi < n_mb;
  const int row0 = mem ? 32 * kbi : 32 * (kbi - n_mb);
  const int n_rows = active ? min(32, (mem ? mem_len : loc_len) - row0) : 0;
  const int shift = loc_len - q_len;              // local row r is visible to tokens t >= r - shift
  auto first_token = [&](int kb) {
    return kb < n_mb ? 0 : max(0, 32 * (kb - n_mb) - shift);
  };
  const int my_tile0 = active ? first_token(kbi) / kQT : 0x7FFFFFFF;
  const int wg_tile0 = first_token(kb_first) / kQT;
  const int n_qt = (q_len + kQT - 1) / kQT;
  const int n_qt_wg = n_qt - wg_tile0;
  const int n_items = group * n_qt_wg;
  const int it_lo = (int)((int64_t)part * n_items / n_parts);
  const int it_hi = (int)((int64_t)(part + 1) * n_items / n_parts);

  // K and V rows of this lane's key as B operands (segments 8*(st/4) + 4*hf + st%4)
  // (a wave without keys reads local row 0, which always exists, and drops it)
  bf16x8 kf[8], vf[8];
  {
    const bool use_mem = active && mem;
    const int row = active ? row0 + min(cl, n_rows - 1) : 0;
    const int rows_len = use_mem ? mem_len : loc_len;
    const uint16_t* kb_ = use_mem ? k_sel : k_loc;
    const uint16_t* vb_ = use_mem ? v_sel : v_loc;
    const size_t off = ((((size_t)b * rows_len + row) * heads_kv + g) * kD);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int seg = 8 * (st >> 2) + 4 * hf + (st & 3);
      const u32x4 kv = load16(kb_ + off + 8 * seg);
      const u32x4 vv = load16(vb_ + off + 8 * seg);
      kf[st] = as_bf16x8(active ? kv : z);
      vf[st] = as_bf16x8(active ? vv : z);
    }
  }
  const int kappa_row = row0 + cl;               // this lane's key row (memory or local)
  const bool key_ok = cl < n_rows;

  // staging of one (query head, 32-token) tile: rows through a buffer resource
  // over the head's q_len rows (rows past the last token read as zeros)
  // (tasks of four rows x one 8-d block cover every chunk of the tile once:
  // each chunk is loaded once and written both as a row and transposed)
  const uint32_t qrs = (uint32_t)heads_q * kD * 2;
  constexpr int kTTasks = (128 + kThreads - 1) / kThreads;   // 128 tasks per tile (whole waves past them idle)
  u32x4 tq[kTTasks][4], to[kTTasks][4];
  float plse = 0.f, pds = 0.f;
  auto gload = [&](int it) {
    const int h = g * group + it / n_qt_wg;
    const int tq0 = (wg_tile0 + it % n_qt_wg) * kQT;
    const size_t base = ((size_t)b * q_len * heads_q + h) * kD;
    const uint32_t nbytes = (uint32_t)((size_t)q_len * qrs - (size_t)h * kD * 2);
    // (base and size through readfirstlane: the compiler did not always prove
    // them uniform, and a descriptor in vector registers makes every load a
    // loop over the lanes' values)
    auto uniform_rsrc = [](const uint16_t* p, uint32_t bytes) {
      const uint64_t a = (uint64_t)(uintptr_t)p;
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
      void* u = reinterpret_cast<void*>((uintptr_t)(((uint64_t)hi << 32) | lo));
      return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
    };
    const __amdgpu_buffer_rsrc_t qr = uniform_rsrc(q + base, nbytes);
    const __amdgpu_buffer_rsrc_t orr = uniform_rsrc(d_out + base, nbytes);
    // the tile's first row goes in the scalar offset, the lane's row in the
    // vector offset (a per-lane scalar offset would make the compiler loop
    // over its distinct values)
    const uint32_t soff = (uint32_t)tq0 * qrs;
#pragma unroll
    for (int i = 0; i < kTTasks; ++i) {
      const int c = tid + kThreads * i;
      if (kThreads > 128 && wave * 64 + kThreads * i >= 128) break;   // whole waves (wave is uniform)
      const int r0 = vtask_row0(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t voff = (uint32_t)(r0 + j) * qrs + (c & 15) * 16;
        tq[i][j] = bload(qr, voff, soff);
        to[i][j] = bload(orr, voff, soff);
      }
    }
    const int tt = tq0 + (tid & (kQT - 1));
    const size_t li = ((size_t)b * heads_q + h) * q_len + min(tt, q_len - 1);
    plse = tt < q_len ? lse[li] * kLog2e : INFINITY;
    pds = tt < q_len ? dsum[li] : 0.f;
  };
  auto lstore = [&](DkvTile& tl) {
#pragma unroll
    for (int i = 0; i < kTTasks; ++i) {
      const int c = tid + kThreads * i;
      if (kThreads > 128 && wave * 64 + kThreads * i >= 128) break;   // whole waves (wave is uniform)
      const int r0 = vtask_row0(c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4*>(&tl.q[(r0 + j) * kKPitch + (c & 15) * 16]) = tq[i][j];
        *reinterpret_cast<u32x4*>(&tl.o[(r0 + j) * kKPitch + (c & 15) * 16]) = to[i][j];
      }
      store_transposed(tl.qt, c >> 5, (c >> 4) & 1, c & 15, tq[i]);
      store_transposed(tl.ot, c >> 5, (c >> 4) & 1, c & 15, to[i]);
    }
    if (tid < kQT) {
      tl.lse2[tid] = plse;
      tl.dsum[tid] = pds;
    }
  };

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  if (it_lo < it_hi) {
    // the next item's loads are in flight while this one is computed (clamped
    // to the unit's last item, so the loads are unconditional)
    gload(it_lo);
    lstore(sm.buf[0]);
    __syncthreads();
    gload(min(it_lo + 1, it_hi - 1));
    for (int it = it_lo; it < it_hi; ++it) {
      const DkvTile& tl = sm.buf[(it - it_lo) & 1];
      const int qt = wg_tile0 + it % n_qt_wg;
      if (qt >= my_tile0) {                        // uniform per wave
        const int tq0 = qt * kQT;
        // S = Q K^T and dP = dO V^T: lane (key cl, half hf) holds query rows acc_row(i, hf)
        const uint8_t* qbase = &tl.q[cl * kKPitch + hf * 64];
        const uint8_t* obase = &tl.o[cl * kKPitch + hf * 64];
        bf16x8 qa[8], oa[8];
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int o = (8 * (st >> 2) + (st & 3)) * 16;
          qa[st] = *reinterpret_cast<const bf16x8*>(qbase + o);
          oa[st] = *reinterpret_cast<const bf16x8*>(obase + o);
        }
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          s = mfma32(qa[st], kf[st], s);
          dp = mfma32(oa[st], vf[st], dp);
        }
        // the operand reads ahead of the MFMAs, eight at a time (one read per
        // MFMA made each MFMA wait for its own read)
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        float l2[16], dd[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&tl.lse2[8 * j + 4 * hf]);
          const f32x4 c = *reinterpret_cast<const f32x4*>(&tl.dsum[8 * j + 4 * hf]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            l2[4 * j + i] = a[i];
            dd[4 * j + i] = c[i];
          }
        }
        // visibility: a real key, and for local keys row <= shift + t; rows
        // past the last token have lse2 = +inf (P = 0).  A hidden element's
        // exponent argument becomes -inf (P = 0, dS = 0) by integer masking of
        // its bits, with no branch: a conditional assignment (to the
        // accumulator, or a select the compiler turned back into control
        // flow) made a branch per element, around which every dK/dV
        // accumulator was copied out of its registers and back on every tile.
        // Element i holds query row 4 hf + c_i of the tile (c_i = 8 (i / 4) + i % 4,
        // 0 .. 27) and is hidden exactly when c_i < u, with u per lane and item:
        // above every c_i without a key, below every c_i for a memory row, and
        // for a local row the first row that sees it less 4 hf (row r sees it
        // iff kappa_row <= shift + tq0 + r), clamped to [-1, 32].  The compiler
        // turns the sign mask into one compare and one select per element.
        const int u = !key_ok ? 32 : (mem ? -1 : min(32, max(-1, kappa_row - shift - tq0 - 4 * hf)));
        auto arg = [&](int i) {
          const float x = fmaf(s[i], scale_log2, -l2[i]);
          const int c = 8 * (i >> 2) + (i & 3);
          const unsigned m = (unsigned)((c - u) >> 31);                        // all ones when hidden
          return __uint_as_float((__float_as_uint(x) & ~m) | (0xFF800000u & m));
        };
        bf16x8 pf[2], dsf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 wp, wd;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i0 = 8 * s2 + 2 * e;
            const float p0 = fast_exp2(arg(i0));
            const float p1 = fast_exp2(arg(i0 + 1));
            wp[e] = pack_bf16x2(p0, p1);
            wd[e] = pack_bf16x2(p0 * (dp[i0] - dd[i0]), p1 * (dp[i0 + 1] - dd[i0 + 1]));
          }
          pf[s2] = as_bf16x8(wp);
          dsf[s2] = as_bf16x8(wd);
        }
        // dV^T += dO^T P and dK^T += Q^T dS (lane (d, hf) reads its 8 queries of group 2*s2 + hf)
        const int tb_ = (hf * kVGStride + vg_lane(cl)) * 16;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          bf16x8 ot[4], qtf[4];
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int o = tb_ + ((2 * s2) * kVGStride + kVGBlock * db) * 16;
            ot[db] = *reinterpret_cast<const bf16x8*>(&tl.ot[o]);
            qtf[db] = *reinterpret_cast<const bf16x8*>(&tl.qt[o]);
          }
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            dv[db] = mfma32(ot[db], pf[s2], dv[db]);
            dk[db] = mfma32(qtf[db], dsf[s2], dk[db]);
          }
        }
      }
      lstore(sm.buf[(it - it_lo + 1) & 1]);
      __syncthreads();
      gload(min(it + 2, it_hi - 1));
    }
  }

  if (!key_ok) return;
  if (n_parts > 1) {
    // float32 partials [part][batch][key][head][d]; key = memory rows, then local rows
    const int kappa = mem ? kappa_row : mem_len + kappa_row;
    const size_t off = ((((size_t)part * batch + b) * n_keys + kappa) * heads_kv + g) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = db * 32 + 8 * qd + 4 * hf;
        const f32x4 wk = {dk[db][4 * qd], dk[db][4 * qd + 1], dk[db][4 * qd + 2], dk[db][4 * qd + 3]};
        const f32x4 wv = {dv[db][4 * qd], dv[db][4 * qd + 1], dv[db][4 * qd + 2], dv[db][4 * qd + 3]};
        *reinterpret_cast<f32x4*>(part_dk + off + d0) = wk;
        *reinterpret_cast<f32x4*>(part_dv + off + d0) = wv;
      }
    return;
  }
  const int rows_len = mem ? mem_len : loc_len;
  const size_t off = (((size_t)b * rows_len + kappa_row) * heads_kv + g) * kD;
  uint16_t* dkrow = (mem ? dk_sel : dk_loc) + off;
  uint16_t* dvrow = (mem ? dv_sel : dv_loc) + off;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = db * 32 + 8 * qd + 4 * hf;
      uint2 wk, wv;
      wk.x = pack_bf16x2(dk[db][4 * qd] * scale, dk[db][4 * qd + 1] * scale);
      wk.y = pack_bf16x2(dk[db][4 * qd + 2] * scale, dk[db][4 * qd + 3] * scale);
      wv.x = pack_bf16x2(dv[db][4 * qd], dv[db][4 * qd + 1]);
      wv.y = pack_bf16x2(dv[db][4 * qd + 2], dv[db][4 * qd + 3]);
      *reinterpret_cast<uint2*>(dkrow + d0) = wk;
      *reinterpret_cast<uint2*>(dvrow + d0) = wv;
    }
}

// Sum of the dk/dv partials in part order (deterministic), scaled and
// rounded to bf16; one thread per 8 elements of a key row.
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(
    const float* __restrict__ part_dk, const float* __restrict__ part_dv, int n_parts, int batch,
    int mem_len, int loc_len, int heads_kv, float scale, uint16_t* __restrict__ dk_sel,
    uint16_t* __restrict__ dv_sel, uint16_t* __restrict__ dk_loc, uint16_t* __restrict__ dv_loc) {
  const int n_keys = mem_len + loc_len;
  const int64_t total = (int64_t)batch * n_keys * heads_kv * (kD / 8);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i % (kD / 8));
  int64_t rest = i / (kD / 8);
  const int g = (int)(rest % heads_kv);
  rest /= heads_kv;
  const int kappa = (int)(rest % n_keys);
  const int b = (int)(rest / n_keys);
  const size_t stride = (size_t)batch * n_keys * heads_kv * kD;
  const size_t off = (((size_t)b * n_keys + kappa) * heads_kv + g) * kD + 8 * c;
  float sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(part_dk + p * stride + off);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(part_dk + p * stride + off + 4);
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(part_dv + p * stride + off);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(part_dv + p * stride + off + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk[e] += k0[e];
      sk[4 + e] += k1[e];
      sv[e] += v0[e];
      sv[4 + e] += v1[e];
    }
  }
  u32x4 wk, wv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    wk[e] = pack_bf16x2(sk[2 * e] * scale, sk[2 * e + 1] * scale);
    wv[e] = pack_bf16x2(sv[2 * e], sv[2 * e + 1]);
  }
  const bool mem = kappa < mem_len;
  const int r = mem ? kappa : kappa - mem_len;
  const size_t o = (((size_t)b * (mem ? mem_len : loc_len) + r) * heads_kv + g) * kD + 8 * c;
  *reinterpret_cast<u32x4*>((mem ? dk_sel : dk_loc) + o) = wk;
  *reinterpret_cast<u32x4*>((mem ? dv_sel : dv_loc) + o) = wv;
}

// Query items per dk/dv work unit before the items are split over parts.
constexpr int kItemsPerUnit = 64;
constexpr int kMaxParts = 16;

int dkdv_parts(int q_len, int heads_q, int heads_kv) {
  const int items = (heads_q / heads_kv) * ((q_len + kQT - 1) / kQT);
  return std::min(kMaxParts, std::max(1, (items + kItemsPerUnit - 1) / kItemsPerUnit));
}

// ---------------------------------------------------------------------------
// vector-ALU kernels (any head dim <= 256, float32 or bf16, any group size)
// ---------------------------------------------------------------------------
constexpr int kGThreads = 256;

// One workgroup per (sequence, token, query head): D, then dq over the
// visible keys, 256 keys at a time (dS of the chunk in LDS, then each thread
// accumulates one element of dq).
template <typename T>
__global__ __launch_bounds__(kGThreads) void attn_bwd_generic_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k_sel, const T* __restrict__ v_sel, int mem_len,
    const T* __restrict__ k_loc, const T* __restrict__ v_loc, int loc_len, const T* __restrict__ out,
    const T* __restrict__ d_out, const float* __restrict__ lse, int batch, int q_len, int heads_q,
    int heads_kv, int dim, float scale, T* __restrict__ dq, float* __restrict__ dsum) {
  __shared__ float qs[256], dos[256], ds_buf[kGThreads], red[kGThreads / 64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int h = (int)(row % heads_q);
  const int t = (int)((row / heads_q) % q_len);
  const int b = (int)(row / ((int64_t)heads_q * q_len));
  const int g = h / (heads_q / heads_kv);
  const size_t qoff = (((size_t)b * q_len + t) * heads_q + h) * dim;
  float part = 0.f;
  if (tid < dim) {
    qs[tid] = Elem<T>::to_f32(q[qoff + tid]);
    const float d = Elem<T>::to_f32(d_out[qoff + tid]);
    dos[tid] = d;
    part = d * Elem<T>::to_f32(out[qoff + tid]);
  }
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  const float d_t = red[0] + red[1] + red[2] + red[3];
  const float lse_t = lse[((size_t)b * heads_q + h) * q_len + t];
  if (tid == 0) dsum[((size_t)b * heads_q + h) * q_len + t] = d_t;
  auto key_row = [&](int j, bool value) -> const T* {
    if (j < mem_len) return (value ? v_sel : k_sel) + (((size_t)b * mem_len + j) * heads_kv + g) * dim;
    return (value ? v_loc : k_loc) + (((size_t)b * loc_len + (j - mem_len)) * heads_kv + g) * dim;
  };
  const int n_vis = mem_len + loc_len - q_len + t + 1;
  float acc = 0.f;
  for (int j0 = 0; j0 < n_vis; j0 += kGThreads) {
    const int j = j0 + tid;
    float ds = 0.f;
    if (j < n_vis) {
      const T* kr = key_row(j, false);
      const T* vr = key_row(j, true);
      float sdot = 0.f, pdot = 0.f;
      for (int e = 0; e < dim; ++e) {
        sdot = fmaf(qs[e], Elem<T>::to_f32(kr[e]), sdot);
        pdot = fmaf(dos[e], Elem<T>::to_f32(vr[e]), pdot);
      }
      const float p = expf(sdot * scale - lse_t);
      ds = p * (pdot - d_t);
    }
    ds_buf[tid] = ds;
    __syncthreads();
    if (tid < dim) {
      const int n = min(kGThreads, n_vis - j0);
      for (int jj = 0; jj < n; ++jj) acc = fmaf(ds_buf[jj], Elem<T>::to_f32(key_row(j0 + jj, false)[tid]), acc);
    }
    __syncthreads();
  }
  if (tid < dim) dq[qoff + tid] = Elem<T>::from_f32(acc * scale);
}

// One workgroup per (sequence, KV head, key): the rows (query head of the
// group, token) that see the key, 256 at a time (P and dS of the chunk in
// LDS, then each thread accumulates one element of dk and dv).
template <typename T>
__global__ __launch_bounds__(kGThreads) void attn_bwd_generic_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k_sel, const T* __restrict__ v_sel, int mem_len,
    const T* __restrict__ k_loc, const T* __restrict__ v_loc, int loc_len, const T* __restrict__ d_out,
    const float* __restrict__ lse, const float* __restrict__ dsum, int batch, int q_len, int heads_q,
    int heads_kv, int dim, float scale, T* __restrict__ dk_sel, T* __restrict__ dv_sel,
    T* __restrict__ dk_loc, T* __restrict__ dv_loc) {
  __shared__ float ks[256], vs[256], p_buf[kGThreads], ds_buf[kGThreads];
  __shared__ int row_buf[kGThreads];
  const int tid = threadIdx.x;
  const int n_keys = mem_len + loc_len;
  int64_t id = blockIdx.x;
  const int kappa = (int)(id % n_keys);
  id /= n_keys;
  const int g = (int)(id % heads_kv);
  const int b = (int)(id / heads_kv);
  const bool mem = kappa < mem_len;
  const int r = mem ? kappa : kappa - mem_len;
  const size_t koff = (((size_t)b * (mem ? mem_len : loc_len) + r) * heads_kv + g) * dim;
  if (tid < dim) {
    ks[tid] = Elem<T>::to_f32((mem ? k_sel : k_loc)[koff + tid]);
    vs[tid] = Elem<T>::to_f32((mem ? v_sel : v_loc)[koff + tid]);
  }
  __syncthreads();
  const int group = heads_q / heads_kv;
  const int t_first = mem ? 0 : max(0, r - (loc_len - q_len));
  const int n_t = q_len - t_first;
  const int n_rows = group * n_t;
  float acc_k = 0.f, acc_v = 0.f;
  for (int r0 = 0; r0 < n_rows; r0 += kGThreads) {
    const int rr = r0 + tid;
    float p = 0.f, ds = 0.f;
    int qrow = 0;
    if (rr < n_rows) {
      const int h = g * group + rr / n_t;
      const int t = t_first + rr % n_t;
      qrow = (b * q_len + t) * heads_q + h;
      const T* qr = q + (size_t)qrow * dim;
      const T* orow = d_out + (size_t)qrow * dim;
      float sdot = 0.f, pdot = 0.f;
      for (int e = 0; e < dim; ++e) {
        sdot = fmaf(Elem<T>::to_f32(qr[e]), ks[e], sdot);
        pdot = fmaf(Elem<T>::to_f32(orow[e]), vs[e], pdot);
      }
      const size_t li = ((size_t)b * heads_q + h) * q_len + t;
      p = expf(sdot * scale - lse[li]);
      ds = p * (pdot - dsum[li]);
    }
    p_buf[tid] = p;
    ds_buf[tid] = ds;
    row_buf[tid] = qrow;
    __syncthreads();
    if (tid < dim) {
      const int n = min(kGThreads, n_rows - r0);
      for (int jj = 0; jj < n; ++jj) {
        const size_t o = (size_t)row_buf[jj] * dim + tid;
        acc_v = fmaf(p_buf[jj], Elem<T>::to_f32(d_out[o]), acc_v);
        acc_k = fmaf(ds_buf[jj], Elem<T>::to_f32(q[o]), acc_k);
      }
    }
    __syncthreads();
  }
  if (tid < dim) {
    (mem ? dk_sel : dk_loc)[koff + tid] = Elem<T>::from_f32(acc_k * scale);
    (mem ? dv_sel : dv_loc)[koff + tid] = Elem<T>::from_f32(acc_v);
  }
}

template <typename T>
hipError_t launch_generic_bwd(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                              const void* k_loc, const void* v_loc, int loc_len, const void* out,
                              const void* d_out, const float* lse, int batch, int q_len, int heads_q,
                              int heads_kv, int dim, float scale, void* dq, void* dk_sel, void* dv_sel,
                              void* dk_loc, void* dv_loc, float* dsum, hipStream_t s) {
  const T* qq = static_cast<const T*>(q);
  hipLaunchKernelGGL(attn_bwd_generic_dq_kernel<T>, dim3((unsigned)((int64_t)batch * q_len * heads_q)),
                     dim3(kGThreads), 0, s, qq, static_cast<const T*>(k_sel), static_cast<const T*>(v_sel),
                     mem_len, static_cast<const T*>(k_loc), static_cast<const T*>(v_loc), loc_len,
                     static_cast<const T*>(out), static_cast<const T*>(d_out), lse, batch, q_len, heads_q,
                     heads_kv, dim, scale, static_cast<T*>(dq), dsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_generic_dkdv_kernel<T>,
                     dim3((unsigned)((int64_t)batch * heads_kv * (mem_len + loc_len))), dim3(kGThreads), 0, s,
                     qq, static_cast<const T*>(k_sel), static_cast<const T*>(v_sel), mem_len,
                     static_cast<const T*>(k_loc), static_cast<const T*>(v_loc), loc_len,
                     static_cast<const T*>(d_out), lse, dsum, batch, q_len, heads_q, heads_kv, dim, scale,
                     static_cast<T*>(dk_sel), static_cast<T*>(dv_sel), static_cast<T*>(dk_loc),
                     static_cast<T*>(dv_loc));
  return hipGetLastError();
}

}  // namespace

namespace {
bool bwd_mfma(int heads_q, int heads_kv, int dim, msa_dtype dt) {
  const int group = heads_q / heads_kv;
  return dt == MSA_BF16 && dim == kD && (group % 4 == 0 || group == 2);
}
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

// D per query row, then (MFMA path with more than one part) the float32 dk/dv partials.
size_t attn_backward_workspace_bytes(int batch, int q_len, int heads_q, int heads_kv, int dim, int mem_len,
                                     int loc_len, msa_dtype dt) {
  size_t bytes = align256((size_t)batch * heads_q * q_len * sizeof(float));
  if (bwd_mfma(heads_q, heads_kv, dim, dt)) {
    const int parts = dkdv_parts(q_len, heads_q, heads_kv);
    if (parts > 1)
      bytes += 2 * align256((size_t)parts * batch * (mem_len + loc_len) * heads_kv * kD * sizeof(float));
  }
  return bytes;
}

hipError_t launch_attn_backward(const void* q, const void* k_sel, const void* v_sel, int mem_len,
                                const void* k_loc, const void* v_loc, int loc_len, const void* out,
                                const void* d_out, const float* lse, int batch, int q_len, int heads_q,
                                int heads_kv, int dim, float scale, msa_dtype dt, void* dq, void* dk_sel,
                                void* dv_sel, void* dk_loc, void* dv_loc, void* ws, hipStream_t s) {
  float* dsum = static_cast<float*>(ws);
  const int group = heads_q / heads_kv;
  if (!bwd_mfma(heads_q, heads_kv, dim, dt)) {
    if (dt == MSA_F32)
      return launch_generic_bwd<float>(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, out, d_out, lse,
                                       batch, q_len, heads_q, heads_kv, dim, scale, dq, dk_sel, dv_sel,
                                       dk_loc, dv_loc, dsum, s);
    return launch_generic_bwd<uint16_t>(q, k_sel, v_sel, mem_len, k_loc, v_loc, loc_len, out, d_out, lse,
                                        batch, q_len, heads_q, heads_kv, dim, scale, dq, dk_sel, dv_sel,
                                        dk_loc, dv_loc, dsum, s);
  }
  constexpr int kNWK = 4;
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
    auto set = [&](const void* kern, size_t bytes) {
      if (e == hipSuccess) e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    };
    set(reinterpret_cast<const void*>(attn_bwd_dq_kernel<4>), sizeof(DqSmem));
    set(reinterpret_cast<const void*>(attn_bwd_dq_kernel<2>), sizeof(DqSmem));
    set(reinterpret_cast<const void*>(attn_bwd_dkdv_kernel<kNWK>), sizeof(DkvSmem));
    return e;
  }();
  if (attr != hipSuccess) return attr;
  const float sl2 = scale * kLog2e;
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* ks16 = static_cast<const uint16_t*>(k_sel);
  const auto* vs16 = static_cast<const uint16_t*>(v_sel);
  const auto* kl16 = static_cast<const uint16_t*>(k_loc);
  const auto* vl16 = static_cast<const uint16_t*>(v_loc);
  const auto* do16 = static_cast<const uint16_t*>(d_out);
  const int nw = group % 4 == 0 ? 4 : 2;
  const unsigned dq_grid = (unsigned)(((q_len + 31) / 32) * batch * heads_kv * (group / nw));
  if (nw == 4)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<4>, dim3(dq_grid), dim3(256), sizeof(DqSmem), s, q16, ks16, vs16,
                       mem_len, kl16, vl16, loc_len, static_cast<const uint16_t*>(out), do16, lse, batch, q_len,
                       heads_q, heads_kv, scale, sl2, static_cast<uint16_t*>(dq), dsum);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<2>, dim3(dq_grid), dim3(128), sizeof(DqSmem), s, q16, ks16, vs16,
                       mem_len, kl16, vl16, loc_len, static_cast<const uint16_t*>(out), do16, lse, batch, q_len,
                       heads_q, heads_kv, scale, sl2, static_cast<uint16_t*>(dq), dsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int parts = dkdv_parts(q_len, heads_q, heads_kv);
  float* part_dk = nullptr;
  float* part_dv = nullptr;
  if (parts > 1) {
    char* p = static_cast<char*>(ws) + align256((size_t)batch * heads_q * q_len * sizeof(float));
    const size_t one = align256((size_t)parts * batch * (mem_len + loc_len) * heads_kv * kD * sizeof(float));
    part_dk = reinterpret_cast<float*>(p);
    part_dv = reinterpret_cast<float*>(p + one);
  }
  const int n_kb = (mem_len + 31) / 32 + (loc_len + 31) / 32;
  const unsigned kv_grid = (unsigned)(((n_kb + kNWK - 1) / kNWK) * parts * batch * heads_kv);
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<kNWK>, dim3(kv_grid), dim3(kNWK * 64), sizeof(DkvSmem), s, q16, ks16,
                     vs16, mem_len, kl16, vl16, loc_len, do16, lse, dsum, batch, q_len, heads_q, heads_kv, scale,
                     sl2, parts, static_cast<uint16_t*>(dk_sel), static_cast<uint16_t*>(dv_sel),
                     static_cast<uint16_t*>(dk_loc), static_cast<uint16_t*>(dv_loc), part_dk, part_dv);
  if ((e = hipGetLastError()) != hipSuccess || parts == 1) return e;
  const int64_t total = (int64_t)batch * (mem_len + loc_len) * heads_kv * (kD / 8);
  hipLaunchKernelGGL(attn_bwd_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part_dk,
                     part_dv, parts, batch, mem_len, loc_len, heads_kv, scale, static_cast<uint16_t*>(dk_sel),
                     static_cast<uint16_t*>(dv_sel), static_cast<uint16_t*>(dk_loc), static_cast<uint16_t*>(dv_loc));
  return hipGetLastError();
}

}  // namespace msa
