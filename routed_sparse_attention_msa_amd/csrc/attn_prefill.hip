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
// chosen so that holds, and V is staged in LDS already in V^T operand order
// (one 16-byte unit = the 8 keys one lane contributes to one MFMA, at one d),
// so each V^T operand is a single 16-byte LDS read.  K rows sit at a padded
// pitch that keeps the operand reads free of bank conflicts; every operand
// read is a per-lane base plus a constant offset.  Each MFMA group's operand
// reads are issued before the group
// (one LDS latency per group, not per MFMA).  K and V rows are fetched with
// buffer loads: a per-lane byte offset fixed for the whole kernel plus a
// per-tile scalar offset and a scalar choice of the memory or local rows'
// resource, so the loads carry no address arithmetic and no branches.  The
// softmax scale is folded into one FMA before exp2, and probabilities are
// packed to bf16 by the hardware converter.
//
// Work split: one workgroup = (sequence, KV head, a pair of 32-token blocks
// taken one after the other: the block with the longest causal rows and its
// mirror with the shortest, so every workgroup has about the same number of
// key tiles).  Its waves
// are the query heads of that KV group (GQA packing: each K/V tile is staged
// once for all of them) times two key halves: one wave set takes the even
// 64-key tiles, the other the odd ones, each with its own double-buffered
// LDS tiles, and the two partial softmax states merge through LDS at the end.
// Splitting the keys inside the workgroup halves the longest workgroup's
// critical path, which bounds a causal prefill whose longest block needs
// every key.  Key tiles cover the memory rows, then the local rows (a tile
// never mixes the two); tiles fully below every query's causal limit skip
// the mask, tiles beyond the last query's limit are never loaded.
#include "attn_common.h"

namespace msa {
namespace {

using namespace attn;

constexpr int kKT = 64;                 // keys per LDS tile
constexpr float kLazy = 8.f;  // log2 headroom of the lazy running max

struct PrefillSmem {
  uint8_t k[2][kKT * kKPitch];            // [key][256 B + pad]
  uint8_t v[2][8 * kVGStride * 16];       // [group][d + d/8][8 bf16]
};

template <int NW, int SPLIT>
__global__ __launch_bounds__(NW * 64 * SPLIT, SPLIT == 1 && NW == 4 ? 2 : 1) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_sel,
    const uint16_t* __restrict__ v_sel, int mem_len, const uint16_t* __restrict__ k_loc,
    const uint16_t* __restrict__ v_loc, int loc_len, int batch, int q_len, int heads_q, int heads_kv,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int kThreads = NW * 64;       // threads of one key half
  extern __shared__ __align__(16) uint8_t smem_raw[];

  // wave index made provably uniform so tile offsets stay in scalar registers
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave_all / NW;         // key half (SPLIT = 2): tiles part, part + 2, ...
  const int wave = wave_all - part * NW;  // query head within the workgroup
  PrefillSmem& sm = reinterpret_cast<PrefillSmem*>(smem_raw)[part];
  const int tid = threadIdx.x - part * kThreads;
  const int lane = tid & 63;
  const int cl = lane & 31, hf = lane >> 5;
  const int group = heads_q / heads_kv;
  const int hsub = group / NW;                  // head sub-groups per KV head
  const int n_tblk = (q_len + 31) / 32;

  // blockIdx -> (token block, sequence, kv head, head sub-group)
  int bid = blockIdx.x;
  const int hs = bid % hsub;
  bid /= hsub;
  const int g = bid % heads_kv;
  bid /= heads_kv;
  const int b = bid % batch;
  const int pair = bid / batch;
  const int h = g * group + hs * NW + wave;
  // A workgroup takes the token block n_tblk-1-pair (the longest causal rows)
  // and then its mirror block `pair` (the shortest), so every workgroup has
  // about the same number of key tiles and one round of workgroups finishes
  // together.
  for (int pass = 0; pass < 2; ++pass) {
  const int tb = pass == 0 ? n_tblk - 1 - pair : pair;
  if (pass == 1) {
    if (tb == n_tblk - 1 - pair) break;         // odd block count: the middle block is alone
    __syncthreads();                            // the first block's merge reads are done
  }
  const int t0 = tb * 32;
  const int t = t0 + cl;                        // this lane's query token
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

  // Key tiles: first the memory rows (always visible), then the local rows
  // the block needs; each tile reads rows of one kind only.  Key index kappa
  // counts [memory rows ; local rows]; token t sees local kappa < causal0 + t + 1.
  const int causal0 = mem_len + loc_len - q_len;
  const int n_mt = (mem_len + kKT - 1) / kKT;
  const int loc_need = loc_len - q_len + min(t0 + 32, q_len);
  const int n_tiles = n_mt + (loc_need + kKT - 1) / kKT;
  const int full_below = causal0 + t0 + 1;                 // local keys < this are visible to all
  auto tile_mem = [&](int tile) { return tile < n_mt; };
  auto tile_row0 = [&](int tile) { return tile < n_mt ? tile * kKT : (tile - n_mt) * kKT; };
  auto tile_kappa0 = [&](int tile) { return tile < n_mt ? tile * kKT : mem_len + (tile - n_mt) * kKT; };

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

  // Staging assignments (fixed for the kernel).
  //  K: chunk c = tid + kThreads*i -> key row c/16 = tid/16 + (kThreads/16)*i, 16 B segment
  //     tid%16 (coalesced rows); one lane byte offset, the row term goes to the scalar offset.
  //  V: task  c = tid + kThreads*i -> group c/32, half (c/16)%2, d-block c%16: four key rows
  //     of 8 d each, rewritten as 8 half-units (4 keys at one d) of that group.
  constexpr int kKChunks = kKT * 16 / kThreads;
  constexpr int kKRowStep = kThreads / 16;
  constexpr int kVTasks = 256 / kThreads;
  const uint32_t goff = (uint32_t)g * kD * 2;
  const int krow0 = tid >> 4;
  const uint32_t k_in_row = goff + (tid & 15) * 16;
  const uint32_t kvoff = (uint32_t)krow0 * rs + k_in_row;
  const uint32_t v_in_row = goff + (tid & 15) * 16;   // d-block = c % 16 = tid % 16
  u32x4 pk[kKChunks], pv[kVTasks][4];
  // Branch-free: rows past the block's needs are loaded too (they exist or
  // read as zeros) and masked; a load per branch would leave the compiler
  // unable to count the loads in flight and make it wait for all of them.
  auto gload = [&](int tile) {
    const bool mem = tile_mem(tile);
    const int row0 = tile_row0(tile);
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) pk[i] = kr.load(mem, row0 + kKRowStep * i, kvoff);
#pragma unroll
    for (int i = 0; i < kVTasks; ++i) {
      const uint32_t voff = (uint32_t)vtask_row0(tid + kThreads * i) * rs + v_in_row;
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[i][j] = vr.load(mem, row0 + j, voff);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKChunks; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(&sm.k[buf][(c >> 4) * kKPitch + (c & 15) * 16]) = pk[i];
    }
#pragma unroll
    for (int i = 0; i < kVTasks; ++i) {
      const int c = tid + kThreads * i;
      const int grp = c >> 5, half = (c >> 4) & 1, dblk = c & 15;
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // d = 8*dblk + 2e and + 2e + 1
        uint2 lo, hi;
        lo.x = perm_lo(pv[i][0][e], pv[i][1][e]);
        lo.y = perm_lo(pv[i][2][e], pv[i][3][e]);
        hi.x = perm_hi(pv[i][0][e], pv[i][1][e]);
        hi.y = perm_hi(pv[i][2][e], pv[i][3][e]);
        *reinterpret_cast<uint2*>(&sm.v[buf][vunit(grp, 8 * dblk + 2 * e) + 8 * half]) = lo;
        *reinterpret_cast<uint2*>(&sm.v[buf][vunit(grp, 8 * dblk + 2 * e + 1) + 8 * half]) = hi;
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;  // running max of the raw scores and this half's running sum
  const float lazy = kLazy / scale_log2;

  // Loads and stores run unconditionally (clamped to the last tile; spare
  // copies are never read): the wait before the first store then covers the
  // query loads on every path, and the step loop carries one fixed set of
  // loads in flight, so no wait in it has to drain them all.
  gload(min(part, n_tiles - 1));
  lstore(0);
  __syncthreads();
  gload(min(part + SPLIT, n_tiles - 1));

  const int n_steps = (n_tiles + SPLIT - 1) / SPLIT;
  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    const int tile = SPLIT * step + part;
    const int kappa0 = tile_kappa0(tile);
    if (tile < n_tiles) {
    // S^T for the tile's two 32-key blocks; lane (key cl, half hf) reads
    // segments 8*(st/4) + 4*hf + st%4 of its key row
    const uint8_t* kbase = &sm.k[buf][cl * kKPitch + hf * 64];
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kf[8];
#pragma unroll
      for (int st = 0; st < 8; ++st)
        kf[st] = *reinterpret_cast<const bf16x8*>(kbase + kb * 32 * kKPitch + (8 * (st >> 2) + (st & 3)) * 16);
      __builtin_amdgcn_sched_barrier(0);
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) s[kb] = mfma32(kf[st], qf[st], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // mask (only the last memory tile when partial, and local tiles that cross
    // the causal limit), tile max of the raw scores
    const bool mem = tile_mem(tile);
    if (mem ? kappa0 + kKT > mem_len : kappa0 + kKT > full_below) {
      const int lim = mem ? mem_len : causal0 + t + 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kappa0 + kb * 32 + acc_row(i, hf) >= lim) s[kb][i] = -INFINITY;
    }
    // three-input max tree (v_max3) over the 32 scores, two chains, then the
    // other lane half
    float mx[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float a = max3(s[kb][0], s[kb][1], s[kb][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) a = max3(a, s[kb][i], s[kb][i + 1]);
      mx[kb] = a;
    }
    const float m4 = max3(mx[0], mx[1], s[0][15]);
    const float mt = half_swap_max(max3(m4, s[1][15], s[1][15]));
    // Lazy running max: it moves only when a score exceeds it by more than
    // kLazy / scale_log2 (probabilities then stay <= 2^kLazy, harmless in
    // float32), so the O^T rescale below is rare after the first tiles.
    // (While a lane has seen no visible key, m stays -inf: alpha is then 1
    // and the exponent offset 0, so masked scores give 0, never NaN.)
    const float m_new = mt > m + lazy ? mt : m;
    const float alpha = m_new == m ? 1.f : fast_exp2((m - m_new) * scale_log2);
    m = m_new;
    const float off = m_new == -INFINITY ? 0.f : -m_new * scale_log2;
    // probabilities (float32 row sum, two chains), rounded to bf16 for PV
    float lsum2[2] = {-0.f, -0.f};   // (-0 is the additive identity: no add of zero)
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[kb][8 * s2 + 2 * e], scale_log2, off));
          const float p1 = fast_exp2(fmaf(s[kb][8 * s2 + 2 * e + 1], scale_log2, off));
          lsum2[s2] += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[kb][s2] = as_bf16x8(w);
      }
    l = l * alpha + (lsum2[0] + lsum2[1]);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    // O^T += V^T P^T: lane (d, hf) reads its 8 keys of group 4kb + 2s2 + hf at
    // column d = 32db + cl, i.e. unit vunit(grp, d) = lane base + a constant.
    const uint8_t* vbase = &sm.v[buf][(hf * kVGStride + cl + (cl >> 3)) * 16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 vf[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          vf[db] = *reinterpret_cast<const bf16x8*>(vbase + ((4 * kb + 2 * s2) * kVGStride + 36 * db) * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma32(vf[db], pf[kb][s2], o[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lstore(buf ^ 1);
    __syncthreads();
    gload(min(tile + 2 * SPLIT, n_tiles - 1));
  }

  if constexpr (SPLIT == 2) {
  // merge the odd-tile half into the even-tile half (same head, same lane)
  float* mg = reinterpret_cast<float*>(smem_raw) + (size_t)wave * 66 * 64;
  if (part == 1) {
    mg[lane] = m;
    mg[64 + lane] = l;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) mg[(2 + db * 16 + i) * 64 + lane] = o[db][i];
  }
  __syncthreads();
  if (part == 0) {
    const float m1 = mg[lane], l1 = mg[64 + lane];
    const float mm = fmaxf(m, m1);
    const float a0 = fast_exp2((m - mm) * scale_log2);
    const float a1 = fast_exp2((m1 - mm) * scale_log2);
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = o[db][i] * a0 + mg[(2 + db * 16 + i) * 64 + lane] * a1;
    m = mm;
  }
  }


  const float l_tot = half_swap_sum(l);
  if (part == 0 && t_ok) {
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
  if (lse != nullptr && hf == 0)
    lse[((size_t)b * heads_q + h) * q_len + t] = (m * scale_log2 + __log2f(l_tot)) * kLn2;
  }
  }  // pass
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
  const unsigned grid = (unsigned)((n_tblk + 1) / 2 * batch * heads_kv * (group / nw));
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
    auto set = [&](auto kern, size_t bytes) {
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    };
    set(attn_prefill_kernel<4, 1>, sizeof(PrefillSmem));
    set(attn_prefill_kernel<2, 1>, sizeof(PrefillSmem));
    set(attn_prefill_kernel<1, 1>, sizeof(PrefillSmem));
    set(attn_prefill_kernel<4, 2>, 2 * sizeof(PrefillSmem));
    set(attn_prefill_kernel<2, 2>, 2 * sizeof(PrefillSmem));
    set(attn_prefill_kernel<1, 2>, 2 * sizeof(PrefillSmem));
    return e;
  }();
  if (attr != hipSuccess) return attr;
  // Split each workgroup's keys over two wave sets when the grid is at most
  // one round of workgroups (each then runs on a CU of its own); with more
  // rounds, two unsplit workgroups share a CU.
  const bool split = (int)grid <= 2 * device_cu_count();
  const float sl2 = scale * kLog2e;
  auto go = [&](auto kern, int threads, size_t smem) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), smem, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k_sel), static_cast<const uint16_t*>(v_sel),
                       mem_len, static_cast<const uint16_t*>(k_loc),
                       static_cast<const uint16_t*>(v_loc), loc_len, batch, q_len, heads_q, heads_kv,
                       sl2, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
  };
  const size_t one = sizeof(PrefillSmem);
  if (split) {
    if (nw == 4) return go(attn_prefill_kernel<4, 2>, 512, 2 * one);
    if (nw == 2) return go(attn_prefill_kernel<2, 2>, 256, 2 * one);
    return go(attn_prefill_kernel<1, 2>, 128, 2 * one);
  }
  if (nw == 4) return go(attn_prefill_kernel<4, 1>, 256, one);
  if (nw == 2) return go(attn_prefill_kernel<2, 1>, 128, one);
  return go(attn_prefill_kernel<1, 1>, 64, one);
}

}  // namespace msa
