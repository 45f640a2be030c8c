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
  uint8_t v[2][8 * kVGStride * 16];       // [group][d + d/16][8 bf16]
};

template <int NW, int SPLIT>
__global__ __launch_bounds__(NW * 64 * SPLIT) void attn_prefill_kernel(
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
    const uint8_t* vbase = &sm.v[buf][(hf * kVGStride + vg_lane(cl)) * 16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 vf[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          vf[db] = *reinterpret_cast<const bf16x8*>(vbase + ((4 * kb + 2 * s2) * kVGStride + kVGBlock * db) * 16);
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


// ---------------------------------------------------------------------------
// Ping-pong variant, for groups of 4 query heads per KV head (the GQA shapes
// of the routed layers; the kernel above serves groups of 1 and 2).  Same
// work split, orientation and online softmax as above, always with two key
// halves; what changes is how the two halves share a SIMD and how tiles reach
// LDS.
//
// The waves of the two key halves that share a SIMD (the same query head) run
// half a step apart: the workgroup's barriers cut time into slots, and in each
// slot one half issues its MFMAs (P V of its previous tile, then S of its
// current one) while the other half runs the softmax of the S it produced in
// the slot before.  The matrix core then works while the other wave's vector
// instructions issue, instead of both waves computing the same phase at the
// same time.
//
// Tiles go from memory straight into LDS (buffer loads with the LDS flag: 16 B
// per lane, a wave instruction fills 1 KiB), so staging costs neither
// registers nor LDS store instructions.  Rows are 256 B, unpadded; the 16-byte
// slots of a row are permuted by XOR (K: slot ^ row % 16, so the 16 lanes of a
// K operand read that take rows 0..15 hit distinct banks; V: a permutation
// chosen for the transposing reads below) and each lane loads the global slot
// that belongs at its LDS position.  The V^T operand of P V is read with the
// transposing LDS read ds_read_b64_tr_b16: within 16 lanes it hands lane j the
// 4 values at column j of 4 consecutive rows, so two reads give a lane the 8
// keys it contributes at its d.  K tiles are triple-buffered, V tiles double:
// a tile's loads are issued two slots before its MFMAs need it.
constexpr int kTileBytes = kKT * 256;
constexpr int kPPKBufs = 3, kPPVBufs = 2;
struct PingPongSmem {
  uint8_t k[kPPKBufs][kTileBytes];
  uint8_t v[kPPVBufs][kTileBytes];
};
constexpr int kPPLoads = 8;              // DMA instructions a wave issues per tile (4 K + 4 V)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int v_swizzle(int r3) { return (4 * r3) ^ (2 * ((r3 >> 1) & 1)); }   // r3 = row % 4
// Buffer descriptor as four scalars: base, stride 0, size in bytes (loads past
// it read zeros), the same flags as the other buffer loads.
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, kRsrcWord3};
}
// 16 bytes per lane from memory into LDS at lds_addr + 16 * lane.  Issued from
// asm: the compiler does not see these loads, so it neither drains them before
// the next LDS read (it cannot tell they write other buffers) nor counts them;
// the kernel's own waits (slot_barrier) order them.  The asm has no outputs.
// M0 is a reserved register, so the compiler warns that the clobber may be
// ignored; this kernel uses M0 for nothing else (its generated code writes M0
// only right before each of these loads).
__device__ __forceinline__ void dma16(const u32x4& r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}
// Barrier that first waits until at most VM of this wave's loads are in flight
// (the newer DMA stays in flight) and its LDS reads have returned.  Written
// out because __syncthreads' fence waits for every load.  The scheduling
// fences keep every instruction in its slot: MFMAs and VALU work touch no
// memory, so the clobber alone would let the compiler move them across.
template <int VM>
__device__ __forceinline__ void slot_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(512, 1) void attn_prefill_pp_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_sel,
    const uint16_t* __restrict__ v_sel, int mem_len, const uint16_t* __restrict__ k_loc,
    const uint16_t* __restrict__ v_loc, int loc_len, int batch, int q_len, int heads_q, int heads_kv,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NW = 4;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave_all / NW;         // key half: tiles part, part + 2, ...
  const int wave = wave_all - part * NW;  // query head within the workgroup
  PingPongSmem& sm = reinterpret_cast<PingPongSmem*>(smem_raw)[part];
  const int lane = threadIdx.x & 63;
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
  const int pair = bid / batch;
  const int h = g * group + hs * NW + wave;

  // A tile that runs past the end of the memory or local rows reads rows a
  // load past the end leaves unwritten; they must hold finite values (P is 0
  // there, but 0 * NaN would not be), so zero every buffer once.  With whole
  // tiles only (the usual shapes) no such row is ever read.
  if (mem_len % kKT != 0 || loc_len % kKT != 0) {
    for (int i = threadIdx.x; i < (int)(2 * sizeof(PingPongSmem) / 16); i += 512)
      reinterpret_cast<u32x4*>(smem_raw)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }

  const uint32_t rs = (uint32_t)heads_kv * kD * 2;
  const uint32_t goff = (uint32_t)g * kD * 2;
  const size_t sel_rows = (size_t)b * mem_len * heads_kv * kD;
  const size_t loc_rows = (size_t)b * loc_len * heads_kv * kD;
  const uint32_t sel_bytes = (uint32_t)((size_t)mem_len * rs);
  const uint32_t loc_bytes = (uint32_t)((size_t)loc_len * rs);
  const u32x4 k_mem = dma_rsrc(k_sel + (mem_len ? sel_rows : 0), sel_bytes);
  const u32x4 k_lc = dma_rsrc(k_loc + loc_rows, loc_bytes);
  const u32x4 v_mem = dma_rsrc(v_sel + (mem_len ? sel_rows : 0), sel_bytes);
  const u32x4 v_lc = dma_rsrc(v_loc + loc_rows, loc_bytes);

  // DMA lane offsets.  Wave instruction c (c = 4i + wave) fills LDS rows
  // 4c .. 4c+3; lane l writes row 4c + l/16 at physical slot l % 16, so it
  // loads the logical slot that the row's XOR maps there.
  const int r4 = lane >> 4;
  const uint32_t dma_k = (uint32_t)r4 * rs + goff + (uint32_t)(((lane & 15) ^ ((4 * wave + r4) & 15)) * 16);
  const uint32_t dma_v = (uint32_t)r4 * rs + goff + (uint32_t)(((lane & 15) ^ v_swizzle(r4)) * 16);
  // Operand read addresses.  Buffers and rows are 256-byte aligned, so a
  // swizzled address is (lane base) XOR (16 * logical slot): one XOR per read.
  // K (S^T = K Q^T): lane (key cl, half hf) at k-step st reads logical slot
  // 8*(st/4) + 4*hf + st%4 of row 32*kb + cl; its base carries the row XOR.
  const uint32_t k_lane = (uint32_t)(cl * 256 + (cl & 15) * 16);
  // V^T (transposing reads): 16-lane group (cl / 16, hf), lane rho in it:
  // row k0 + rho/4, d = 32*db + 16*(cl/16) + 4*(rho%4) .. +3, with
  // k0 = 32kb + 16s2 + 4hf (+8 for the second read); d-block db is XOR 64*db.
  const int rho = lane & 15;
  const uint32_t v_lane = (uint32_t)((4 * hf + (rho >> 2)) * 256 +
                                     (((2 * (cl >> 4) + ((rho >> 1) & 1)) ^ v_swizzle(rho >> 2)) * 16) + (rho & 1) * 8);
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t k_base0 = (uint32_t)(uintptr_t)(lds_u8*)(&sm.k[0][0]);   // LDS byte addresses
  const uint32_t v_base0 = (uint32_t)(uintptr_t)(lds_u8*)(&sm.v[0][0]);

  // Q^T operand of token block tb (lane: query cl, half hf)
  bf16x8 qf[8];
  auto load_q = [&](int tb) {
    const int t = tb * 32 + cl;
    const uint16_t* qrow = q + (((size_t)b * q_len + (t < q_len ? t : 0)) * heads_q + h) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[s] = as_bf16x8(t < q_len ? load16(qrow + 64 * (s >> 2) + 32 * hf + 8 * (s & 3)) : z);
    }
  };
  const bool two_blocks = pair != n_tblk - 1 - pair;   // odd block count: the middle block is alone
  load_q(n_tblk - 1 - pair);

  for (int pass = 0; pass < 2; ++pass) {
  const int tb = pass == 0 ? n_tblk - 1 - pair : pair;
  if (pass == 1) {
    if (!two_blocks) break;
    slot_barrier<63>();                         // the first block's merge reads are done (its stores may still be in flight)
  }
  const int t0 = tb * 32;
  const int t = t0 + cl;
  const bool t_ok = t < q_len;
  const int causal0 = mem_len + loc_len - q_len;
  const int n_mt = (mem_len + kKT - 1) / kKT;
  const int loc_need = loc_len - q_len + min(t0 + 32, q_len);
  const int n_tiles = n_mt + (loc_need + kKT - 1) / kKT;
  const int full_below = causal0 + t0 + 1;
  const int n0 = (n_tiles + 1) / 2, n1 = n_tiles / 2;
  const int n_me = part == 0 ? n0 : n1;

  // the part's j-th tile is tile 2j + part; loads past the last are clamped
  // DMA of wave instruction i (of 4) of the part's tile j into buffer buf
  auto issue_k1 = [&](int j, int buf, int i) {
    const int tile = min(2 * j + part, n_tiles - 1);
    const bool mem = tile < n_mt;
    const uint32_t row0 = (uint32_t)(mem ? tile * kKT : (tile - n_mt) * kKT);
    const int c = 4 * i + wave;
    dma16(mem ? k_mem : k_lc, k_base0 + buf * kTileBytes + c * 1024, dma_k, (row0 + 4 * c) * rs);
  };
  auto issue_v1 = [&](int j, int buf, int i) {
    const int tile = min(2 * j + part, n_tiles - 1);
    const bool mem = tile < n_mt;
    const uint32_t row0 = (uint32_t)(mem ? tile * kKT : (tile - n_mt) * kKT);
    const int c = 4 * i + wave;
    dma16(mem ? v_mem : v_lc, v_base0 + buf * kTileBytes + c * 1024, dma_v, (row0 + 4 * c) * rs);
  };
  auto issue_k = [&](int j, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_k1(j, buf, i);
  };
  auto issue_v = [&](int j, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_v1(j, buf, i);
  };

  // (Q of this block was loaded before: at the start, or after the previous
  // block's loop, so that its latency hides behind that block's merge.)
  issue_k(0, 0);
  issue_v(0, 0);
  issue_k(1, 1);
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float lazy = kLazy / scale_log2;
  f32x16 s[2];
  bf16x8 pf[2][2];

  // MFMA slot: O^T += V^T P^T of the part's tile j, then S^T = K Q^T of the
  // tile in K buffer kbuf.  Software-pipelined: the operand reads of each
  // MFMA group are issued before the MFMAs of the group before it.
  auto mfma_slot = [&](int j, int kbuf, int kj, int kjbuf) {   // and loads K of the part's tile kj
    const uint32_t vb = (v_base0 + (j & 1) * kTileBytes) | v_lane;
    const uint32_t kbase = (k_base0 + kbuf * kTileBytes) | k_lane;
    auto read_v = [&](bf16x8 (&vf)[4], int grp) {     // grp = 2 kb + s2
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t a = (vb ^ (64u * db)) + grp * 16 * 256;
        const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
        const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(a + 8 * 256));
        vf[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto read_k = [&](bf16x8 (&kf)[8], int kb) {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const uint32_t a = (kbase ^ (16u * (8 * (st >> 2) + 4 * hf + (st & 3)))) + kb * 32 * 256;
        kf[st] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>((uintptr_t)a);
      }
    };
    bf16x8 vf[2][4], kf[2][8];
    read_v(vf[0], 0);
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      if (grp < 3) read_v(vf[(grp + 1) & 1], grp + 1);
      else read_k(kf[0], 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = mfma32(vf[grp & 1][db], pf[grp >> 1][grp & 1], o[db]);
      __builtin_amdgcn_sched_barrier(0);
      issue_k1(kj, kjbuf, grp);               // while the group's MFMAs run
      __builtin_amdgcn_sched_barrier(0);
    }
    read_k(kf[1], 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) s[kb] = mfma32(kf[kb][st], qf[st], s[kb]);
    }
  };
  auto qk = [&](int kbuf) {                     // S^T of the tile in K buffer kbuf (first slot)
    const uint32_t kbase = (k_base0 + kbuf * kTileBytes) | k_lane;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kf[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const uint32_t a = (kbase ^ (16u * (8 * (st >> 2) + 4 * hf + (st & 3)))) + kb * 32 * 256;
        kf[st] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>((uintptr_t)a);
      }
      __builtin_amdgcn_sched_barrier(0);
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) s[kb] = mfma32(kf[st], qf[st], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The second half runs one slot behind the first.  Slots: [S of tile 0],
  // then per tile j: [softmax of tile j] [P V of tile j, S of tile j+1].  The
  // last S reads the clamped copy of the last tile and is not used.
  //
  // Loads (per wave, in issue order): K0 V0 K1 before the first slot, K2 in
  // it, then V(j+1) in the softmax slot of tile j and K(j+3) in the MFMA slot
  // after it, each into the buffer last read one slot earlier.  The CU's
  // address unit accepts DMA instructions one at a time, so they are spread
  // out: one per MFMA group (the matrix core keeps running while the wave
  // waits) and one per group of exponentials.  Every tile still lands three
  // slots before its first use, and the wait at the end of a softmax slot
  // leaves exactly the two newest tiles' loads (8) in flight.
  if (part == 1) slot_barrier<kPPLoads + 4>();
  slot_barrier<kPPLoads>();                     // K of tile 0 is in LDS (V0 and K1 may be in flight)
  qk(0);
  issue_k(2, 2);
  slot_barrier<kPPLoads + 4>();                 // (a bound: at most 12 loads are in flight here)
  int kbuf = 0;                                 // K buffer of the part's tile j (j % 3)
  for (int j = 0; j < n_me; ++j) {
    // ---- softmax slot: P of tile j; loads of V(j+1) ----
    // The rare O^T rescale comes before the exponentials, so they stay in
    // this slot's final block.
    const int vb_next = (j + 1) & 1;
    const int tile = 2 * j + part;
    const bool mem = tile < n_mt;
    const int kappa0 = mem ? tile * kKT : mem_len + (tile - n_mt) * kKT;
    if (mem ? kappa0 + kKT > mem_len : kappa0 + kKT > full_below) {
      const int lim = mem ? mem_len : causal0 + t + 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kappa0 + kb * 32 + acc_row(i, hf) >= lim) s[kb][i] = -INFINITY;
    }
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
    const float m_new = mt > m + lazy ? mt : m;
    const float alpha = m_new == m ? 1.f : fast_exp2((m - m_new) * scale_log2);
    m = m_new;
    const float off = m_new == -INFINITY ? 0.f : -m_new * scale_log2;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    l *= alpha;
    __builtin_amdgcn_sched_barrier(0);
    float lsum2[2] = {-0.f, -0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        issue_v1(j + 1, vb_next, 2 * kb + s2);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[kb][8 * s2 + 2 * e], scale_log2, off));
          const float p1 = fast_exp2(fmaf(s[kb][8 * s2 + 2 * e + 1], scale_log2, off));
          lsum2[s2] += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[kb][s2] = as_bf16x8(w);
        __builtin_amdgcn_sched_barrier(0);
      }
    l += lsum2[0] + lsum2[1];
    kbuf = kbuf == 2 ? 0 : kbuf + 1;
    slot_barrier<kPPLoads>();                   // K(j+1) and V(j) have landed
    // ---- MFMA slot, loading K(j+3) into the buffer of tile j ----
    mfma_slot(j, kbuf, j + 3, kbuf == 0 ? 2 : kbuf - 1);
    slot_barrier<kPPLoads + 4>();
  }
  // Every load has landed before LDS is reused; both halves then pass the
  // same number of barriers (part 0: 2 n0 + 2 so far, part 1: 2 n1 + 3).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  {
    const int done = part == 0 ? 2 * n0 + 2 : 2 * n1 + 3;
    const int total = max(2 * n0 + 2, 2 * n1 + 3);
    for (int i = done; i < total; ++i) slot_barrier<63>();
  }
  // One more barrier: a half without padding drained its loads only after
  // its last barrier above, and its clamped tile loads land in the buffers
  // the merge overwrites.
  slot_barrier<63>();
  if (pass == 0 && two_blocks) load_q(pair);    // Q of the second block (qf is dead here)

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
  slot_barrier<63>();
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
    set(attn_prefill_kernel<2, 1>, sizeof(PrefillSmem));
    set(attn_prefill_kernel<1, 1>, sizeof(PrefillSmem));
    set(attn_prefill_kernel<2, 2>, 2 * sizeof(PrefillSmem));
    set(attn_prefill_kernel<1, 2>, 2 * sizeof(PrefillSmem));
    set(attn_prefill_pp_kernel, 2 * sizeof(PingPongSmem));
    return e;
  }();
  if (attr != hipSuccess) return attr;
  // Groups of 4 query heads: the ping-pong kernel (one workgroup per CU, its
  // keys split over two wave sets), whatever the grid.  Groups of 1 or 2:
  // split the keys when the grid is at most one round of workgroups (each
  // then runs on a CU of its own); with more rounds, two unsplit workgroups
  // share a CU.
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
  if (nw == 4) return go(attn_prefill_pp_kernel, 512, 2 * sizeof(PingPongSmem));
  if (split) {
    if (nw == 2) return go(attn_prefill_kernel<2, 2>, 256, 2 * one);
    return go(attn_prefill_kernel<1, 2>, 128, 2 * one);
  }
  if (nw == 2) return go(attn_prefill_kernel<2, 1>, 128, one);
  return go(attn_prefill_kernel<1, 1>, 64, one);
}

}  // namespace msa
