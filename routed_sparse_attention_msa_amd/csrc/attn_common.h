// Shared pieces of the bf16 MFMA attention kernels (forward and backward):
// the 32x32x16 MFMA, the accumulator row map, the LDS layouts of K rows and
// of transposed operand groups, bf16 packing and buffer-resource loads.
#pragma once

#include "internal.h"

namespace msa {
namespace attn {

constexpr int kD = 128;                 // head dim of the MFMA kernels
constexpr int kVGStride = 136;          // 16 B units per operand-group row: 128 d + one pad unit per 16
constexpr int kKPitch = 272;            // bytes per row in LDS: 256 + 16 pad (conflict-free reads)
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
// Row of accumulator element i held by lane half hf (the column is the lane % 32).
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }
// Transposed operand groups: group G = 4*kb + 2*s2 + hf holds rows
// 32kb + 16s2 + 4hf + {0..3, 8..11} of a tile, one 16-byte unit (8 rows at
// one d) per d, so that a lane's 8 contraction values of one MFMA are one read.
// One pad unit follows every 16 d.  A b128 read is served 16 lanes at a time
// from a 256 B (16-unit) bank line: the 16 lanes of a phase read 16
// consecutive d of one group, which land on 16 distinct units.  The staging
// stores (d = 8*dblk + 2e for dblk 0..15) land on units 8*(dblk % 2) + dblk/2
// + 2e: distinct too.  (A pad per 8 d put d = 0 and d = 15 on one unit.)
__device__ __forceinline__ int vunit(int grp, int d) { return (grp * kVGStride + d + (d >> 4)) * 16; }
// Unit offset, within its group, of column d = 32*db + cl: the lane's base
// vg_lane(cl) plus the constant kVGBlock * db.
__device__ __forceinline__ int vg_lane(int cl) { return cl + (cl >> 4); }
constexpr int kVGBlock = 34;
// First row of transposed-staging task c (4 rows, one 8-d block).
__device__ __forceinline__ int vtask_row0(int c) {
  const int grp = c >> 5, half = (c >> 4) & 1;
  return 32 * (grp >> 2) + 16 * ((grp >> 1) & 1) + 4 * (grp & 1) + 8 * half;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// max of three scores in one instruction.  Written out because the library
// max would first quiet each MFMA result (one extra instruction per input);
// the scores are finite or -inf, never NaN.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Reductions across the two 32-lane halves of a wave without LDS: the lane
// swap leaves (low half, high half) of x in the two results at every lane.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Store four rows (one 8-d block each: r[0..3]) of a tile into the transposed
// operand groups: unit (grp, d) gets rows {4 of them} as 8-byte halves.
__device__ __forceinline__ void store_transposed(uint8_t* base, int grp, int half, int dblk, const u32x4 (&r)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {   // d = 8*dblk + 2e and 2e + 1
    uint2 lo, hi;
    lo.x = perm_lo(r[0][e], r[1][e]);
    lo.y = perm_lo(r[2][e], r[3][e]);
    hi.x = perm_hi(r[0][e], r[1][e]);
    hi.y = perm_hi(r[2][e], r[3][e]);
    *reinterpret_cast<uint2*>(base + vunit(grp, 8 * dblk + 2 * e) + 8 * half) = lo;
    *reinterpret_cast<uint2*>(base + vunit(grp, 8 * dblk + 2 * e + 1) + 8 * half) = hi;
  }
}

// Memory rows and local rows of one (sequence, KV head), each behind a buffer
// resource based at the sequence's first row and sized to its rows: a row
// past the end reads as zeros.
struct KVRows {
  __amdgpu_buffer_rsrc_t sel, loc;
  uint32_t rs;                       // row stride in bytes (heads_kv * 256)
  // 16 bytes at byte voff of row `row0` of the memory (mem) or local rows; the
  // choice is uniform, so it is a scalar select and the load has no branch.
  __device__ __forceinline__ u32x4 load(bool mem, int row0, uint32_t voff) const {
    return bload(mem ? sel : loc, voff, (uint32_t)row0 * rs);
  }
};

}  // namespace attn
}  // namespace msa
