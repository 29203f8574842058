// Device-side helpers shared by the ISA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "isa_layout.h"

namespace isa {

// A wave-uniform 64-bit value (read from LDS, say) moved to scalar registers.
__device__ __forceinline__ long long uniform64(long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// First element of slice bh = x*H + h of a caller tensor addressed by m
// (bh < 2^16; x by the multiply of RowMap.hmul, no division).
__device__ __forceinline__ long long rm_head(const RowMap& m, long long bh) {
  const unsigned ub = (unsigned)bh, uh = (unsigned)m.H;
  const unsigned x = uh == 1u ? ub : __umulhi(ub, m.hmul);
  return (long long)x * m.sb + (long long)(ub - x * uh) * m.sh;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;  // LDS operand of ds_read_b64_tr_b16
typedef __attribute__((address_space(3))) char lds_char;
typedef uint16_t bf16_t;  // bfloat16 storage in global memory

// ---------------------------------------------------------------------------
// element conversions

__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t to_bf16(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(bf16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)to_bf16(lo) | ((uint32_t)to_bf16(hi) << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return to_bf16(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ---------------------------------------------------------------------------
// MFMA operand types: 8 contraction elements per lane.
//
// For a 32x32 output tile, lane l holds A[row l%32][k 8*(l/32)+0..7] and
// B[k 8*(l/32)+0..7][col l%32]; the accumulator reg r of lane l is
// D[row 8*(r/4) + 4*(l/32) + r%4][col l%32].  bf16 uses one
// v_mfma_f32_32x32x16_bf16; f32 uses eight v_mfma_f32_32x32x2_f32, the j-th
// contracting element j of both halves, so both types share one register
// layout.

template <typename T> struct Operand;
template <> struct Operand<bf16_t> { typedef bf16x8 type; };
template <> struct Operand<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x16 mma32(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// 8 probabilities -> B operand of the P.V product.
__device__ __forceinline__ void make_operand(const float* p, bf16x8& out) {
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = (__bf16)p[j];
}
__device__ __forceinline__ void make_operand(const float* p, f32x8& out) {
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = p[j];
}

// ---------------------------------------------------------------------------
// 16-byte LDS chunk swizzle.  A tile row of `cpr` 16-byte chunks stores
// logical chunk c at physical chunk c ^ f(row): sixteen consecutive rows
// read at one logical chunk hit sixteen distinct bank groups.
__device__ __forceinline__ int swz(int c, int row, int cpr) {
  return cpr >= 16 ? (c ^ (row & 15)) : (c ^ (((row >> 1) ^ (row >> 4)) & 7));
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (global_load_lds): each lane's bytes land at
// the wave's LDS base (m0) + size x lane.  The compiler does not see them:
// callers wait by count (s_waitcnt vmcnt) and keep LDS reads of the target
// apart with barriers.  m0 is restored, so no register changes behind the
// compiler's back.

// 16 bytes per lane from base + voff into LDS at lds + 16 x lane.
__device__ __forceinline__ void dma16(unsigned lds, const void* base, unsigned voff) {
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

// 4 bytes per lane from base + voff into LDS at lds + 4 x lane.
__device__ __forceinline__ void dma4(unsigned lds, const void* base, unsigned voff) {
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

// Swizzle of the 256-byte LDS rows of the ping-pong kernels: 16-byte chunk
// c of row r sits at chunk c ^ lds_swz(r).
__device__ __forceinline__ int lds_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// The same for 128-byte rows (d = 64), two rows to the 64 banks: chunk c of
// row r sits at chunk c ^ lds_swz64(r).  Over 16 consecutive rows the rows of
// one parity take 8 distinct values (the K operand reads: 16 rows at one
// chunk on 16 distinct 16-byte bank groups), and rows r, r + 2 of a 4-row
// group differ above bit 0 (the V^T transpose reads: 4 rows at a chunk pair).
__device__ __forceinline__ int lds_swz64(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }

// Two direct loads of 16 bytes per lane from base + v0 / v1 into LDS at
// l0 / l1 + 16 x lane, in one asm block; waited for by count.
__device__ __forceinline__ void dma16x2(unsigned l0, unsigned l1, const void* base, unsigned v0, unsigned v1) {
  unsigned saved;  // m0 is restored, so the asm leaves no register changed behind the compiler's back
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %5\n\t"
      "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(l0), "s"(l1), "v"(v0), "v"(v1), "s"(base)
      : "memory");
}

// The direct loads of one step of a gathered-key ping-pong loop in one asm
// block (m0 saved once): two 4-row halves of a wave's K rows into lk and
// lk + 1024, the same of its V rows into lv and lv + 1024 (row r, the lane's
// 16-byte chunk at byte c0 / c1 of the row, rows rs bytes apart in K and V:
// address r * rs + c, a 24-bit multiply-add), then 4 bytes per lane of the
// key-row table from tb + toff into lt + 4 x lane.  Each row address is formed between the m0 write and
// its load, which gives the load the wait state it needs after m0 changes.
// Only s_mov writes scalar registers here (SCC is left alone).
__device__ __forceinline__ void dma_kvt(unsigned lk, unsigned lv, const void* kb, const void* vb, unsigned rs,
                                        unsigned rk0, unsigned rk1, unsigned rv0, unsigned rv1, unsigned c0,
                                        unsigned c1, unsigned lt, const void* tb, unsigned toff) {
  unsigned saved, t0, t1, t2, t3;
  const unsigned lk1 = lk + 1024u, lv1 = lv + 1024u;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lk]\n\t"
      "v_mad_u32_u24 %[t0], %[rk0], %[rs], %[c0]\n\t"
      "global_load_lds_dwordx4 %[t0], %[kb]\n\t"
      "s_mov_b32 m0, %[lk1]\n\t"
      "v_mad_u32_u24 %[t1], %[rk1], %[rs], %[c1]\n\t"
      "global_load_lds_dwordx4 %[t1], %[kb]\n\t"
      "s_mov_b32 m0, %[lv]\n\t"
      "v_mad_u32_u24 %[t2], %[rv0], %[rs], %[c0]\n\t"
      "global_load_lds_dwordx4 %[t2], %[vb]\n\t"
      "s_mov_b32 m0, %[lv1]\n\t"
      "v_mad_u32_u24 %[t3], %[rv1], %[rs], %[c1]\n\t"
      "global_load_lds_dwordx4 %[t3], %[vb]\n\t"
      "s_mov_b32 m0, %[lt]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %[toff], %[tb]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
      : [lk] "s"(lk), [lk1] "s"(lk1), [lv] "s"(lv), [lv1] "s"(lv1), [kb] "s"(kb), [vb] "s"(vb), [rs] "s"(rs),
        [rk0] "v"(rk0), [rk1] "v"(rk1), [rv0] "v"(rv0),
        [rv1] "v"(rv1), [c0] "v"(c0), [c1] "v"(c1), [lt] "s"(lt), [tb] "s"(tb), [toff] "v"(toff)
      : "memory");
}

// Issue order of a fused X phase (NPV P.V MFMAs with two operand reads each,
// then NQK K.Q^T MFMAs with one): the reads of MFMAs 0..LA-1, then each MFMA
// followed by the reads of the MFMA LA places later.
template <int LA, int NPV = 16, int NQK = 16, int M = 0>
__device__ __forceinline__ void pp_issue_order() {
  constexpr int kMFMA = 0x8, kDSR = 0x100;
  if constexpr (M == 0) __builtin_amdgcn_sched_group_barrier(kDSR, LA <= NPV ? 2 * LA : NPV + LA, 0);
  __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
  if constexpr (M + LA < NPV + NQK) __builtin_amdgcn_sched_group_barrier(kDSR, M + LA < NPV ? 2 : 1, 0);
  if constexpr (M + 1 < NPV + NQK) pp_issue_order<LA, NPV, NQK, M + 1>();
}

// ---------------------------------------------------------------------------
// Workgroup id remap so that consecutive logical workgroups (which share a
// head's keys) land on the same XCD: the hardware deals workgroups to the
// 8 XCDs round-robin.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = bid & 7, s = bid >> 3;
  return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

__device__ __forceinline__ float wave_shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Source row of virtual row v of a route whose query blocks are list[0..k)
// (ascending): row list[v / b] * b + v % b, or -1 past the end of the list,
// past the end of a short last block, or for an out-of-range block entry.
__device__ __forceinline__ int route_row(const int* list, int k, int b, int nb, int Ns, long long v) {
  if (v < 0 || v >= (long long)k * b) return -1;
  const unsigned vv = (unsigned)v, ub = (unsigned)b;
  const unsigned i = vv / ub;
  const int blk = list[i];
  const int row = blk * b + (int)(vv - i * ub);
  return (blk >= 0 && blk < nb && row < Ns) ? row : -1;
}

}  // namespace isa
