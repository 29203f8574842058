// Device helpers of the stream-K split of the full route, shared by the
// bf16 and FP8 flash kernels.  A is the kernel's argument struct; it carries
// sk_U, sk_G, sk_P, sk_T, sk_R0, sk_K, sk_grid, sk_q, sk_x (the split, as the
// host launcher sets it from the layout) and row_tiles.
#pragma once

#include "isa_device.h"
#include "isa_layout.h"

namespace isa {

// Stream-K split of the full route (Osama et al., "Stream-K: Work-centric
// Parallel Decomposition for Dense Matrix-Matrix Multiplication on the GPU",
// its data-parallel + stream-K hybrid, applied to the key tiles of the
// route's row tiles): whole row tiles in rounds of one per workgroup, so
// that the workgroups of an XCD sweep one head's keys together, then the
// units of the remaining row tiles in equal ranges, range g covering units
// [sk_bound(g), sk_bound(g + 1)).  A row tile inside one range is finished
// by that range's workgroup; one that meets several ranges is cut into
// parts there, part p taken by range sk_range_of(first unit) + p, and
// merged.  A cut row tile's key tiles are taken in rotated order, from the
// first range boundary inside it: unit t of the row tile is key tile
// (t - delta) mod T, delta the boundary's offset (0 when a range starts at
// the row tile).  The range that starts there then reads key tile 0 first,
// as the whole row tiles of its neighbours on the XCD do, so that ranges
// with the same offset read the same K/V tiles at about the same time.
// Every part still covers consecutive key tiles, and the last (padding)
// tiles come at the end of a part.
template <class A>
__device__ __forceinline__ long long sk_bound(const A& a, long long g) { return g * a.sk_U / a.sk_G; }
// the range holding unit u: the largest g with sk_bound(g) <= u
template <class A>
__device__ __forceinline__ int sk_range_of(const A& a, long long u) {
  return (int)(((u + 1) * a.sk_G + a.sk_U - 1) / a.sk_U - 1);
}
// Which row tile a work item takes.  The row tiles are cut into eight
// consecutive blocks, one per XCD (block x: sk_q + (x < sk_x) row tiles from
// x sk_q + min(x, sk_x)); the sk_grid / 8 workgroups of XCD x take the first
// sk_K * sk_grid / 8 of its block whole, in rounds, and the ranges of that
// XCD's workgroups the rest, so that an XCD's work stays on a few heads.
// Whole-round item: round r of logical workgroup g (XCD g / (sk_grid / 8)).
template <class A>
__device__ __forceinline__ int sk_round_row(const A& a, int r, int g) {
  const int per = a.sk_grid >> 3, x = g / per;
  return x * a.sk_q + min(x, a.sk_x) + r * per + (g - x * per);
}
// Range phase: row tile s of the sequence that the ranges cut (the blocks'
// remainders, in block order).
template <class A>
__device__ __forceinline__ int sk_rest_row(const A& a, int s) {
  const int per = a.sk_grid >> 3, qq = a.sk_q - a.sk_K * per;   // a block's remainder: qq or qq + 1
  const int x = s < a.sk_x * (qq + 1) ? s / (qq + 1) : a.sk_x + (s - a.sk_x * (qq + 1)) / max(qq, 1);
  return s + (x + 1) * a.sk_K * per;
}
// The work of stream-K workgroup g (logical id) of a grid of G: kdp whole
// row tiles (round r: sk_round_row(r, g)), then the nsk row tiles that its
// range [u0, u1) meets, key tiles t00 .. of range-phase row tile R0 through
// row tile R0 + nsk - 1 (t1l key tiles of the last).  part0: the part of row
// tile R0 that the range takes when that row tile starts in an earlier
// range (later items start in this one: part 0 or whole); tb0: its first
// key tile in rotated order.  (64-bit quotients come out in vector
// registers: made scalar again.)
struct SkItems { int g, kdp, nsk, R0, t00, t1l, part0, tb0; };
template <class A>
__device__ __forceinline__ SkItems sk_items(const A& a, int g) {
  SkItems s;
  s.g = g;
  s.kdp = a.sk_K;
  const int T = a.sk_T;
  long long u0 = 0, u1 = 0;
  if (g < a.sk_G) {
    u0 = sk_bound(a, g);
    u1 = sk_bound(a, g + 1);
  }
  s.R0 = __builtin_amdgcn_readfirstlane((int)(u0 / T));
  s.nsk = __builtin_amdgcn_readfirstlane(u1 > u0 ? (int)((u1 - 1) / T) - s.R0 + 1 : 0);
  s.t00 = __builtin_amdgcn_readfirstlane((int)(u0 - (long long)s.R0 * T));
  s.t1l = __builtin_amdgcn_readfirstlane((int)(u1 - (long long)(s.R0 + s.nsk - 1) * T));
  s.part0 = __builtin_amdgcn_readfirstlane(s.t00 > 0 ? g - sk_range_of(a, (long long)s.R0 * T) : 0);
  // key tiles of a cut row tile run from its first inner range boundary,
  // delta units in: t -> t - delta mod T
  int tb0 = s.t00;
  if (s.t00 > 0) {
    const long long base = (long long)s.R0 * T;
    if (sk_bound(a, g - s.part0) != base) tb0 = s.t00 - (int)(sk_bound(a, g - s.part0 + 1) - base);
  }
  s.tb0 = __builtin_amdgcn_readfirstlane(tb0);
  return s;
}
// Item r of those: row tile (bh, rt); part < 0 for the whole row tile, else
// 8 Rs + p for part p of range-phase row tile Rs (its partial buffer slot);
// t_begin: its first key tile in rotated order, the nt key tiles following
// it without wrapping.
struct SkItem { int bh, rt, part, t_begin, nt; };
template <class A>
__device__ __forceinline__ SkItem sk_item(const A& a, const SkItems& s, int r) {
  const int T = a.sk_T;
  int Ri, t0 = 0, t1 = T, tb = 0, part = -1;
  if (r < s.kdp) {
    Ri = sk_round_row(a, r, s.g);
  } else {
    const int q = r - s.kdp;
    Ri = sk_rest_row(a, s.R0 + q);
    if (q == 0) t0 = s.t00;
    if (q == s.nsk - 1) t1 = s.t1l;
    if (t0 > 0 || t1 < T) part = 8 * (s.R0 + q) + (q == 0 ? s.part0 : 0);
    // a later item starts at its row tile's first unit, inside this range:
    // the boundary is this range's end, t1 units in
    tb = q == 0 ? s.tb0 : (t1 < T ? T - t1 : 0);
  }
  const int bh = Ri / a.row_tiles;
  return SkItem{bh, Ri - bh * a.row_tiles, part, tb, t1 - t0};
}

}  // namespace isa
