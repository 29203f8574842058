// Host-side plan of one ISA call: argument checks, block counts and the
// carve-up of the caller's workspace.  No HIP types; compiled into the
// library and usable from plain C++.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "isa.h"

namespace isa {

constexpr int kTileKeys = 64;      // keys per attention tile
constexpr int kSalRows = 32;       // pooled queries per saliency workgroup
#ifndef ISA_FLASH_WAVES
#define ISA_FLASH_WAVES 8
#endif
#ifndef ISA_FLASH_PIPE
#define ISA_FLASH_PIPE 0
#endif
constexpr int kFlashWaves = ISA_FLASH_WAVES;    // waves per full-attention workgroup
constexpr int kFlashPipe = ISA_FLASH_PIPE;      // issue S(j+1) before the softmax of S(j)
constexpr int kFlashRows = 32 * kFlashWaves;    // query rows per full-attention workgroup
constexpr int kCUs = 256;          // compute units of the target GPU (split-K balance)
constexpr int kMaxSplits = 8;
constexpr int kItemCost = 3;      // fixed cost of a full-route work item, in key tiles (split choice)
constexpr int kPpMinTiles64 = 48;  // key tiles per workgroup from which d = 64 takes the ping-pong kernel
constexpr size_t kWsAlign = 256;
constexpr int kMaxBH = 65535;            // B*H: grid-y of the per-head launches
constexpr int64_t kMaxSpan = int64_t(1) << 31;   // bytes of one head of a tensor (32-bit offsets)
constexpr int64_t kMaxRowStride = int64_t(1) << 24;   // bytes between rows (24-bit multiplies)
constexpr int kMaxRows = (1 << 24) - 1;  // Ns + Nc

// Row addressing of one caller tensor [B,H,rows,d]: element strides of the
// batch, head and row dimensions (d is unit-stride) and the head count; row
// r of slice bh = x*H + h starts at element x*sb + h*sh + r*sn.  hmul =
// ceil(2^32 / H) (0 for H = 1) gives x = (bh * hmul) >> 32 exactly for
// bh < 2^16: with hmul*H = 2^32 + e, 0 <= e < H, the product overshoots
// bh/H by bh*e/(H 2^32) < 1/H, less than the gap to the next integer.
struct RowMap {
  int64_t sb, sh;
  int32_t sn;          // < 2^23 elements (row step under 2^24 bytes)
  int32_t H;
  uint32_t hmul;
  int32_t pad;
};

// Bytes from the first to the last byte of one head of a tensor of `rows`
// rows of d elements of es bytes addressed by m.
inline int64_t span_bytes(const RowMap& m, int rows, int d, int es) {
  return ((int64_t)(rows > 0 ? rows - 1 : 0) * m.sn + d) * es;
}

struct Layout {
  int64_t BH;          // B*H slices
  RowMap q, k, v, o;   // Q (and dQ, Qc), K (and dK), V (and dV), O (and dO, Oc)
  int Ns, Nc, Nk, d, b, es;   // es = element size of Q/K/V/O
  int nb_s, nb_c, M;   // source blocks, context blocks, all blocks
  int kc, kq, mk;      // kept context blocks, full-route query blocks, kept blocks
  int mk_pad;          // mk rounded up to kTileKeys
  int tail_s, tail_c;  // rows in the last source / context block
  int sal_tiles;       // ceil(nb_s / kSalRows)
  int64_t ctx_tok;     // kc*b: context key tokens of the full route (with tail padding)
  int64_t full_rows;   // kq*b virtual full-route query rows
  int64_t taylor_rows; // (nb_s-kq)*b virtual Taylor-route query rows
  int full_splits;     // key-range splits of the full-route attention: the FP8 variant, d = 64, the backward's dQ
  // bf16 full route (d = 128; d = 64 from kPpMinTiles64 key tiles per
  // workgroup), on sk_grid workgroups (0: off, full_splits parts): row tiles
  // Ri = bh * row tiles + rt.  Workgroup g first takes whole row tiles
  // g, g + sk_grid, ... (sk_rounds of them, row tiles below sk_rounds *
  // sk_grid), then range g of the (row tile, key tile) units of the rest,
  // u = (Ri - sk_rounds * sk_grid) * key tiles + t, cut into sk_G equal
  // ranges (range g: units [g U / sk_G, (g + 1) U / sk_G)).  A row tile
  // inside one range needs no merge; one meets at most sk_P ranges (its
  // parts).
  int sk_grid, sk_rounds, sk_G, sk_P;
  int n_keytab;        // full-route key rows per head, rounded up to kTileKeys
  // byte offsets into the workspace
  size_t off_qbar, off_kbar, off_vbar, off_salp, off_sal, off_kept;
  size_t off_pkhi, off_pklo, off_pv, off_pbias, off_ctxrows;
  size_t off_keyrows;  // [BH][n_keytab] int32: row of K/V of every full-route key (0 for padding)
  size_t off_peak, off_sh, off_fullq, off_taylq;
  size_t off_part_o, off_part_ml;
  size_t off_lse;      // [BH][Ns] log2-domain log-sum-exp of each source row's softmax
  size_t total;
};

// Validates *desc and fills *L.  Returns ISA_OK or the error of isa.h.
isa_status make_layout(const isa_desc* desc, Layout* L);

// True when no two elements of the [B,rows,d] x m.H tensor addressed by m
// share an address (the strides of an output).
bool map_disjoint(const RowMap& m, int B, int rows, int d);

// isa_context_forward: Q and O maps of the context query rows [B,H,Nc,d]
// (the q and o strides of *desc, with Nc rows; contiguous defaults).
isa_status context_maps(const isa_desc* desc, Layout* L);

// Validates `n` tensor pointers: non-null and 16-byte aligned.
isa_status check_tensors(const void* const* ptrs, int n);

// Validates a workspace pointer and size against `need` bytes.
isa_status check_workspace(const void* ws, size_t bytes, size_t need);

// Backward pass (bf16): keys per dK/dV workgroup (8 waves x 32) and query
// rows staged per step.
constexpr int kBwdKeys = 256;
constexpr int kBwdRows = 64;
constexpr int kBwdMaxParts = 16;   // parts of a split key tile of the last dK/dV round

struct BwdLayout {
  int dkv_splits;      // query-row splits of the pooled (Taylor) dK/dV pass
  int dkv_key_tiles;   // ceil(mk / kBwdKeys)
  // byte offsets into the backward workspace
  size_t off_delta;    // [BH][Ns] fp32: rowsum(dO * O)
  size_t off_part_dkv; // [dkv_splits][BH][mk_pad][2][d] fp32 pooled-key gradient partials
  size_t off_dkvbar;   // [BH][mk_pad][2][d] fp32: pooled-key gradients (dkbar, dvbar)
  size_t off_part_dq;  // [BH][full row tiles * kFlashRows][full_splits][d] fp32 split-K partials of dQ
  // Full-route dK and dV at d = 128 (item = head x 256-key tile, all the
  // route's query tiles): the items past kv_rounds * kCUs are the last,
  // part-filled round; with kv_parts > 1 each of them is cut into kv_parts
  // ranges of query tiles, one workgroup each, their fp32 partials merged.
  int kv_rounds, kv_rest, kv_parts;
  size_t off_part_kv;  // [kv_rest * kv_parts][kBwdKeys][d] fp32 partials (dK, then dV)
  // Full-route dQ at d = 128 (item = head x 256-row tile, all key tiles):
  // the same cut of its last round into dq_parts key ranges (0: not cut; the
  // partials then take off_part_dq as [dq_rest * dq_parts][kFlashRows][d]).
  int dq_rounds, dq_rest, dq_parts;
  int n_rowtab;        // full-route virtual rows per head, rounded up to 64
  size_t off_rrow;     // [BH][n_rowtab] int32: source row of each full-route row (0 for padding)
  size_t off_rlse;     // [BH][n_rowtab] fp32: its forward log-sum-exp (+inf for padding)
  size_t off_rdel;     // [BH][n_rowtab] fp32: its D = dO . O (0 for padding)
  size_t total;
};

// Fills *B for the layout L (ISA_ERR_UNSUPPORTED unless bf16).
isa_status make_bwd_layout(const Layout& L, BwdLayout* B);

// FP8 variant of the full route: the key list in e4m3 with its scales.
struct Fp8Layout {
  int nkp;             // key list length rounded up to 64
  int ntile;           // nkp / 64
  size_t off_k8;       // [BH][nkp][d] e4m3
  size_t off_ks;       // [BH][nkp][d/32] e8m0
  size_t off_v8t;      // [BH][ntile][d][64] e4m3, transposed per tile
  size_t off_vs;       // [BH][ntile][d][2] e8m0
  size_t total;
};

// Fills *F for the layout L (ISA_ERR_UNSUPPORTED unless bf16).
isa_status make_fp8_layout(const Layout& L, Fp8Layout* F);

// Key-range splits for `units` workgroups of `ntiles` key tiles each, on
// kCUs compute units running one workgroup each: the count that minimises
// (rounds of workgroups) x (tiles per workgroup + fixed cost), 1 unless a
// split saves at least 2%.
int choose_splits(int64_t units, int ntiles);

}  // namespace isa
