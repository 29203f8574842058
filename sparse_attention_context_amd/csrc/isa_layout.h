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
constexpr size_t kWsAlign = 256;

struct Layout {
  int64_t BH;          // B*H slices
  int Ns, Nc, Nk, d, b, es;   // es = element size of Q/K/V/O
  int nb_s, nb_c, M;   // source blocks, context blocks, all blocks
  int kc, kq, mk;      // kept context blocks, full-route query blocks, kept blocks
  int mk_pad;          // mk rounded up to kTileKeys
  int tail_s, tail_c;  // rows in the last source / context block
  int sal_tiles;       // ceil(nb_s / kSalRows)
  int64_t ctx_tok;     // kc*b: context key tokens of the full route (with tail padding)
  int64_t full_rows;   // kq*b virtual full-route query rows
  int64_t taylor_rows; // (nb_s-kq)*b virtual Taylor-route query rows
  int full_splits;     // key-range splits of the full-route attention (bf16)
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

// Backward pass (bf16): keys per dK/dV workgroup (8 waves x 32) and query
// rows staged per step.
constexpr int kBwdKeys = 256;
constexpr int kBwdRows = 64;

struct BwdLayout {
  int dkv_splits;      // query-row splits of the pooled (Taylor) dK/dV pass
  int dkv_key_tiles;   // ceil(mk / kBwdKeys)
  // byte offsets into the backward workspace
  size_t off_delta;    // [BH][Ns] fp32: rowsum(dO * O)
  size_t off_part_dkv; // [dkv_splits][BH][mk_pad][2][d] fp32 pooled-key gradient partials
  size_t off_dkvbar;   // [BH][mk_pad][2][d] fp32: pooled-key gradients (dkbar, dvbar)
  size_t off_part_dq;  // [BH][full row tiles * kFlashRows][full_splits][d] fp32 split-K partials of dQ
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
