// Backward pass of ISA (bf16, gfx950 MFMA), the selection plan frozen.
//
// The layer of "Lightning Unified Video Editing via In-Context Sparse
// Attention" (English abstract): full-route rows attend exactly over the
// tokens of the kept key set, Taylor rows over the kept pooled blocks with
// weights n_j.  The pages give no backward pass; these kernels compute the
// derivatives of that forward for L = sum(dO * O), with the selection
// (kept_ctx, full_q) held fixed:
//   D_i  = dO_i . o_i
//   ds_ij = p_ij (dO_i . v_j - D_i)        (p the row's softmax, pooled: n_j-weighted)
//   dq_i = sum_j ds_ij k_j / sqrt d,  dk_j = sum_i ds_ij q_i / sqrt d,  dv_j = sum_i p_ij dO_i
// and a pooled key's gradient is shared equally by the rows of its block
// (dk_t += dkbar_j / n_j), since kbar_j is their mean.  p is recomputed from
// the forward's per-row log-sum-exp: p = exp2(x - lse), x = S*log2(e)/sqrt d
// (tokens) or that plus log2 n_j (pooled).
//
// Kernels (in isa_backward order):
//   delta       D for every source row
//   dk, dv pooled  Taylor rows x kept pooled blocks: per-split partials of dkbar, dvbar
//   dkv reduce     partials summed in split order
//   dk, dv full    full rows x kept tokens: dK (dV) of every source and kept
//                  context row, plus the pooled share of its block
//   zero        dK, dV rows of pruned context blocks
//   dq full     full rows x kept tokens (split-K like the forward) + merge
//   dq pooled   Taylor rows x kept pooled blocks
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16; lane l: row l%32, k = 8(l/32)..+7 of
// A; the same k of column l%32 of B; accumulator reg r of lane l is row
// 8(r/4) + 4(l/32) + r%4, column l%32):
//   dq kernel   (rows fixed, keys streamed, 8 waves x 32 rows): S^T = K Q^T and
//     dP^T = V dO^T put one query per lane, so ds^T is already the B operand
//     of dQ^T += K^T ds^T, whose A operand K^T comes from LDS transpose reads.
//   dk/dv kernels (keys fixed, rows streamed, 8 waves x 32 keys): S = Q K^T and
//     dP = dO V^T put one key per lane, so p and ds are the B operands of
//     dV^T += dO^T p and dK^T += Q^T ds; dO^T and Q^T come from transpose reads.
// Each tile kept for both plain and transposed reads is stored twice in LDS:
// with 16 bytes of row padding (conflict-free 16-byte row reads) and with 64
// (conflict-free transpose reads).
#include "isa_device.h"
#include "isa_kernels.h"

namespace isa {

#ifndef ISA_BWD_DV_PP
#define ISA_BWD_DV_PP 1
#endif
constexpr bool kUseDvPP = ISA_BWD_DV_PP;
#ifndef ISA_BWD_DK_PP
#define ISA_BWD_DK_PP 1
#endif
constexpr bool kUseDkPP = ISA_BWD_DK_PP;
#ifndef ISA_BWD_DQ_PP
#define ISA_BWD_DQ_PP 1
#endif
constexpr bool kUseDqPP = ISA_BWD_DQ_PP;

static_assert(kFlashRows == 256, "the dQ kernel and its merge use 256-row tiles");

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  RowMap rmq, rmk, rmv, rmo;   // element strides: Q and dQ, K and dK, V and dV, O and dO
  const float* lse;      // [BH][Ns] from the forward
  float* delta;          // [BH][Ns]
  const int* ctx_rows;   // [BH][ctx_tok]
  const int* kept;       // [BH][kc]
  long long ctx_tok;
  int kc, nb_c, b, tail_s, tail_c;
  const void* pkhi;      // [BH][mk_pad][D] kept pooled keys (hi, lo) and values
  const void* pklo;
  const void* pv;
  const float* pbias;    // [BH][mk_pad] log2 n_j, -inf for padding
  int mk, mk_pad;
  const int* q_list;     // route block list [BH][q_k]
  int q_k, nb_s;
  long long n_rows;      // virtual rows of the route per head
  float* part_dq;        // [BH][row_tiles*256][nsplit][D]
  float* part_dkv;       // [nsplit][BH][mk_pad][2][D]
  float* dkvbar;         // [BH][mk_pad][2][D]
  int nsplit, tiles_per_split;
  int Ns, Nk;
  int row_tiles, key_tiles;
  int n_wg;
  long long BH;
  float scale_log2;      // log2(e)/sqrt(d)
  float inv_sqrt_d;
  const int* key_rows;   // [BH][n_keytab] row of every full-route key (0 for padding)
  int n_keytab;
  int* rrow;             // [BH][n_rowtab] full route in row order: source row (0 for padding),
  float* rlse;           //   log-sum-exp (+inf for padding) and
  float* rdel;           //   D (0 for padding)
  int n_rowtab;
  long long delta_wgs;   // workgroups of the delta launch that cover the source rows
  // full-route dK / dV at d = 128: the last round's kv_rest items cut into
  // kv_parts ranges of query tiles (0: not cut), their partials in part_kv
  int kv_rounds, kv_rest, kv_parts;
  float* part_kv;        // [kv_rest * kv_parts][kBwdKeys][D]
  // full-route dQ at d = 128: the same cut of its last round of row tiles
  // into dq_parts key ranges (partials [dq_rest * dq_parts][256][D] in part_dq)
  int dq_rounds, dq_rest, dq_parts;
};

// Work item of the full-route dK and dV kernels at d = 128: head bh, key
// tile kt, query tiles q0 .. q0 + nq - 1 of the route.  Uncut (kv_parts = 0):
// item lid = bh * key_tiles + kt, all query tiles.  Cut: the n_wg / 8
// workgroups of XCD x (logical ids x L .., L = n_wg / 8) take 32 kv_rounds
// whole items of their own (consecutive items: one head's key tiles) and
// then their share of the parts of the last round's items, part p of item
// kCUs kv_rounds + s covering query tiles [p Q / P, (p + 1) Q / P) and
// writing partial slot s P + p (slot < 0: a whole item, written directly).
// (The cut in general: item id of `rounds` whole rounds of kCUs, then part p
// of item kCUs rounds + s, covering [p span / parts, (p + 1) span / parts).)
struct CutItem { int id, r0, n, slot; bool live; };
__device__ __forceinline__ CutItem cut_item(int n_wg, int rounds, int rest, int parts, int span) {
  CutItem it = {0, 0, span, -1, true};
  const int lid = xcd_remap(blockIdx.x, n_wg);
  it.id = lid;
  if (parts > 0) {
    const int L = n_wg >> 3, x = lid / L, i = lid - x * L, nw = (kCUs / 8) * rounds;
    if (i < nw) {
      it.id = x * nw + i;
    } else {
      const int p_idx = x * (L - nw) + (i - nw);
      if (p_idx >= rest * parts) {
        it.live = false;   // padding of the XCD's share
        return it;
      }
      const int sp = p_idx / parts, p = p_idx - sp * parts;
      it.id = kCUs * rounds + sp;
      it.r0 = p * span / parts;
      it.n = (p + 1) * span / parts - it.r0;
      it.slot = p_idx;
    }
  }
  return it;
}
struct KvItem { int bh, kt, q0, nq, slot; bool live; };
__device__ __forceinline__ KvItem kv_item(const BwdArgs& a, int qtiles) {
  const CutItem c = cut_item(a.n_wg, a.kv_rounds, a.kv_rest, a.kv_parts, qtiles);
  const int bh = c.id / a.key_tiles;
  return KvItem{bh, c.id - bh * a.key_tiles, c.r0, c.n, c.slot, c.live};
}

// A part's raw sum over its query tiles (lane: key w*32 + l32 of the tile,
// d = 32 t + 8 g + 4 h + e), for isa_bwd_kv_merge_kernel.
template <int NT>
__device__ __forceinline__ void kv_store_part(const BwdArgs& a, int slot, int w, int l32, int h, const f32x16* acc) {
  constexpr int D = NT * 32;
  float* pp = a.part_kv + ((long long)slot * kBwdKeys + w * 32 + l32) * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(pp + 32 * t + 8 * g + 4 * h) = f32x4{acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2], acc[t][4 * g + 3]};
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i, 8 elements per lane, D/8 lanes per row.

// Workgroups past delta_wgs write the full route in row order (rrow, rlse,
// rdel: one entry per virtual row, padding to whole tiles of 64), with D
// formed by the same code as for the source rows.
template <int D>
__global__ __launch_bounds__(256) void isa_bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int e = (threadIdx.x % LPR) * 8;
  long long row;       // bh * Ns + source row (the workspace's row order)
  long long bh;
  bool ok;
  long long rv = -1;   // route entry (bh * n_rowtab + v) of the route workgroups
  if ((long long)blockIdx.x < a.delta_wgs) {
    row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    ok = row < a.BH * a.Ns;
    bh = ok ? row / a.Ns : 0;
  } else {
    rv = ((long long)blockIdx.x - a.delta_wgs) * RPB + threadIdx.x / LPR;
    bh = rv / a.n_rowtab;
    const int r = bh < a.BH ? route_row(a.q_list + bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, rv - bh * a.n_rowtab) : -1;
    ok = r >= 0;
    row = bh * a.Ns + (r < 0 ? 0 : r);
    if (bh >= a.BH) rv = -1;
  }
  float s = 0.f;
  if (ok) {
    // (non-temporal: a streaming read of O and dO, which share O's strides)
    const long long off = rm_head(a.rmo, bh) + (row - bh * a.Ns) * a.rmo.sn + e;
    const u32x4 o = __builtin_nontemporal_load((const u32x4*)((const bf16_t*)a.O + off));
    const u32x4 g = __builtin_nontemporal_load((const u32x4*)((const bf16_t*)a.dO + off));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s += __uint_as_float(o[i] << 16) * __uint_as_float(g[i] << 16) +
           __uint_as_float(o[i] & 0xffff0000u) * __uint_as_float(g[i] & 0xffff0000u);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);
  if (rv < 0) {
    if (ok && e == 0) a.delta[row] = s;
  } else if (e == 0) {
    const long long bh = rv / a.n_rowtab;
    a.rrow[rv] = ok ? (int)(row - bh * a.Ns) : 0;
    a.rlse[rv] = ok ? a.lse[row] : INFINITY;
    a.rdel[rv] = ok ? s : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dQ: 8 waves x 32 query rows, key tiles of 64 (two halves of 32), 2-stage
// LDS ring.  POOLED: keys are the kept pooled blocks (hi + lo logits, bias
// log2 n_j); else the full route's gathered tokens.

template <int D, bool POOLED>
__global__ __launch_bounds__(512) void isa_bwd_dq_kernel(BwdArgs a) {
  typedef bf16x8 Op;
  constexpr int NW = 8, NTHR = NW * 64, BN = 64, BM = 32 * NW, ES = 2;
  constexpr int KRB = D * ES, KCPR = KRB / 16;
  constexpr int KRS = KRB + 16, TRS = KRB + 64;
  constexpr int NKT = POOLED ? 2 : 1;
  constexpr int KT = BN * KRS, TT = BN * TRS;
  constexpr int OFF_V = NKT * KT, OFF_KT = OFF_V + KT;   // stage: K (hi[, lo]) | V | K for transpose reads
  constexpr int STAGE = OFF_KT + TT;
  constexpr int NSTAGE = 2;
  constexpr int NKC = BN * KCPR / NTHR;
  constexpr int NT = D / 32;
  static_assert(NKC >= 1, "tile mapping");

  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * STAGE];
  __shared__ __attribute__((aligned(16))) float sbias[POOLED ? NSTAGE : 1][BN];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  // work item lid: row tile fastest, then key split, then head (as the
  // forward flash kernels), so that the workgroups running at once on an XCD
  // share one K/V range in its L2
  const int lid = xcd_remap(blockIdx.x, a.n_wg);
  const int rt = lid % a.row_tiles;
  const int rest = lid / a.row_tiles;
  const int split = rest % a.nsplit;
  const int bh = rest / a.nsplit;

  const long long vrow = (long long)rt * BM + w * 32 + l32;
  const int qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  Op qB[D / 16], gB[D / 16];
  float lse_r = INFINITY, del_r = 0.f;  // rows off the route: p = 0
  {
    const long long r = (long long)bh * a.Ns + (qrow < 0 ? 0 : qrow);
    const long long qr = qrow < 0 ? 0 : qrow;
    const bf16_t* qp = (const bf16_t*)a.Q + rm_head(a.rmq, bh) + qr * a.rmq.sn + 8 * h;
    const bf16_t* gp = (const bf16_t*)a.dO + rm_head(a.rmo, bh) + qr * a.rmo.sn + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qB[s] = *(const Op*)(qp + 16 * s);
      gB[s] = *(const Op*)(gp + 16 * s);
    }
    if (qrow >= 0) {
      lse_r = a.lse[r];
      del_r = a.delta[r];
    }
  }

  int n_keys, n_valid;
  if constexpr (POOLED) {
    n_keys = n_valid = a.mk_pad;
  } else {
    n_keys = a.Ns + (int)a.ctx_tok;
    const bool tail_kept = a.kc > 0 && a.kept[(long long)bh * a.kc + a.kc - 1] == a.nb_c - 1;
    n_valid = n_keys - (tail_kept ? a.b - a.tail_c : 0);
  }
  const int ntiles = (n_keys + BN - 1) / BN;
  const int t_begin = split * a.tiles_per_split;
  const int nt = max(0, min(a.tiles_per_split, ntiles - t_begin));
  const int t_last = t_begin + nt - 1;

  const char* Kg;
  const char* Kg_lo = nullptr;
  const char* Vg;
  long long krs = KRB, vrs = KRB;   // bytes between key rows, value rows
  if constexpr (POOLED) {
    Kg = (const char*)a.pkhi + (long long)bh * a.mk_pad * KRB;
    Kg_lo = (const char*)a.pklo + (long long)bh * a.mk_pad * KRB;
    Vg = (const char*)a.pv + (long long)bh * a.mk_pad * KRB;
  } else {
    Kg = (const char*)a.K + rm_head(a.rmk, bh) * ES;
    Vg = (const char*)a.V + rm_head(a.rmv, bh) * ES;
    krs = a.rmk.sn * ES;
    vrs = a.rmv.sn * ES;
  }
  const int* crow = POOLED ? nullptr : a.ctx_rows + (long long)bh * a.ctx_tok;
  const int ctx_last = (int)a.ctx_tok - 1;

  struct Staged { u32x4 k[NKT][NKC]; u32x4 v[NKC]; float bias; };
  // global row of key t of the range (padding -> row 0, masked later)
  auto key_row = [&](int t) -> int {
    if constexpr (POOLED) {
      return t;
    } else {
      if (t < a.Ns) return t;
      int c = 0;
      if (ctx_last >= 0) c = crow[min(max(t - a.Ns, 0), ctx_last)];
      return t < n_valid && c >= 0 ? c : 0;
    }
  };
  auto load = [&](int tile) -> Staged {
    Staged g;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int q = tid + NTHR * i;
      const int row = key_row(tile * BN + q / KCPR);
      const int c = q % KCPR;
      g.k[0][i] = *(const u32x4*)(Kg + (long long)row * krs + c * 16);
      if constexpr (POOLED) g.k[1][i] = *(const u32x4*)(Kg_lo + (long long)row * krs + c * 16);
      g.v[i] = *(const u32x4*)(Vg + (long long)row * vrs + c * 16);
    }
    g.bias = 0.f;
    if constexpr (POOLED) {
      if (tid < BN) g.bias = a.pbias[(long long)bh * a.mk_pad + tile * BN + tid];
    }
    return g;
  };
  auto store = [&](int stage, const Staged& g) {
    char* S0 = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int q = tid + NTHR * i;
      const int kr = q / KCPR, c = q % KCPR;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) *(u32x4*)(S0 + kt * KT + kr * KRS + c * 16) = g.k[kt][i];
      *(u32x4*)(S0 + OFF_V + kr * KRS + c * 16) = g.v[i];
      *(u32x4*)(S0 + OFF_KT + kr * TRS + c * 16) = g.k[0][i];
    }
    if constexpr (POOLED) {
      if (tid < BN) sbias[stage][tid] = g.bias;
    }
  };

  const int kbase = l32 * KRS + 16 * h;
  // K^T operand of lane (l32, h) in 16-lane group g, m = lane%16: transposed
  // reads at key rows 16 s + 4 h + m/4 (+8), d = 32 t + 16 (g%2) + 4 (m%4)
  const int tbase = OFF_KT + (4 * h + ((lane & 15) >> 2)) * TRS + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * ES;
  const float sc = a.scale_log2;

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};

  auto tile_step = [&](int j, int stage) {
    const char* S0 = smem + stage * STAGE;
    const int t0 = (t_begin + j) * BN;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const char* Ks = S0 + kbase + half * 32 * KRS;
      f32x16 St = f32x16{}, Pt = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        St = mma32(*(const Op*)(Ks + 32 * s), qB[s], St);
        if constexpr (POOLED) St = mma32(*(const Op*)(Ks + KT + 32 * s), qB[s], St);
        Pt = mma32(*(const Op*)(Ks + OFF_V + 32 * s), gB[s], Pt);
      }
      Op dsB[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = half * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        float x;
        if constexpr (POOLED) {
          x = fmaf(St[r], sc, sbias[stage][key]);
        } else {
          x = t0 + key < n_valid ? St[r] * sc : -INFINITY;
        }
        const float p = __builtin_amdgcn_exp2f(x - lse_r);
        dsB[r >> 3][r & 7] = (__bf16)(p * (Pt[r] - del_r));
      }
      const lds_char* Ts = (const lds_char*)S0 + tbase + half * 32 * TRS;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const lds_char* p = Ts + 16 * s * TRS + 32 * t * ES;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * TRS));
          const Op kt = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[t] = mma32(kt, dsB[s], acc[t]);
        }
    }
  };

  if (nt > 0) {
    store(0, load(t_begin));
    __syncthreads();
  }
  for (int j = 0; j < nt; ++j) {
    const Staged g = load(min(t_begin + j + 1, t_last));
    tile_step(j, j & 1);
    if (j + 1 < nt) store((j + 1) & 1, g);
    __syncthreads();
  }

  if (qrow < 0 && a.nsplit == 1) return;
  if (a.nsplit == 1) {
    bf16_t* op = (bf16_t*)a.dQ + rm_head(a.rmq, bh) + (long long)qrow * a.rmq.sn;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& c = acc[t];
        const float sd = a.inv_sqrt_d;
        *(u32x2*)(op + 32 * t + 8 * g + 4 * h) = u32x2{pack_bf16x2(c[4 * g] * sd, c[4 * g + 1] * sd),
                                                       pack_bf16x2(c[4 * g + 2] * sd, c[4 * g + 3] * sd)};
      }
  } else {
    float* pp = a.part_dq + (((long long)bh * a.row_tiles * BM + vrow) * a.nsplit + split) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& c = acc[t];
        *(f32x4*)(pp + 32 * t + 8 * g + 4 * h) = f32x4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
      }
  }
}

// dQ of full-route rows from the split partials, summed in split order:
// every row tile's full_splits parts (d = 64), or the dq_parts parts of the
// cut row tiles of the last round (dq_parts > 0: the launch covers their rows).
template <int D>
__global__ __launch_bounds__(256) void isa_bwd_dq_merge_kernel(BwdArgs a) {
  constexpr int TPR = D / 4, RPB = 256 / TPR;
  long long gid = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int e = (threadIdx.x % TPR) * 4;
  long long prow, pstep;   // partial rows prow + k pstep
  int np;
  if (a.dq_parts > 0) {
    const long long sp = gid / kFlashRows, r = gid - sp * kFlashRows;
    if (sp >= a.dq_rest) return;
    prow = sp * a.dq_parts * kFlashRows + r;
    pstep = kFlashRows;
    np = a.dq_parts;
    gid = ((long long)kCUs * a.dq_rounds + sp) * kFlashRows + r;   // the row tile's rows
  } else {
    prow = gid * a.nsplit;
    pstep = 1;
    np = a.nsplit;
  }
  const long long rows_head = (long long)a.row_tiles * kFlashRows;
  const long long bh = gid / rows_head;
  const long long vrow = gid - bh * rows_head;
  if (bh >= a.BH) return;
  const int qrow = route_row(a.q_list + bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  if (qrow < 0) return;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < np; ++k) s += *(const f32x4*)(a.part_dq + (prow + k * pstep) * D + e);
  s *= a.inv_sqrt_d;
  *(u32x2*)((bf16_t*)a.dQ + rm_head(a.rmq, bh) + (long long)qrow * a.rmq.sn + e) =
      u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
}

// ---------------------------------------------------------------------------
// dK or dV: 8 waves x 32 keys (2 waves per SIMD), query rows staged 64 at a
// time (two steps of 32), 2-stage LDS ring.  Each lane owns one key column,
// so a key past the range only disturbs its own (unwritten) column and needs
// no mask.  The dK and dV halves are separate kernels: each then keeps one
// accumulator set and fits two waves per SIMD in plain VGPRs, for the price
// of computing the logits twice.
//   DV: S = Q K^T, p = exp2(S sc [+ log2 n_j] - lse), dV^T += dO^T p
//   DK: S, p as above, dP = dO V^T, ds = p (dP - D), dK^T += Q^T ds
// POOLED: keys are the kept pooled blocks, rows the Taylor route, output
// per-split partials of dkbar (dvbar); else keys are the full route's
// tokens, rows the full route, and the epilogue adds the pooled share of
// the key's block and writes dK (dV).

template <int D, bool POOLED, bool DK>
__global__ __launch_bounds__(512) void isa_bwd_dkdv_kernel(BwdArgs a) {
  typedef bf16x8 Op;
  constexpr int NW = 8, NTHR = NW * 64, BK = 32 * NW, BR = kBwdRows, ES = 2;
  constexpr int KRB = D * ES, KCPR = KRB / 16;
  constexpr int KRS = KRB + 16, TRS = KRB + 64;
  constexpr int QT = BR * KRS, QTT = BR * TRS;
  // stage, DK: Q | dO | Q for transpose reads | lse | D;  DV: Q | dO for transpose reads | lse
  constexpr int OFF_G = QT;
  constexpr int OFF_T = DK ? 2 * QT : QT;
  constexpr int OFF_L = OFF_T + QTT;
  constexpr int OFF_D = OFF_L + BR * 4;
  constexpr int STAGE = OFF_D + (DK ? BR * 4 : 0);
  constexpr int NSTAGE = 2;
  constexpr int NRC = BR * KCPR / NTHR;   // 16-byte chunks per thread per Q (and dO) tile
  constexpr int NT = D / 32;
  static_assert(NRC >= 1, "tile mapping");
  static_assert(BK == kBwdKeys, "keys per workgroup");

  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int lid = xcd_remap(blockIdx.x, a.n_wg);
  const int split = lid % a.nsplit;
  const int rest = lid / a.nsplit;
  const int bh = rest / a.key_tiles;
  const int kt = rest - bh * a.key_tiles;

  // ---- this lane's key (column of S): row of K/V, validity, bias
  const int kv = kt * BK + w * 32 + l32;
  int krow;
  bool kvalid;
  const char* Kg;
  const char* Vg;
  float kbias = 0.f;
  if constexpr (POOLED) {
    kvalid = kv < a.mk;
    krow = min(kv, a.mk_pad - 1);
    Kg = (const char*)a.pkhi + ((long long)bh * a.mk_pad + krow) * KRB;
    Vg = (const char*)a.pv + ((long long)bh * a.mk_pad + krow) * KRB;
    kbias = a.pbias[(long long)bh * a.mk_pad + krow];
  } else {
    const int n_keys = a.Ns + (int)a.ctx_tok;
    if (kv < a.Ns) {
      krow = kv;
    } else if (kv < n_keys) {
      krow = a.ctx_rows[(long long)bh * a.ctx_tok + (kv - a.Ns)];
    } else {
      krow = -1;
    }
    kvalid = krow >= 0;
    krow = kvalid ? krow : 0;
    Kg = (const char*)a.K + (rm_head(a.rmk, bh) + (long long)krow * a.rmk.sn) * ES;
    Vg = (const char*)a.V + (rm_head(a.rmv, bh) + (long long)krow * a.rmv.sn) * ES;
  }
  Op kB[D / 16], kBl[POOLED ? D / 16 : 1], vB[DK ? D / 16 : 1];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kB[s] = *(const Op*)(Kg + (16 * s + 8 * h) * ES);
    if constexpr (DK) vB[s] = *(const Op*)(Vg + (16 * s + 8 * h) * ES);
    if constexpr (POOLED)
      kBl[s] = *(const Op*)((const char*)a.pklo + ((long long)bh * a.mk_pad + krow) * KRB + (16 * s + 8 * h) * ES);
  }

  // ---- query rows of this split
  const long long nsteps = (a.n_rows + BR - 1) / BR;
  const long long per = (nsteps + a.nsplit - 1) / a.nsplit;
  const long long s_begin = split * per;
  const int ns = (int)max(0LL, min(per, nsteps - s_begin));
  const int* qlist = a.q_list + (long long)bh * a.q_k;
  const long long qhead = rm_head(a.rmq, bh), ghead = rm_head(a.rmo, bh);

  struct Staged { u32x4 q[NRC]; u32x4 g[NRC]; float l, d; };
  auto load = [&](long long step) -> Staged {
    Staged st;
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int q = tid + NTHR * i;
      const int r = route_row(qlist, a.q_k, a.b, a.nb_s, a.Ns, step * BR + q / KCPR);
      const long long rr = r < 0 ? 0 : r;
      st.q[i] = *(const u32x4*)((const bf16_t*)a.Q + qhead + rr * a.rmq.sn + (q % KCPR) * 8);
      st.g[i] = *(const u32x4*)((const bf16_t*)a.dO + ghead + rr * a.rmo.sn + (q % KCPR) * 8);
    }
    st.l = INFINITY;  // rows off the route: p = 0
    st.d = 0.f;
    if (tid < BR) {
      const int r = route_row(qlist, a.q_k, a.b, a.nb_s, a.Ns, step * BR + tid);
      if (r >= 0) {
        st.l = a.lse[(long long)bh * a.Ns + r];
        if constexpr (DK) st.d = a.delta[(long long)bh * a.Ns + r];
      }
    }
    return st;
  };
  auto store = [&](int stage, const Staged& st) {
    char* S0 = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int q = tid + NTHR * i;
      const int r = q / KCPR, c = q % KCPR;
      *(u32x4*)(S0 + r * KRS + c * 16) = st.q[i];
      if constexpr (DK) {
        *(u32x4*)(S0 + OFF_G + r * KRS + c * 16) = st.g[i];
        *(u32x4*)(S0 + OFF_T + r * TRS + c * 16) = st.q[i];
      } else {
        *(u32x4*)(S0 + OFF_T + r * TRS + c * 16) = st.g[i];
      }
    }
    if (tid < BR) {
      ((float*)(S0 + OFF_L))[tid] = st.l;
      if constexpr (DK) ((float*)(S0 + OFF_D))[tid] = st.d;
    }
  };

  const int abase = l32 * KRS + 16 * h;
  // transposed reads: rows (queries) 16 s + 4 h + m/4 (+8), d = 32 t + 16 (g%2) + 4 (m%4)
  const int tbase = OFF_T + (4 * h + ((lane & 15) >> 2)) * TRS + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * ES;
  const float sc = a.scale_log2;

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};

  auto rows_step = [&](int stage) {
    const char* S0 = smem + stage * STAGE;
#pragma unroll
    for (int qs = 0; qs < BR / 32; ++qs) {
      const char* Qs = S0 + abase + qs * 32 * KRS;
      f32x16 S = f32x16{}, P = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const Op qa = *(const Op*)(Qs + 32 * s);
        S = mma32(qa, kB[s], S);
        if constexpr (POOLED) S = mma32(qa, kBl[s], S);
        if constexpr (DK) P = mma32(*(const Op*)(Qs + OFF_G + 32 * s), vB[s], P);
      }
      // rows of reg r: qs*32 + 8(r/4) + 4h + r%4
      const float* ls = (const float*)(S0 + OFF_L) + qs * 32 + 4 * h;
      const float* ds = (const float*)(S0 + OFF_D) + qs * 32 + 4 * h;
      Op oB[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)(ls + 8 * g);
        f32x4 d4 = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (DK) d4 = *(const f32x4*)(ds + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float p = POOLED ? __builtin_amdgcn_exp2f(fmaf(S[r], sc, kbias) - l4[e])
                                 : __builtin_amdgcn_exp2f(fmaf(S[r], sc, -l4[e]));
          oB[r >> 3][r & 7] = (__bf16)(DK ? p * (P[r] - d4[e]) : p);
        }
      }
      const lds_char* Ts = (const lds_char*)S0 + tbase + qs * 32 * TRS;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int o = 16 * s * TRS + 32 * t * ES;
          const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ts + o));
          const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ts + o + 8 * TRS));
          acc[t] = mma32(__builtin_bit_cast(Op, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7)), oB[s], acc[t]);
        }
    }
  };

  if (ns > 0) {
    store(0, load(s_begin));
    __syncthreads();
  }
  for (int j = 0; j < ns; ++j) {
    const Staged st = load(s_begin + min(j + 1, ns - 1));
    rows_step(j & 1);
    if (j + 1 < ns) store((j + 1) & 1, st);
    __syncthreads();
  }

  // ---- epilogue: lane holds key kv, d = 32 t + 8 g + 4 h + e
  const float scale = DK ? a.inv_sqrt_d : 1.0f;
  if constexpr (POOLED) {
    if (kv >= a.mk_pad) return;
    float* pk = a.part_dkv + (((long long)split * a.BH + bh) * a.mk_pad + kv) * 2 * D + (DK ? 0 : D);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(pk + 32 * t + 8 * g + 4 * h) =
            f32x4{acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2], acc[t][4 * g + 3]} * scale;
  } else {
    if (!kvalid) return;
    // pooled key of the key's block and its count
    int j, n;
    if (kv < a.Ns) {
      j = kv / a.b;
      n = j == a.nb_s - 1 ? a.tail_s : a.b;
    } else {
      const int u = (kv - a.Ns) / a.b;
      j = a.nb_s + u;
      n = a.kept[(long long)bh * a.kc + u] == a.nb_c - 1 ? a.tail_c : a.b;
    }
    const float inv_n = 1.0f / (float)n;
    const float* pb = a.dkvbar + ((long long)bh * a.mk_pad + j) * 2 * D + (DK ? 0 : D);
    bf16_t* out = (bf16_t*)(DK ? a.dK : a.dV) + rm_head(DK ? a.rmk : a.rmv, bh) + (long long)krow * (DK ? a.rmk : a.rmv).sn;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * t + 8 * g + 4 * h;
        const f32x4 bb = *(const f32x4*)(pb + d0);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(acc[t][4 * g + e], scale, bb[e] * inv_n);
        *(u32x2*)(out + d0) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
}

// ---------------------------------------------------------------------------
// dV of the full route at d = 128 on the ping-pong schedule of the forward
// flash kernel, with the roles of rows and keys exchanged: a workgroup holds
// 256 keys (8 waves x 32, one key per lane, K of the key in registers) and
// streams the route's rows in tiles of 64; Q and dO tiles come by direct
// loads into four-stage LDS rings (swizzled rows, as in the forward), their
// source rows and log-sum-exps from the row-ordered route arrays.
//   X_j  dV^T += dO(j-1)^T P(j-1), then S(j) = Q(j) K^T      (MFMA)
//   Y_j  loads of Q(j+3), dO(j+2), lse(j+3) and the row table of tile j+6;
//        P(j) = exp2(S(j) log2(e)/sqrt(d) - lse) in bf16       (VALU)
// Group 0 (waves 0-3) runs X_j in phase 2j and Y_j in 2j+1, group 1 one
// phase later; a stage is refilled only after the last read of its previous
// tile, and every tile is in LDS two phases before its first read (the
// phase arithmetic of the forward kernel, with Q in the place of K and dO
// in the place of V).  The lse tile of step t is loaded by wave 0 in Y_{t-3}
// into slot t % 4 and read in Y_t by both groups.  Padding rows have
// lse = +inf (p = 0).  The arithmetic is that of isa_bwd_dkdv_kernel.
#ifndef ISA_BWD_LOOKAHEAD
#define ISA_BWD_LOOKAHEAD 5
#endif
__global__ __launch_bounds__(512) void isa_bwd_dv_pp_kernel(BwdArgs a) {
  typedef bf16x8 Op;
  constexpr int D = 128, BN = 64, NST = 4, ES = 2;
  constexpr int RB = D * 2, TB = BN * RB, NT = D / 32;
  static_assert(kBwdKeys == 256, "keys per workgroup");

  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * TB];   // Q ring, then dO ring
  __shared__ __attribute__((aligned(16))) int stab[8][4][64];         // per-wave row-table ring
  __shared__ __attribute__((aligned(256))) float slse[NST][BN];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const KvItem item = kv_item(a, a.n_rowtab / BN);
  if (!item.live) return;
  const int bh = item.bh, kt = item.kt;

  // ---- this lane's key: row of K/V and validity (as isa_bwd_dkdv_kernel)
  const int kv = kt * kBwdKeys + w * 32 + l32;
  const int n_keys = a.Ns + (int)a.ctx_tok;
  int krow;
  if (kv < a.Ns) krow = kv;
  else if (kv < n_keys) krow = a.ctx_rows[(long long)bh * a.ctx_tok + (kv - a.Ns)];
  else krow = -1;
  const bool kvalid = krow >= 0;
  krow = kvalid ? krow : 0;
  Op kB[D / 16];
  {
    const char* Kg = (const char*)a.K + (rm_head(a.rmk, bh) + (long long)krow * a.rmk.sn) * ES;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kB[s] = *(const Op*)(Kg + (16 * s + 8 * h) * ES);
  }

  const int nt = item.nq;   // row tiles of the route in the item, from item.q0
  const char* Qg = (const char*)a.Q + rm_head(a.rmq, bh) * 2;
  const char* Gg = (const char*)a.dO + rm_head(a.rmo, bh) * 2;
  const unsigned qrs = (unsigned)a.rmq.sn * 2u, grs = (unsigned)a.rmo.sn * 2u;   // row steps in bytes
  const int* tab = a.rrow + (long long)bh * a.n_rowtab + item.q0 * BN;
  const float* lseg = a.rlse + (long long)bh * a.n_rowtab + item.q0 * BN;

  // This wave loads rows 32*grp + 8*wg + 4*i + lane/16 (i = 0, 1) of each
  // tile; the row-table entries of its 8 rows of tile t come to slot t % 4 of
  // its LDS ring by a direct load in step t-6 and are read in step t-4.
  const int lrow0 = 32 * grp + 8 * wg + (lane >> 4);
  struct Rows { int r[2]; };
  const unsigned stab_w = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_char*)&stab[0][0][0]) +
                          __builtin_amdgcn_readfirstlane(w) * (unsigned)sizeof(stab[0]);
  auto fetch_rows = [&](int j, int tile) {
    const int k = 4 * (lane & 1) + ((lane >> 1) & 3);
    dma4(stab_w + (unsigned)(j & 3) * (unsigned)sizeof(stab[0][0]), tab, (unsigned)(tile * BN + 32 * grp + 8 * wg + k) * 4u);
  };
  auto rows_of = [&](int j) -> Rows {
    const int2 v = *(const int2*)&stab[w][j & 3][2 * (lane >> 4)];
    return Rows{{v.x, v.y}};
  };
  const unsigned lds_q = (unsigned)(size_t)(lds_char*)smem;
  const unsigned lds_g = lds_q + NST * TB;
  const unsigned lds_l = (unsigned)(size_t)(lds_char*)&slse[0][0];
  unsigned lchunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) lchunk[i] = (unsigned)(((lane & 15) ^ lds_swz(lrow0 + 4 * i)) * 16);
  const unsigned wrow = __builtin_amdgcn_readfirstlane((32 * grp + 8 * wg) * RB);
  auto issue_tile = [&](unsigned ring, int stage, const char* base, Rows rows, unsigned rs) {
    const unsigned d0 = ring + wrow + (unsigned)stage * TB;
    dma16x2(d0, d0 + 4 * RB, base, __umul24((unsigned)rows.r[0], rs) + lchunk[0],
            __umul24((unsigned)rows.r[1], rs) + lchunk[1]);
  };
  auto issue_lse = [&](int slot, int tile) {
    if (w == 0) dma4(lds_l + (unsigned)slot * BN * 4, lseg + tile * BN, (unsigned)lane * 4u);
  };

  // operand offsets (as the forward kernel): Q row 32*ti + l32, chunk 2s + h;
  // dO^T transpose reads at rows 16s + 4h + m/4 (+8), d = 32t + 16(g%2) + 4(m%4)
  int koff[8], voff[NT][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = l32 * RB + ((((2 * s + h) ^ lds_swz(l32)) * 16));
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int m = lane & 15;
      const int kr = 4 * h + (m >> 2) + 8 * hi;
      const int c = 4 * t + 2 * ((lane >> 4) & 1) + ((m & 3) >> 1);
      voff[t][hi] = NST * TB + kr * RB + ((c ^ lds_swz(kr)) * 16) + 8 * (m & 1);
    }

  struct STile { f32x16 t[2]; };
  struct PTile { Op p[4]; };
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  const float sc = a.scale_log2;

  // X phase: 16 MFMAs of dO^T P, then 16 of Q K^T, reads LA MFMAs ahead
  auto x_phase = [&](int gstage, const PTile& P, int qstage) -> STile {
    constexpr int LA = ISA_BWD_LOOKAHEAD;
    const lds_char* Gs = (const lds_char*)smem + gstage * TB;
    const lds_char* Qs = (const lds_char*)smem + qstage * TB;
    Op opv[16], opk[16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Gs + voff[t][0] + 16 * q * RB));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Gs + voff[t][1] + 16 * q * RB));
        opv[4 * t + q] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) opk[2 * q + ti] = *(const Op*)(Qs + koff[q] + 32 * ti * RB);
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m >> 2] = mma32(opv[m], P.p[m & 3], acc[m >> 2]);
    STile S;
    S.t[0] = f32x16{};
    S.t[1] = f32x16{};
#pragma unroll
    for (int m = 0; m < 16; ++m) S.t[m & 1] = mma32(opk[m], kB[m >> 1], S.t[m & 1]);
    pp_issue_order<LA>();
    return S;
  };
  // P = exp2(S sc - lse_row); rows of reg r of tile ti: 32 ti + 8 (r/4) + 4h + r%4
  auto probs = [&](int slot, const STile& S) -> PTile {
    PTile P;
    const float* ls = slse[slot];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)(ls + 32 * ti + 8 * g + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          P.p[2 * ti + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S.t[ti][r], sc, -l4[e]));
        }
      }
    return P;
  };
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  auto cl = [&](int j) { return min(j, nt - 1); };
  if (nt > 0) {
    Rows rk, rv;   // rows of tiles j+3 (Q) and j+2 (dO) entering step j
    {
      fetch_rows(cl(0), cl(0));
      fetch_rows(cl(1), cl(1));
      fetch_rows(cl(2), cl(2));
      fetch_rows(cl(3), cl(3));
      __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
      const Rows r0 = rows_of(cl(0)), r1 = rows_of(cl(1));
      rv = rows_of(cl(2));
      rk = rows_of(cl(3));
      issue_tile(lds_q, 0, Qg, r0, qrs);
      issue_tile(lds_g, 0, Gg, r0, grs);
      issue_tile(lds_q, 1, Qg, r1, qrs);
      issue_tile(lds_g, 1, Gg, r1, grs);
      issue_tile(lds_q, 2, Qg, rv, qrs);   // (dO(2) is loaded by the first step)
      issue_lse(0, cl(0));
      issue_lse(1, cl(1));
      issue_lse(2, cl(2));
      fetch_rows(cl(4), cl(4));
      fetch_rows(cl(5), cl(5));
      // dO stage 3 is first loaded in step 1; step 0 reads it as zeros
      u32x4* vz = (u32x4*)(smem + NST * TB + 3 * TB);
#pragma unroll
      for (int q = 0; q < TB / (16 * 512); ++q) vz[tid + 512 * q] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    }
    phase_barrier();
    if (grp == 1) phase_barrier();   // group 1 runs one phase behind group 0
    STile S = {};
    PTile P = {};
    auto step = [&](int j) {
      const int Z = j & 3;
      __builtin_amdgcn_s_setprio(3);
      S = x_phase((Z + 3) & 3, P, Z);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
      // Y_j
      issue_tile(lds_q, (Z + 3) & 3, Qg, rk, qrs);
      issue_tile(lds_g, (Z + 2) & 3, Gg, rv, grs);
      issue_lse((Z + 3) & 3, cl(j + 3));
      const Rows rn = rows_of(cl(j + 4));
      fetch_rows(cl(j + 6), cl(j + 6));
      if (j < nt) P = probs(Z, S);
      rv = rk;
      rk = rn;
      // the loads of Y_{j-1} have landed before the barrier that closes Y_j
      if (w == 0) __builtin_amdgcn_s_waitcnt(0x0f76);   // vmcnt(6)
      else __builtin_amdgcn_s_waitcnt(0x0f75);          // vmcnt(5)
      phase_barrier();
    };
    for (int j = 0; j <= nt; ++j) step(j);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // no load into this workgroup's LDS outlives it
    if (grp == 0) phase_barrier();   // balances group 1's extra barrier
  }

  // ---- epilogue: dV of the key plus the pooled share of its block (as
  // isa_bwd_dkdv_kernel); lane holds key kv, d = 32 t + 8 g + 4 h + e.  A
  // part of a cut item leaves its raw sum to the merge.
  if (item.slot >= 0) {
    kv_store_part<NT>(a, item.slot, w, l32, h, acc);
    return;
  }
  if (!kvalid) return;
  int j, n;
  if (kv < a.Ns) {
    j = kv / a.b;
    n = j == a.nb_s - 1 ? a.tail_s : a.b;
  } else {
    const int u = (kv - a.Ns) / a.b;
    j = a.nb_s + u;
    n = a.kept[(long long)bh * a.kc + u] == a.nb_c - 1 ? a.tail_c : a.b;
  }
  const float inv_n = 1.0f / (float)n;
  const float* pb = a.dkvbar + ((long long)bh * a.mk_pad + j) * 2 * D + D;
  bf16_t* out = (bf16_t*)a.dV + rm_head(a.rmv, bh) + (long long)krow * a.rmv.sn;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * t + 8 * g + 4 * h;
      const f32x4 bb = *(const f32x4*)(pb + d0);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(acc[t][4 * g + e], 1.0f, bb[e] * inv_n);
      *(u32x2*)(out + d0) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
}

// dK of the full route at d = 128, on the schedule of isa_bwd_dv_pp_kernel
// with K and V of the key in registers:
//   X_j  dK^T += Q(j-1)^T dS(j-1), then S(j) = Q(j) K^T and dP(j) = dO(j) V^T
//   Y_j  loads of Q(j+3), dO(j+3), lse and D of tile j+3 and the row table of
//        tile j+6; dS(j) = P(j) (dP(j) - D) in bf16, P = exp2(S sc - lse)
// Q(t) is read in X_t and X_{t+1}, so its ring has five stages (stage t % 5,
// refilled in Y_{t-3} after the last read of Q(t-5) in X_{t-4}); dO(t) is
// read in X_t only (four stages, as K in the forward kernel).  lse and D of
// tile t come to slot t % 4 by waves 0 and 1 in Y_{t-3}.
#ifndef ISA_BWD_DK_LOOKAHEAD
#define ISA_BWD_DK_LOOKAHEAD 3
#endif
__global__ __launch_bounds__(512) void isa_bwd_dk_pp_kernel(BwdArgs a) {
  typedef bf16x8 Op;
  constexpr int D = 128, BN = 64, NQ = 5, NG = 4, ES = 2;
  constexpr int RB = D * 2, TB = BN * RB, NT = D / 32;
  static_assert(kBwdKeys == 256, "keys per workgroup");

  __shared__ __attribute__((aligned(1024))) char smem[(NQ + NG) * TB];   // Q ring, then dO ring
  __shared__ __attribute__((aligned(16))) int stab[8][4][64];            // per-wave row-table ring
  __shared__ __attribute__((aligned(256))) float sld[2][4][BN];          // lse, D rings

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const KvItem item = kv_item(a, a.n_rowtab / BN);
  if (!item.live) return;
  const int bh = item.bh, kt = item.kt;

  // ---- this lane's key (as isa_bwd_dkdv_kernel)
  const int kv = kt * kBwdKeys + w * 32 + l32;
  const int n_keys = a.Ns + (int)a.ctx_tok;
  int krow;
  if (kv < a.Ns) krow = kv;
  else if (kv < n_keys) krow = a.ctx_rows[(long long)bh * a.ctx_tok + (kv - a.Ns)];
  else krow = -1;
  const bool kvalid = krow >= 0;
  krow = kvalid ? krow : 0;
  Op kB[D / 16], vB[D / 16];
  {
    const char* Kg = (const char*)a.K + (rm_head(a.rmk, bh) + (long long)krow * a.rmk.sn) * ES;
    const char* Vg = (const char*)a.V + (rm_head(a.rmv, bh) + (long long)krow * a.rmv.sn) * ES;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kB[s] = *(const Op*)(Kg + (16 * s + 8 * h) * ES);
      vB[s] = *(const Op*)(Vg + (16 * s + 8 * h) * ES);
    }
  }

  const int nt = item.nq;   // row tiles of the route in the item, from item.q0
  const char* Qg = (const char*)a.Q + rm_head(a.rmq, bh) * 2;
  const char* Gg = (const char*)a.dO + rm_head(a.rmo, bh) * 2;
  const unsigned qrs = (unsigned)a.rmq.sn * 2u, grs = (unsigned)a.rmo.sn * 2u;   // row steps in bytes
  const int* tab = a.rrow + (long long)bh * a.n_rowtab + item.q0 * BN;
  const float* lseg = a.rlse + (long long)bh * a.n_rowtab + item.q0 * BN;
  const float* delg = a.rdel + (long long)bh * a.n_rowtab + item.q0 * BN;

  const int lrow0 = 32 * grp + 8 * wg + (lane >> 4);
  struct Rows { int r[2]; };
  const unsigned stab_w = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_char*)&stab[0][0][0]) +
                          __builtin_amdgcn_readfirstlane(w) * (unsigned)sizeof(stab[0]);
  auto fetch_rows = [&](int j, int tile) {
    const int k = 4 * (lane & 1) + ((lane >> 1) & 3);
    dma4(stab_w + (unsigned)(j & 3) * (unsigned)sizeof(stab[0][0]), tab, (unsigned)(tile * BN + 32 * grp + 8 * wg + k) * 4u);
  };
  auto rows_of = [&](int j) -> Rows {
    const int2 v = *(const int2*)&stab[w][j & 3][2 * (lane >> 4)];
    return Rows{{v.x, v.y}};
  };
  const unsigned lds_q = (unsigned)(size_t)(lds_char*)smem;
  const unsigned lds_g = lds_q + NQ * TB;
  const unsigned lds_ld = (unsigned)(size_t)(lds_char*)&sld[0][0][0];
  unsigned lchunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) lchunk[i] = (unsigned)(((lane & 15) ^ lds_swz(lrow0 + 4 * i)) * 16);
  const unsigned wrow = __builtin_amdgcn_readfirstlane((32 * grp + 8 * wg) * RB);
  auto issue_tile = [&](unsigned ring, int stage, const char* base, Rows rows, unsigned rs) {
    const unsigned d0 = ring + wrow + (unsigned)stage * TB;
    dma16x2(d0, d0 + 4 * RB, base, __umul24((unsigned)rows.r[0], rs) + lchunk[0],
            __umul24((unsigned)rows.r[1], rs) + lchunk[1]);
  };
  auto issue_ld = [&](int slot, int tile) {   // lse by wave 0, D by wave 1
    if (w == 0) dma4(lds_ld + (unsigned)slot * BN * 4, lseg + tile * BN, (unsigned)lane * 4u);
    if (w == 1) dma4(lds_ld + (unsigned)(4 + slot) * BN * 4, delg + tile * BN, (unsigned)lane * 4u);
  };

  // operand offsets within a tile: rows 32*ti + l32, chunk 2s + h (Q, dO);
  // Q^T transpose reads at rows 16s + 4h + m/4 (+8), d = 32t + 16(g%2) + 4(m%4)
  int koff[8], voff[NT][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = l32 * RB + ((((2 * s + h) ^ lds_swz(l32)) * 16));
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int m = lane & 15;
      const int kr = 4 * h + (m >> 2) + 8 * hi;
      const int c = 4 * t + 2 * ((lane >> 4) & 1) + ((m & 3) >> 1);
      voff[t][hi] = kr * RB + ((c ^ lds_swz(kr)) * 16) + 8 * (m & 1);
    }

  struct STile { f32x16 t[2]; };
  struct PTile { Op p[4]; };
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  const float sc = a.scale_log2;

  // X phase: 16 MFMAs of Q^T dS, then 16 of Q K^T and 16 of dO V^T
  auto x_phase = [&](int qprev, const PTile& dS, int qcur, int gcur, STile& S, STile& dP) {
    constexpr int LA = ISA_BWD_DK_LOOKAHEAD;
    const lds_char* Ts = (const lds_char*)smem + qprev * TB;
    const lds_char* Qs = (const lds_char*)smem + qcur * TB;
    const lds_char* Gs = (const lds_char*)smem + (NQ + gcur) * TB;
    Op opv[16], opk[32];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ts + voff[t][0] + 16 * q * RB));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ts + voff[t][1] + 16 * q * RB));
        opv[4 * t + q] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        opk[2 * q + ti] = *(const Op*)(Qs + koff[q] + 32 * ti * RB);
        opk[16 + 2 * q + ti] = *(const Op*)(Gs + koff[q] + 32 * ti * RB);
      }
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m >> 2] = mma32(opv[m], dS.p[m & 3], acc[m >> 2]);
    S.t[0] = f32x16{};
    S.t[1] = f32x16{};
    dP.t[0] = f32x16{};
    dP.t[1] = f32x16{};
#pragma unroll
    for (int m = 0; m < 16; ++m) S.t[m & 1] = mma32(opk[m], kB[m >> 1], S.t[m & 1]);
#pragma unroll
    for (int m = 0; m < 16; ++m) dP.t[m & 1] = mma32(opk[16 + m], vB[m >> 1], dP.t[m & 1]);
    pp_issue_order<LA, 16, 32>();
  };
  // dS = P (dP - D), P = exp2(S sc - lse); rows of reg r of tile ti: 32 ti + 8 (r/4) + 4h + r%4
  auto dsoft = [&](int slot, const STile& S, const STile& dP) -> PTile {
    PTile dS;
    const float* ls = sld[0][slot];
    const float* ds = sld[1][slot];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)(ls + 32 * ti + 8 * g + 4 * h);
        const f32x4 d4 = *(const f32x4*)(ds + 32 * ti + 8 * g + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(S.t[ti][r], sc, -l4[e]));
          dS.p[2 * ti + (r >> 3)][r & 7] = (__bf16)(p * (dP.t[ti][r] - d4[e]));
        }
      }
    return dS;
  };
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  auto cl = [&](int j) { return min(j, nt - 1); };
  if (nt > 0) {
    Rows rk;   // rows of tile j+3 entering step j
    {
      fetch_rows(cl(0), cl(0));
      fetch_rows(cl(1), cl(1));
      fetch_rows(cl(2), cl(2));
      fetch_rows(cl(3), cl(3));
      __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
      const Rows r0 = rows_of(cl(0)), r1 = rows_of(cl(1)), r2 = rows_of(cl(2));
      rk = rows_of(cl(3));
      issue_tile(lds_q, 0, Qg, r0, qrs);
      issue_tile(lds_g, 0, Gg, r0, grs);
      issue_tile(lds_q, 1, Qg, r1, qrs);
      issue_tile(lds_g, 1, Gg, r1, grs);
      issue_tile(lds_q, 2, Qg, r2, qrs);
      issue_tile(lds_g, 2, Gg, r2, grs);
      issue_ld(0, cl(0));
      issue_ld(1, cl(1));
      issue_ld(2, cl(2));
      fetch_rows(cl(4), cl(4));
      fetch_rows(cl(5), cl(5));
      // Q stage 4 is first loaded in step 1; step 0 reads it as zeros
      u32x4* qz = (u32x4*)(smem + 4 * TB);
#pragma unroll
      for (int q = 0; q < TB / (16 * 512); ++q) qz[tid + 512 * q] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    }
    phase_barrier();
    if (grp == 1) phase_barrier();   // group 1 runs one phase behind group 0
    STile S = {}, dP = {};
    PTile dS = {};
    int q_prev = 4, q_cur = 0;   // Q stages of tiles j-1 and j
    for (int j = 0; j <= nt; ++j) {
      const int Z = j & 3;
      __builtin_amdgcn_s_setprio(3);
      x_phase(q_prev, dS, q_cur, Z, S, dP);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
      // Y_j
      const int q3 = q_cur + 3 < NQ ? q_cur + 3 : q_cur + 3 - NQ;   // (j + 3) % 5
      issue_tile(lds_q, q3, Qg, rk, qrs);
      issue_tile(lds_g, (Z + 3) & 3, Gg, rk, grs);
      issue_ld((Z + 3) & 3, cl(j + 3));
      const Rows rn = rows_of(cl(j + 4));
      fetch_rows(cl(j + 6), cl(j + 6));
      if (j < nt) dS = dsoft(Z, S, dP);
      rk = rn;
      q_prev = q_cur;
      q_cur = q_cur + 1 < NQ ? q_cur + 1 : 0;
      // the loads of Y_{j-1} have landed before the barrier that closes Y_j
      if (w < 2) __builtin_amdgcn_s_waitcnt(0x0f76);   // vmcnt(6)
      else __builtin_amdgcn_s_waitcnt(0x0f75);         // vmcnt(5)
      phase_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // no load into this workgroup's LDS outlives it
    if (grp == 0) phase_barrier();   // balances group 1's extra barrier
  }

  // ---- epilogue: dK of the key (scaled by 1/sqrt d) plus the pooled share
  // of its block (as isa_bwd_dkdv_kernel); lane holds key kv, d = 32 t + 8 g + 4 h + e.
  // A part of a cut item leaves its raw sum to the merge.
  if (item.slot >= 0) {
    kv_store_part<NT>(a, item.slot, w, l32, h, acc);
    return;
  }
  if (!kvalid) return;
  int j, n;
  if (kv < a.Ns) {
    j = kv / a.b;
    n = j == a.nb_s - 1 ? a.tail_s : a.b;
  } else {
    const int u = (kv - a.Ns) / a.b;
    j = a.nb_s + u;
    n = a.kept[(long long)bh * a.kc + u] == a.nb_c - 1 ? a.tail_c : a.b;
  }
  const float inv_n = 1.0f / (float)n;
  const float* pb = a.dkvbar + ((long long)bh * a.mk_pad + j) * 2 * D;
  bf16_t* out = (bf16_t*)a.dK + rm_head(a.rmk, bh) + (long long)krow * a.rmk.sn;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * t + 8 * g + 4 * h;
      const f32x4 bb = *(const f32x4*)(pb + d0);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(acc[t][4 * g + e], a.inv_sqrt_d, bb[e] * inv_n);
      *(u32x2*)(out + d0) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
}

// dQ of the full route at d = 128 on the ping-pong schedule of the forward
// flash kernel (rows fixed: 8 waves x 32 query rows, Q, dO, lse and D of
// the row in registers; key tiles of 64 streamed, split-K as the forward):
//   X_j  dQ^T += K(j-1)^T dS(j-1)^T, then S(j)^T = K(j) Q^T and
//        dP(j)^T = V(j) dO^T
//   Y_j  loads of K(j+3), V(j+3) and the key-row table of tile j+6;
//        dS = P (dP - D), P = exp2(S log2(e)/sqrt(d) - lse) (one fma, as the
//        dK and dV kernels; isa_bwd_dq_kernel rounds the product first),
//        keys past the route's last valid key masked
// K(t) is read in X_t and X_{t+1} (five-stage ring, as Q in the dK kernel);
// V(t) in X_t only (four stages).
#ifndef ISA_BWD_DQ_LOOKAHEAD
#define ISA_BWD_DQ_LOOKAHEAD 3
#endif
__global__ __launch_bounds__(512) void isa_bwd_dq_pp_kernel(BwdArgs a) {
  typedef bf16x8 Op;
  constexpr int D = 128, BN = 64, BM = 256, NK = 5, NV = 4, ES = 2;
  constexpr int RB = D * 2, TB = BN * RB, NT = D / 32;
  static_assert(BM == kFlashRows, "tile mapping");

  __shared__ __attribute__((aligned(1024))) char smem[(NK + NV) * TB];   // K ring, then V ring
  __shared__ __attribute__((aligned(16))) int stab[8][4][64];            // per-wave key-table ring

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  // Work item (head bh, row tile rt) over all key tiles, or, in the cut last
  // round, over the key range of its part (cut_item: an XCD's workgroups take
  // whole row tiles of their own, consecutive row tiles of a head sharing its
  // K/V in L2, then their share of the parts)
  const int n_keys = a.Ns + (int)a.ctx_tok;
  const int ntiles = (n_keys + BN - 1) / BN;
  const CutItem item = cut_item(a.n_wg, a.dq_rounds, a.dq_rest, a.dq_parts, ntiles);
  if (!item.live) return;
  const int bh = item.id / a.row_tiles;
  const int rt = item.id - bh * a.row_tiles;

  const long long vrow = (long long)rt * BM + w * 32 + l32;
  const int qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  Op qB[D / 16], gB[D / 16];
  float lse_r = INFINITY, del_r = 0.f;  // rows off the route: p = 0
  {
    const long long r = (long long)bh * a.Ns + (qrow < 0 ? 0 : qrow);
    const long long qr = qrow < 0 ? 0 : qrow;
    const bf16_t* qp = (const bf16_t*)a.Q + rm_head(a.rmq, bh) + qr * a.rmq.sn + 8 * h;
    const bf16_t* gp = (const bf16_t*)a.dO + rm_head(a.rmo, bh) + qr * a.rmo.sn + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qB[s] = *(const Op*)(qp + 16 * s);
      gB[s] = *(const Op*)(gp + 16 * s);
    }
    if (qrow >= 0) {
      lse_r = a.lse[r];
      del_r = a.delta[r];
    }
  }

  const bool tail_kept = a.kc > 0 && a.kept[(long long)bh * a.kc + a.kc - 1] == a.nb_c - 1;
  const int n_valid = n_keys - (tail_kept ? a.b - a.tail_c : 0);
  const int t_begin = item.r0;
  const int nt = item.n;

  const char* Kg = (const char*)a.K + rm_head(a.rmk, bh) * 2;
  const char* Vg = (const char*)a.V + rm_head(a.rmv, bh) * 2;
  const unsigned krs = (unsigned)a.rmk.sn * 2u, vrs = (unsigned)a.rmv.sn * 2u;   // row steps in bytes
  const int* tab = a.key_rows + (long long)bh * a.n_keytab;

  const int lrow0 = 32 * grp + 8 * wg + (lane >> 4);
  struct Rows { int r[2]; };
  const unsigned stab_w = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_char*)&stab[0][0][0]) +
                          __builtin_amdgcn_readfirstlane(w) * (unsigned)sizeof(stab[0]);
  auto fetch_rows = [&](int j, int tile) {
    const int k = 4 * (lane & 1) + ((lane >> 1) & 3);
    dma4(stab_w + (unsigned)(j & 3) * (unsigned)sizeof(stab[0][0]), tab, (unsigned)(tile * BN + 32 * grp + 8 * wg + k) * 4u);
  };
  auto rows_of = [&](int j) -> Rows {
    const int2 v = *(const int2*)&stab[w][j & 3][2 * (lane >> 4)];
    return Rows{{v.x, v.y}};
  };
  const unsigned lds_k = (unsigned)(size_t)(lds_char*)smem;
  const unsigned lds_v = lds_k + NK * TB;
  unsigned lchunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) lchunk[i] = (unsigned)(((lane & 15) ^ lds_swz(lrow0 + 4 * i)) * 16);
  const unsigned wrow = __builtin_amdgcn_readfirstlane((32 * grp + 8 * wg) * RB);
  auto issue_tile = [&](unsigned ring, int stage, const char* base, Rows rows, unsigned rs) {
    const unsigned d0 = ring + wrow + (unsigned)stage * TB;
    dma16x2(d0, d0 + 4 * RB, base, __umul24((unsigned)rows.r[0], rs) + lchunk[0],
            __umul24((unsigned)rows.r[1], rs) + lchunk[1]);
  };

  int koff[8], voff[NT][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = l32 * RB + ((((2 * s + h) ^ lds_swz(l32)) * 16));
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int m = lane & 15;
      const int kr = 4 * h + (m >> 2) + 8 * hi;
      const int c = 4 * t + 2 * ((lane >> 4) & 1) + ((m & 3) >> 1);
      voff[t][hi] = kr * RB + ((c ^ lds_swz(kr)) * 16) + 8 * (m & 1);
    }

  struct STile { f32x16 t[2]; };
  struct PTile { Op p[4]; };
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  const float sc = a.scale_log2;

  auto x_phase = [&](int kprev, const PTile& dS, int kcur, int vcur, STile& S, STile& dP) {
    constexpr int LA = ISA_BWD_DQ_LOOKAHEAD;
    const lds_char* Ts = (const lds_char*)smem + kprev * TB;
    const lds_char* Ks = (const lds_char*)smem + kcur * TB;
    const lds_char* Vs = (const lds_char*)smem + (NK + vcur) * TB;
    Op opv[16], opk[32];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ts + voff[t][0] + 16 * q * RB));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ts + voff[t][1] + 16 * q * RB));
        opv[4 * t + q] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        opk[2 * q + ti] = *(const Op*)(Ks + koff[q] + 32 * ti * RB);
        opk[16 + 2 * q + ti] = *(const Op*)(Vs + koff[q] + 32 * ti * RB);
      }
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m >> 2] = mma32(opv[m], dS.p[m & 3], acc[m >> 2]);
    S.t[0] = f32x16{};
    S.t[1] = f32x16{};
    dP.t[0] = f32x16{};
    dP.t[1] = f32x16{};
#pragma unroll
    for (int m = 0; m < 16; ++m) S.t[m & 1] = mma32(opk[m], qB[m >> 1], S.t[m & 1]);
#pragma unroll
    for (int m = 0; m < 16; ++m) dP.t[m & 1] = mma32(opk[16 + m], gB[m >> 1], dP.t[m & 1]);
    pp_issue_order<LA, 16, 32>();
  };
  // dS = P (dP - D) with P = exp2(S sc - lse); keys of reg r of tile ti:
  // 32 ti + 8 (r/4) + 4h + r%4
  auto dsoft = [&](int j, STile& S, const STile& dP) -> PTile {
    const int t0 = (t_begin + j) * BN;
    if (t0 + BN > n_valid) {
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3) >= n_valid) S.t[ti][r] = -INFINITY;
    }
    PTile dS;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S.t[ti][r], sc, -lse_r));
        dS.p[2 * ti + (r >> 3)][r & 7] = (__bf16)(p * (dP.t[ti][r] - del_r));
      }
    return dS;
  };
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  auto cl = [&](int j) { return min(j, nt - 1); };
  auto tl = [&](int j) { return t_begin + cl(j); };
  if (nt > 0) {
    Rows rk;   // rows of tile j+3 entering step j
    {
      fetch_rows(cl(0), tl(0));
      fetch_rows(cl(1), tl(1));
      fetch_rows(cl(2), tl(2));
      fetch_rows(cl(3), tl(3));
      __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
      const Rows r0 = rows_of(cl(0)), r1 = rows_of(cl(1)), r2 = rows_of(cl(2));
      rk = rows_of(cl(3));
      issue_tile(lds_k, 0, Kg, r0, krs);
      issue_tile(lds_v, 0, Vg, r0, vrs);
      issue_tile(lds_k, 1, Kg, r1, krs);
      issue_tile(lds_v, 1, Vg, r1, vrs);
      issue_tile(lds_k, 2, Kg, r2, krs);
      issue_tile(lds_v, 2, Vg, r2, vrs);
      fetch_rows(cl(4), tl(4));
      fetch_rows(cl(5), tl(5));
      // K stage 4 is first loaded in step 1; step 0 reads it as zeros
      u32x4* kz = (u32x4*)(smem + 4 * TB);
#pragma unroll
      for (int q = 0; q < TB / (16 * 512); ++q) kz[tid + 512 * q] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    }
    phase_barrier();
    if (grp == 1) phase_barrier();   // group 1 runs one phase behind group 0
    STile S = {}, dP = {};
    PTile dS = {};
    int k_prev = 4, k_cur = 0;   // K stages of tiles j-1 and j
    for (int j = 0; j <= nt; ++j) {
      const int Z = j & 3;
      __builtin_amdgcn_s_setprio(3);
      x_phase(k_prev, dS, k_cur, Z, S, dP);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
      // Y_j
      const int k3 = k_cur + 3 < NK ? k_cur + 3 : k_cur + 3 - NK;   // (j + 3) % 5
      issue_tile(lds_k, k3, Kg, rk, krs);
      issue_tile(lds_v, (Z + 3) & 3, Vg, rk, vrs);
      const Rows rn = rows_of(cl(j + 4));
      fetch_rows(cl(j + 6), tl(j + 6));
      if (j < nt) dS = dsoft(j, S, dP);
      rk = rn;
      k_prev = k_cur;
      k_cur = k_cur + 1 < NK ? k_cur + 1 : 0;
      // the loads of Y_{j-1} have landed before the barrier that closes Y_j
      __builtin_amdgcn_s_waitcnt(0x0f75);   // vmcnt(5)
      phase_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // no load into this workgroup's LDS outlives it
    if (grp == 0) phase_barrier();   // balances group 1's extra barrier
  }

  // ---- epilogue (as isa_bwd_dq_kernel): dQ of a whole row tile, or the raw
  // sum of a part of a cut one ([slot][256 rows][D], merged by
  // isa_bwd_dq_merge_kernel)
  if (qrow < 0 && item.slot < 0) return;
  if (item.slot < 0) {
    bf16_t* op = (bf16_t*)a.dQ + rm_head(a.rmq, bh) + (long long)qrow * a.rmq.sn;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& c = acc[t];
        const float sd = a.inv_sqrt_d;
        *(u32x2*)(op + 32 * t + 8 * g + 4 * h) = u32x2{pack_bf16x2(c[4 * g] * sd, c[4 * g + 1] * sd),
                                                       pack_bf16x2(c[4 * g + 2] * sd, c[4 * g + 3] * sd)};
      }
  } else {
    float* pp = a.part_dq + ((long long)item.slot * BM + w * 32 + l32) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& c = acc[t];
        *(f32x4*)(pp + 32 * t + 8 * g + 4 * h) = f32x4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
      }
  }
}

// dK (DK) or dV of the keys of the cut items of the full-route dK / dV
// kernels: the sum of their parts in part order, then those kernels'
// epilogue (dK scaled by 1/sqrt d, plus the pooled share of the key's block,
// in bf16).  Four d per thread, D / 4 threads per key.
template <bool DK>
__global__ __launch_bounds__(256) void isa_bwd_kv_merge_kernel(BwdArgs a) {
  constexpr int D = 128, TPR = D / 4, RPB = 256 / TPR;
  const long long gid = (long long)blockIdx.x * RPB + threadIdx.x / TPR;   // key of the cut items
  const int e = (threadIdx.x % TPR) * 4;
  if (gid >= (long long)a.kv_rest * kBwdKeys) return;
  const int sp = (int)(gid / kBwdKeys), r = (int)(gid - (long long)sp * kBwdKeys);
  const int id = kCUs * a.kv_rounds + sp;
  const int bh = id / a.key_tiles, kt = id - bh * a.key_tiles;
  const int kv = kt * kBwdKeys + r;
  const int n_keys = a.Ns + (int)a.ctx_tok;
  int krow;
  if (kv < a.Ns) krow = kv;
  else if (kv < n_keys) krow = a.ctx_rows[(long long)bh * a.ctx_tok + (kv - a.Ns)];
  else krow = -1;
  if (krow < 0) return;
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.kv_parts; ++p)
    sum += *(const f32x4*)(a.part_kv + ((long long)(sp * a.kv_parts + p) * kBwdKeys + r) * D + e);
  int j, n;
  if (kv < a.Ns) {
    j = kv / a.b;
    n = j == a.nb_s - 1 ? a.tail_s : a.b;
  } else {
    const int u = (kv - a.Ns) / a.b;
    j = a.nb_s + u;
    n = a.kept[(long long)bh * a.kc + u] == a.nb_c - 1 ? a.tail_c : a.b;
  }
  const float inv_n = 1.0f / (float)n;
  const f32x4 bb = *(const f32x4*)(a.dkvbar + ((long long)bh * a.mk_pad + j) * 2 * D + (DK ? 0 : D) + e);
  const float sd = DK ? a.inv_sqrt_d : 1.0f;
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = fmaf(sum[i], sd, bb[i] * inv_n);
  bf16_t* out = DK ? (bf16_t*)a.dK + rm_head(a.rmk, bh) + (long long)krow * a.rmk.sn
                   : (bf16_t*)a.dV + rm_head(a.rmv, bh) + (long long)krow * a.rmv.sn;
  *(u32x2*)(out + e) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// dkbar, dvbar = sum of the pooled partials over splits, in split order
// (zero when there are no Taylor rows: nsplit = 0).
template <int D>
__global__ __launch_bounds__(256) void isa_bwd_dkv_reduce_kernel(BwdArgs a) {
  const long long n = a.BH * a.mk_pad * 2 * D / 4;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < a.nsplit; ++k) s += *(const f32x4*)(a.part_dkv + ((long long)k * n + i) * 4);
  *(f32x4*)(a.dkvbar + i * 4) = s;
}

// Zeroes the dK, dV rows of the context blocks that were pruned (B4).
template <int D>
__global__ __launch_bounds__(256) void isa_bwd_zero_pruned_kernel(BwdArgs a) {
  const int c = blockIdx.x;
  const long long bh = blockIdx.y;
  const int* kp = a.kept + bh * a.kc;
  int lo = 0, hi = a.kc;  // binary search in the ascending kept list
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (kp[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  if (lo < a.kc && kp[lo] == c) return;
  const int r0 = a.Ns + c * a.b;
  const int nr = c == a.nb_c - 1 ? a.tail_c : a.b;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const long long kh = rm_head(a.rmk, bh), vh = rm_head(a.rmv, bh);
  for (int q = threadIdx.x; q < nr * CPR; q += 256) {
    const long long r = r0 + q / CPR, e = (q % CPR) * 8;
    *(u32x4*)((bf16_t*)a.dK + kh + r * a.rmk.sn + e) = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)((bf16_t*)a.dV + vh + r * a.rmv.sn + e) = u32x4{0u, 0u, 0u, 0u};
  }
}

// ---------------------------------------------------------------------------

static BwdArgs bwd_args(const Layout& L, const BwdLayout& W, const BwdBufs& B) {
  BwdArgs a = {};
  a.Q = B.Q; a.K = B.K; a.V = B.V; a.O = B.O; a.dO = B.dO;
  a.dQ = B.dQ; a.dK = B.dK; a.dV = B.dV;
  a.rmq = L.q; a.rmk = L.k; a.rmv = L.v; a.rmo = L.o;
  a.lse = (const float*)(B.ws + L.off_lse);
  a.delta = (float*)(B.bws + W.off_delta);
  a.ctx_rows = (const int*)(B.ws + L.off_ctxrows);
  a.kept = (const int*)(B.ws + L.off_kept);
  a.ctx_tok = L.ctx_tok;
  a.kc = L.kc; a.nb_c = L.nb_c; a.b = L.b; a.tail_s = L.tail_s; a.tail_c = L.tail_c;
  a.pkhi = B.ws + L.off_pkhi; a.pklo = B.ws + L.off_pklo; a.pv = B.ws + L.off_pv;
  a.pbias = (const float*)(B.ws + L.off_pbias);
  a.mk = L.mk; a.mk_pad = L.mk_pad;
  a.nb_s = L.nb_s;
  a.part_dq = (float*)(B.bws + W.off_part_dq);
  a.part_kv = (float*)(B.bws + W.off_part_kv);
  a.part_dkv = (float*)(B.bws + W.off_part_dkv);
  a.dkvbar = (float*)(B.bws + W.off_dkvbar);
  a.nsplit = 1;
  a.Ns = L.Ns; a.Nk = L.Nk;
  a.BH = L.BH;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)L.d));
  a.inv_sqrt_d = (float)(1.0 / sqrt((double)L.d));
  a.key_rows = (const int*)(B.ws + L.off_keyrows);
  a.n_keytab = L.n_keytab;
  a.rrow = (int*)(B.bws + W.off_rrow);
  a.rlse = (float*)(B.bws + W.off_rlse);
  a.rdel = (float*)(B.bws + W.off_rdel);
  a.n_rowtab = W.n_rowtab;
  return a;
}

template <int D>
static hipError_t bwd_t(const Layout& L, const BwdLayout& W, const BwdBufs& B, BwdWhat what, hipStream_t s) {
  BwdArgs a = bwd_args(L, W, B);
  const int* fullq = (const int*)(B.ws + L.off_fullq);
  const int* taylq = (const int*)(B.ws + L.off_taylq);
  switch (what) {
    case BwdWhat::kDelta: {
      constexpr int RPB = 256 / (D / 8);
      const long long rows = L.BH * L.Ns;
      a.delta_wgs = (rows + RPB - 1) / RPB;
      a.q_list = fullq; a.q_k = L.kq;
      const long long rwgs = (L.BH * W.n_rowtab + RPB - 1) / RPB;
      hipLaunchKernelGGL((isa_bwd_delta_kernel<D>), dim3((unsigned)(a.delta_wgs + rwgs)), dim3(256), 0, s, a);
      break;
    }
    case BwdWhat::kDkPooled:
    case BwdWhat::kDvPooled: {
      if (L.taylor_rows == 0) return hipSuccess;
      a.q_list = taylq; a.q_k = L.nb_s - L.kq; a.n_rows = L.taylor_rows;
      a.nsplit = W.dkv_splits;
      a.key_tiles = W.dkv_key_tiles;
      const long long nwg = L.BH * a.key_tiles * a.nsplit;
      a.n_wg = (int)nwg;
      if (what == BwdWhat::kDkPooled)
        hipLaunchKernelGGL((isa_bwd_dkdv_kernel<D, true, true>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((isa_bwd_dkdv_kernel<D, true, false>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      break;
    }
    case BwdWhat::kDkvReduce: {
      a.nsplit = L.taylor_rows == 0 ? 0 : W.dkv_splits;
      const long long n = L.BH * L.mk_pad * 2 * D / 4;
      hipLaunchKernelGGL((isa_bwd_dkv_reduce_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
      break;
    }
    case BwdWhat::kDkFull:
    case BwdWhat::kDvFull: {
      a.q_list = fullq; a.q_k = L.kq; a.n_rows = L.full_rows;
      a.key_tiles = (int)((L.Ns + L.ctx_tok + kBwdKeys - 1) / kBwdKeys);
      long long nwg = L.BH * a.key_tiles;
      const bool dk = what == BwdWhat::kDkFull;
      // the ping-pong kernels cut the last, part-filled round (W.kv_parts)
      const bool pp = D == 128 && (dk ? kUseDkPP : kUseDvPP);
      const bool cut = pp && W.kv_parts > 0;
      if (cut) {
        if ((long long)kCUs * W.kv_rounds + W.kv_rest != nwg) return hipErrorInvalidValue;
        a.kv_rounds = W.kv_rounds;
        a.kv_rest = W.kv_rest;
        a.kv_parts = W.kv_parts;
        nwg = 8 * ((long long)(kCUs / 8) * W.kv_rounds + ((long long)W.kv_rest * W.kv_parts + 7) / 8);
      }
      a.n_wg = (int)nwg;
      if (dk && pp)
        hipLaunchKernelGGL(isa_bwd_dk_pp_kernel, dim3((unsigned)nwg), dim3(512), 0, s, a);
      else if (dk)
        hipLaunchKernelGGL((isa_bwd_dkdv_kernel<D, false, true>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      else if (pp)
        hipLaunchKernelGGL(isa_bwd_dv_pp_kernel, dim3((unsigned)nwg), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((isa_bwd_dkdv_kernel<D, false, false>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      if (cut) {
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        const unsigned mg = (unsigned)((long long)W.kv_rest * kBwdKeys / (256 / (128 / 4)));
        if (dk) hipLaunchKernelGGL(isa_bwd_kv_merge_kernel<true>, dim3(mg), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(isa_bwd_kv_merge_kernel<false>, dim3(mg), dim3(256), 0, s, a);
      }
      break;
    }
    case BwdWhat::kZeroPruned: {
      if (L.nb_c == 0 || L.kc == L.nb_c) return hipSuccess;
      hipLaunchKernelGGL((isa_bwd_zero_pruned_kernel<D>), dim3((unsigned)L.nb_c, (unsigned)L.BH), dim3(256), 0, s, a);
      break;
    }
    case BwdWhat::kDqFull:
    case BwdWhat::kDqPooled: {
      const bool full = what == BwdWhat::kDqFull;
      if (full && L.full_rows == 0) return hipSuccess;
      if (!full && L.taylor_rows == 0) return hipSuccess;
      a.q_list = full ? fullq : taylq;
      a.q_k = full ? L.kq : L.nb_s - L.kq;
      a.n_rows = full ? L.full_rows : L.taylor_rows;
      a.nsplit = full ? L.full_splits : 1;
      a.row_tiles = (int)((a.n_rows + kFlashRows - 1) / kFlashRows);
      const long long keys = full ? (long long)L.Ns + L.ctx_tok : (long long)L.mk_pad;
      const int ntiles = (int)((keys + 63) / 64);
      a.tiles_per_split = (ntiles + a.nsplit - 1) / a.nsplit;
      long long nwg = (long long)a.row_tiles * L.BH * a.nsplit;
      const bool pp = full && D == 128 && kUseDqPP;
      if (pp) {
        // whole row tiles, the part-filled last round cut into W.dq_parts key ranges
        const long long items = (long long)a.row_tiles * L.BH;
        if ((long long)kCUs * W.dq_rounds + W.dq_rest != items) return hipErrorInvalidValue;
        a.dq_rounds = W.dq_rounds;
        a.dq_rest = W.dq_rest;
        a.dq_parts = W.dq_parts;
        nwg = W.dq_parts > 0 ? 8 * ((long long)(kCUs / 8) * W.dq_rounds + ((long long)W.dq_rest * W.dq_parts + 7) / 8)
                             : items;
      }
      a.n_wg = (int)nwg;
      if (pp)
        hipLaunchKernelGGL(isa_bwd_dq_pp_kernel, dim3((unsigned)nwg), dim3(512), 0, s, a);
      else if (full)
        hipLaunchKernelGGL((isa_bwd_dq_kernel<D, false>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((isa_bwd_dq_kernel<D, true>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      break;
    }
    case BwdWhat::kDqMerge: {
      const bool pp = D == 128 && kUseDqPP;   // (as kDqFull)
      if (L.full_rows == 0 || (pp ? W.dq_parts == 0 : L.full_splits <= 1)) return hipSuccess;
      a.q_list = fullq; a.q_k = L.kq; a.n_rows = L.full_rows;
      a.nsplit = L.full_splits;
      a.row_tiles = (int)((L.full_rows + kFlashRows - 1) / kFlashRows);
      constexpr int RPB = 256 / (D / 4);
      long long rows = (long long)a.row_tiles * kFlashRows * L.BH;
      if (pp) {
        a.dq_rounds = W.dq_rounds;
        a.dq_rest = W.dq_rest;
        a.dq_parts = W.dq_parts;
        rows = (long long)W.dq_rest * kFlashRows;
      }
      hipLaunchKernelGGL((isa_bwd_dq_merge_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a);
      break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_backward(const Layout& L, const BwdLayout& W, const BwdBufs& B, BwdWhat what, hipStream_t s) {
  return L.d == 128 ? bwd_t<128>(L, W, B, what, s) : bwd_t<64>(L, W, B, what, s);
}

}  // namespace isa
