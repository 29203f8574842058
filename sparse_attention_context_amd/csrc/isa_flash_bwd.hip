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
};

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i, 8 elements per lane, D/8 lanes per row.

template <int D>
__global__ __launch_bounds__(256) void isa_bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int e = (threadIdx.x % LPR) * 8;
  const bool ok = row < a.BH * a.Ns;
  float s = 0.f;
  if (ok) {
    const u32x4 o = *(const u32x4*)((const bf16_t*)a.O + row * D + e);
    const u32x4 g = *(const u32x4*)((const bf16_t*)a.dO + row * D + e);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s += __uint_as_float(o[i] << 16) * __uint_as_float(g[i] << 16) +
           __uint_as_float(o[i] & 0xffff0000u) * __uint_as_float(g[i] & 0xffff0000u);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);
  if (ok && e == 0) a.delta[row] = s;
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
  const int lid = xcd_remap(blockIdx.x, a.n_wg);
  const int split = lid % a.nsplit;
  const int rest = lid / a.nsplit;
  const int bh = rest / a.row_tiles;
  const int rt = rest - bh * a.row_tiles;

  const long long vrow = (long long)rt * BM + w * 32 + l32;
  const int qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  Op qB[D / 16], gB[D / 16];
  float lse_r = INFINITY, del_r = 0.f;  // rows off the route: p = 0
  {
    const long long r = (long long)bh * a.Ns + (qrow < 0 ? 0 : qrow);
    const bf16_t* qp = (const bf16_t*)a.Q + r * D + 8 * h;
    const bf16_t* gp = (const bf16_t*)a.dO + r * D + 8 * h;
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
  if constexpr (POOLED) {
    Kg = (const char*)a.pkhi + (long long)bh * a.mk_pad * KRB;
    Kg_lo = (const char*)a.pklo + (long long)bh * a.mk_pad * KRB;
    Vg = (const char*)a.pv + (long long)bh * a.mk_pad * KRB;
  } else {
    Kg = (const char*)a.K + (long long)bh * a.Nk * KRB;
    Vg = (const char*)a.V + (long long)bh * a.Nk * KRB;
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
      g.k[0][i] = *(const u32x4*)(Kg + (long long)row * KRB + c * 16);
      if constexpr (POOLED) g.k[1][i] = *(const u32x4*)(Kg_lo + (long long)row * KRB + c * 16);
      g.v[i] = *(const u32x4*)(Vg + (long long)row * KRB + c * 16);
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
    bf16_t* op = (bf16_t*)a.dQ + ((long long)bh * a.Ns + qrow) * D;
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

// dQ of full-route rows from the split partials, summed in split order.
template <int D>
__global__ __launch_bounds__(256) void isa_bwd_dq_merge_kernel(BwdArgs a) {
  constexpr int TPR = D / 4, RPB = 256 / TPR;
  const long long gid = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int e = (threadIdx.x % TPR) * 4;
  const long long rows_head = (long long)a.row_tiles * kFlashRows;
  const long long bh = gid / rows_head;
  const long long vrow = gid - bh * rows_head;
  if (bh >= a.BH) return;
  const int qrow = route_row(a.q_list + bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  if (qrow < 0) return;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < a.nsplit; ++k) s += *(const f32x4*)(a.part_dq + (gid * a.nsplit + k) * D + e);
  s *= a.inv_sqrt_d;
  *(u32x2*)((bf16_t*)a.dQ + (bh * a.Ns + qrow) * D + e) = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
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
    Kg = (const char*)a.K + ((long long)bh * a.Nk + krow) * KRB;
    Vg = (const char*)a.V + ((long long)bh * a.Nk + krow) * KRB;
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

  struct Staged { u32x4 q[NRC]; u32x4 g[NRC]; float l, d; };
  auto load = [&](long long step) -> Staged {
    Staged st;
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int q = tid + NTHR * i;
      const int r = route_row(qlist, a.q_k, a.b, a.nb_s, a.Ns, step * BR + q / KCPR);
      const long long off = ((long long)bh * a.Ns + (r < 0 ? 0 : r)) * D + (q % KCPR) * 8;
      st.q[i] = *(const u32x4*)((const bf16_t*)a.Q + off);
      st.g[i] = *(const u32x4*)((const bf16_t*)a.dO + off);
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
    bf16_t* out = (bf16_t*)(DK ? a.dK : a.dV) + ((long long)bh * a.Nk + krow) * D;
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
  for (int q = threadIdx.x; q < nr * CPR; q += 256) {
    const long long off = (bh * a.Nk + r0 + q / CPR) * D + (q % CPR) * 8;
    *(u32x4*)((bf16_t*)a.dK + off) = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)((bf16_t*)a.dV + off) = u32x4{0u, 0u, 0u, 0u};
  }
}

// ---------------------------------------------------------------------------

static BwdArgs bwd_args(const Layout& L, const BwdLayout& W, const BwdBufs& B) {
  BwdArgs a = {};
  a.Q = B.Q; a.K = B.K; a.V = B.V; a.O = B.O; a.dO = B.dO;
  a.dQ = B.dQ; a.dK = B.dK; a.dV = B.dV;
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
  a.part_dkv = (float*)(B.bws + W.off_part_dkv);
  a.dkvbar = (float*)(B.bws + W.off_dkvbar);
  a.nsplit = 1;
  a.Ns = L.Ns; a.Nk = L.Nk;
  a.BH = L.BH;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)L.d));
  a.inv_sqrt_d = (float)(1.0 / sqrt((double)L.d));
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
      hipLaunchKernelGGL((isa_bwd_delta_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a);
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
      const long long nwg = L.BH * a.key_tiles;
      a.n_wg = (int)nwg;
      if (what == BwdWhat::kDkFull)
        hipLaunchKernelGGL((isa_bwd_dkdv_kernel<D, false, true>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((isa_bwd_dkdv_kernel<D, false, false>), dim3((unsigned)nwg), dim3(512), 0, s, a);
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
      const long long nwg = (long long)a.row_tiles * L.BH * a.nsplit;
      a.n_wg = (int)nwg;
      if (full)
        hipLaunchKernelGGL((isa_bwd_dq_kernel<D, false>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((isa_bwd_dq_kernel<D, true>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      break;
    }
    case BwdWhat::kDqMerge: {
      if (L.full_rows == 0 || L.full_splits <= 1) return hipSuccess;
      a.q_list = fullq; a.q_k = L.kq; a.n_rows = L.full_rows;
      a.nsplit = L.full_splits;
      a.row_tiles = (int)((L.full_rows + kFlashRows - 1) / kFlashRows);
      constexpr int RPB = 256 / (D / 4);
      const long long rows = (long long)a.row_tiles * kFlashRows * L.BH;
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
