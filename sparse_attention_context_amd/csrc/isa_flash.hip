// Flash-style attention of ISA on gfx950 bf16 MFMA: full route, dense
// baseline and the pooled (sharpness + 0-th order Taylor) pass.
//
// "Lightning Unified Video Editing via In-Context Sparse Attention" (English
// abstract) sends high-error query blocks to full attention and the rest to a
// 0-th order Taylor sparse attention, after grouping queries by sharpness.
//  * full route (FK_GATHER): exact softmax attention over every source token
//    plus every token of the kept context blocks, K/V rows gathered through
//    the kept-context row table (d = 64) or the full-route key-row table,
//    one row per key of the route (d = 128);
//  * dense (FK_DENSE): every source query over every key row, the global
//    self-attention softmax(q k^T / sqrt d) v of the intelliparadigm.com page,
//    section 1 -- the library's own dense baseline;
//  * pooled (FK_POOLED): the same online softmax over the kept pooled blocks,
//    each weighted by its count n_j (an additive log2 n_j in the exp2
//    domain).  Its output is the Taylor route; the peak probability of that
//    softmax, exp2(max - ref) / l, is the query sharpness.  Pooled keys come
//    as bf16 hi + lo parts (two MFMAs) so the logits carry ~2^-17.
//
// Two kernels: isa_flash_kernel (below) runs the pooled pass at d = 64 and
// the stand-alone pooled stages; isa_flash_pp_kernel runs the token modes
// (d = 128 and 64) with the same arithmetic on a ping-pong wave schedule and
// direct global->LDS loads, and isa_flash_pp_pooled_kernel the pooled pass at
// d = 128.
//
// Workgroup: NW waves, 32 query rows each; key tiles of 64.  Each wave
// computes S^T = K Q^T with 32x32x16 MFMAs (lane = one query, 32 keys), the
// online softmax in fp32 on exp2, and O^T += V^T P^T: P^T is already the
// B-operand layout, and the V^T operand is read from a row-major V tile with
// the LDS transpose read ds_read_b64_tr_b16 (within each 16-lane group, lane
// i receives element i%4 of the 8 bytes loaded by lane 4j + i/4, j = 0..3;
// lanes that load 4 consecutive d of key rows K0 + m/4 therefore receive 4
// keys of one d).  K rows are padded by 16 bytes and V rows by 64, which
// keeps the operand reads free of bank conflicts and makes every operand
// address a per-lane base plus an immediate.
//
// Pipeline per tile j (one barrier per tile, 2-stage LDS ring): global loads
// of tile j+1 (row table looked up one tile earlier, so no load waits on a
// lookup) | lookup of tile j+2's rows | S = K(j) Q^T | softmax |
// O += V(j)^T P^T | tile j+1 registers -> LDS.  A row's reference maximum only moves when
// a tile raises that row's max by more than 2^8 in the exp2 domain (then its
// accumulator is rescaled); exp2 arguments stay <= 8, exact in fp32 sums and
// bf16 probabilities.  The true running max is tracked separately for the
// peak probability.
//
// The full route's key ranges are split across workgroups: on the ping-pong
// kernels by the stream-K split below (whole row tiles, then equal ranges),
// on isa_flash_kernel (short d = 64 work) into nsplit equal parts.  Each
// part writes its own normalised output in bf16 with its reference max and
// sum in fp32, and the merge kernel takes the sum-weighted mean of a row's
// parts in part order (deterministic).
#include "isa_device.h"
#include "isa_kernels.h"
#include "isa_split.h"

#include <type_traits>

#ifndef ISA_PP_LOOKAHEAD
#define ISA_PP_LOOKAHEAD 5
#endif
// the persistent full-route kernel: 3 measured about 1 % faster than 5 there
// (4 in between, 2 no better than 3)
#ifndef ISA_PPS_LOOKAHEAD
#define ISA_PPS_LOOKAHEAD 3
#endif
#ifndef ISA_FLASH_PPS
#define ISA_FLASH_PPS 1
#endif

namespace isa {

constexpr bool kUsePps = ISA_FLASH_PPS;

enum { FK_DENSE = 0, FK_GATHER = 1, FK_POOLED = 2 };
enum { FR_IDENTITY = 0, FR_TABLE = 1 };

struct FlashArgs {
  const void* Q;
  void* O;
  const void* K;        // token modes: [B,H,Nk,D] through mk
  const void* V;
  RowMap rmq, rmo, rmk, rmv;   // element strides of Q, O, K, V
  int o_span;           // bytes of one head of O: ((rows - 1) * mo.sn + D) * 2 < 2^31
  const int* ctx_rows;  // gather: [BH][ctx_tok] absolute rows, -1 past a short last block
  const int* kept;      // gather: [BH][kc]
  const int* key_rows;  // gather, d = 128: [BH][n_keytab] row of every full-route key (0 for padding)
  int n_keytab;
  long long ctx_tok;
  int kc, nb_c, b, tail_c;
  const void* pkhi;     // pooled: [BH][mk_pad][D]
  const void* pklo;
  const void* pv;
  const float* pbias;   // pooled: [BH][mk_pad] log2 n_j, -inf for padding
  int mk_pad;
  int mk, tail_s;       // pooled: kept blocks per head (source + kept context); rows of the last source block
  const int* q_list;    // route block list: [BH][q_k] (table rows)
  int q_k, nb_s;        // blocks in the list per head; source blocks
  long long n_rows;     // virtual query rows per head
  float* peak;          // pooled: [BH][Ns]
  float* lse;           // [BH][Ns] log2-domain log-sum-exp of each written row (null: not kept)
  // split partials: [BH][row_tiles*BM][nsplit][D] normalised outputs and
  // [..][2] (max, sum) for the equal splits; [Rs][sk_P][BM][..] for the
  // stream-K split's cut row tiles
  bf16_t* part_o;
  float* part_ml;
  int nsplit, tiles_per_split;
  int Ns, Nk;
  int row_tiles;
  int n_wg;
  float scale_log2;     // log2(e)/sqrt(d)
  // full route at d = 128 (row tiles Ri = bh * row_tiles + rt): row tiles
  // below sk_R0 whole, sk_K per persistent workgroup; the units
  // u = (Ri - sk_R0) * sk_T + t of the rest (sk_U of them) in sk_G equal
  // ranges, a row tile in at most sk_P of them
  long long sk_U;
  int sk_G, sk_P, sk_T, sk_R0, sk_K;
  // row tiles in eight blocks of sk_q or sk_q + 1 (the first sk_x blocks),
  // one per XCD of the sk_grid persistent workgroups (see sk_round_row)
  int sk_grid, sk_q, sk_x;
};

// Pooled mode: key tile kt of the packed kept set (keys 64 kt .. 64 kt + 63)
// is uniform when every one of its blocks holds b rows, so that its bias is
// log2 b in every column -- no padding, not the short last source block,
// not a short last context block that is kept (ctx_tail: the head keeps
// it).  Such a tile's logits S*sc + log2 b need no per-element bias: the
// maximum is taken over S and each exponent is one fma, S*sc + (log2 b -
// m_ref).  Both pooled kernels apply the same rule, so they stay bit-identical.
__device__ __forceinline__ bool pooled_uniform_tile(const FlashArgs& a, int kt, bool ctx_tail) {
  const int k0 = kt * 64, k1 = k0 + 64;
  if (k1 > a.mk) return false;
  if (a.tail_s != a.b && a.nb_s - 1 >= k0 && a.nb_s - 1 < k1) return false;
  if (ctx_tail && a.mk - 1 >= k0 && a.mk - 1 < k1) return false;
  return true;
}
__device__ __forceinline__ bool pooled_ctx_tail(const FlashArgs& a, long long bh) {
  return a.kc > 0 && a.tail_c != a.b && a.kept[bh * a.kc + a.kc - 1] == a.nb_c - 1;
}

template <int D, int KM, int RM, int NW, bool WO, bool WP>
__global__ __launch_bounds__(NW * 64) void isa_flash_kernel(FlashArgs a) {
  typedef bf16x8 Op;
  constexpr bool GATHER = KM == FK_GATHER, POOLED = KM == FK_POOLED;
  constexpr int NTHR = NW * 64;
  constexpr int ES = 2, BN = 64, BM = 32 * NW;
  // LDS stages of the K/V ring; tile j+PF is loaded while tile j is computed
  // (two stages measured faster than three: fewer registers for the ring).
  constexpr int NSTAGE = 2;
  constexpr int PF = NSTAGE - 1;
  constexpr int KRB = D * ES, KCPR = KRB / 16;   // global K/V row: bytes, 16-byte chunks
  constexpr int KRS = KRB + 16;                  // LDS K row stride (one chunk of padding)
  constexpr int VRS = KRB + 64;                  // LDS V row stride (4 rows x 64 B on distinct banks)
  constexpr int KT = BN * KRS, VT = WO ? BN * VRS : 0;
  constexpr int NKT = POOLED ? 2 : 1;            // K tiles per stage (hi, lo)
  constexpr int STAGE = NKT * KT + VT;
  constexpr int NKC = BN * KCPR / NTHR;          // 16-byte chunks per thread per K (or V) tile
  constexpr int NT = D / 32;
  constexpr int NR = NKC;                        // key rows a thread loads per tile (K and V share them)
  static_assert(NKC >= 1, "tile mapping");

  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * STAGE];
  __shared__ __attribute__((aligned(16))) float sbias[POOLED ? NSTAGE : 1][BN];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  // work item lid: row tile fastest, then key split, then head, so that the
  // workgroups running at once on an XCD share one K/V range in its L2
  const int lid = xcd_remap(blockIdx.x, a.n_wg);
  const int rt = lid % a.row_tiles;
  const int rest = lid / a.row_tiles;
  const int split = rest % a.nsplit;
  const int bh = rest / a.nsplit;

  // ---- query row of this lane (invalid rows read row 0 and store nothing)
  const long long vrow = (long long)rt * BM + w * 32 + l32;
  int qrow;
  if constexpr (RM == FR_TABLE) qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  else qrow = vrow < a.Ns ? (int)vrow : -1;
  Op qB[D / 16];
  {
    const bf16_t* qp = (const bf16_t*)a.Q + rm_head(a.rmq, bh) + (long long)(qrow < 0 ? 0 : qrow) * a.rmq.sn + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qB[s] = *(const Op*)(qp + 16 * s);
  }

  // ---- key range of this workgroup
  int n_keys, n_valid;
  bool ctx_tail = false;   // pooled: the head keeps a short last context block
  if constexpr (GATHER) {
    n_keys = a.Ns + (int)a.ctx_tok;
    const bool tail_kept = a.kc > 0 && a.kept[(long long)bh * a.kc + a.kc - 1] == a.nb_c - 1;
    n_valid = n_keys - (tail_kept ? a.b - a.tail_c : 0);
  } else if constexpr (POOLED) {
    n_keys = n_valid = a.mk_pad;  // padding rows carry bias -inf
    ctx_tail = pooled_ctx_tail(a, bh);
  } else {
    n_keys = n_valid = a.Nk;
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
  const int* crow = GATHER ? a.ctx_rows + (long long)bh * a.ctx_tok : nullptr;
  const int ctx_last = (int)a.ctx_tok - 1;

  struct Rows { int r[NR]; };
  struct Staged { u32x4 k[NKT][NKC]; u32x4 v[WO ? NKC : 1]; float bias; };
  struct STile { f32x16 t[2]; };

  auto key_of = [&](int r) -> int { return (tid + NTHR * r) / KCPR; };
  // source rows of the thread's keys of tile `tile` (padding -> row 0, masked later)
  auto lookup = [&](int tile) -> Rows {
    Rows rows;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int t = tile * BN + key_of(r);
      if constexpr (GATHER) {
        int c = 0;
        if (ctx_last >= 0) c = crow[min(max(t - a.Ns, 0), ctx_last)];
        rows.r[r] = t < a.Ns ? t : (t < n_valid && c >= 0 ? c : 0);
      } else if constexpr (POOLED) {
        rows.r[r] = t;
      } else {
        rows.r[r] = t < n_valid ? t : 0;
      }
    }
    return rows;
  };
  auto load = [&](Rows rows, int tile) -> Staged {
    Staged g;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = (tid + NTHR * i) % KCPR;
      g.k[0][i] = *(const u32x4*)(Kg + (long long)rows.r[i] * krs + c * 16);
      if constexpr (POOLED) g.k[NKT - 1][i] = *(const u32x4*)(Kg_lo + (long long)rows.r[i] * krs + c * 16);
    }
    if constexpr (WO) {
#pragma unroll
      for (int i = 0; i < NKC; ++i) {
        const int c = (tid + NTHR * i) % KCPR;
        g.v[i] = *(const u32x4*)(Vg + (long long)rows.r[i] * vrs + c * 16);
      }
    }
    g.bias = 0.f;
    if constexpr (POOLED) {
      if (tid < BN) g.bias = a.pbias[(long long)bh * a.mk_pad + tile * BN + tid];
    }
    return g;
  };
  auto store = [&](int stage, Staged g) {
    char* Ks = smem + stage * STAGE;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < NKC; ++i) {
        const int q = tid + NTHR * i;
        const int kr = q / KCPR, c = q % KCPR;
        *(u32x4*)(Ks + kt * KT + kr * KRS + c * 16) = g.k[kt][i];
      }
    if constexpr (WO) {
      char* Vs = Ks + NKT * KT;
#pragma unroll
      for (int i = 0; i < NKC; ++i) {
        const int q = tid + NTHR * i;
        const int kr = q / KCPR, c = q % KCPR;
        *(u32x4*)(Vs + kr * VRS + c * 16) = g.v[i];
      }
    }
    if constexpr (POOLED) {
      if (tid < BN) sbias[stage][tid] = g.bias;
    }
  };
  // Operands: lane (l32, h) reads row 32*i + l32, elements 16*s + 8*h .. +7
  // of a padded tile: one per-lane base, the rest are immediate offsets.
  const int kbase = l32 * KRS + 16 * h;
  // V^T operand of lane (l32, h) in 16-lane group g = lane/16, m = lane%16:
  // transposed reads at key rows 16 s + 4 h + m/4 (+8), d = 32 t + 16 (g%2) + 4 (m%4)
  const int vbase = NKT * KT + (4 * h + ((lane & 15) >> 2)) * VRS + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * ES;
  auto qk = [&](int stage) -> STile {
    const char* Ks = smem + stage * STAGE + kbase;
    STile S;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      S.t[ti] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        S.t[ti] = mma32(*(const Op*)(Ks + 32 * ti * KRS + 32 * s), qB[s], S.t[ti]);
        if constexpr (POOLED) S.t[ti] = mma32(*(const Op*)(Ks + KT + 32 * ti * KRS + 32 * s), qB[s], S.t[ti]);
      }
    }
    return S;
  };

  f32x16 acc[WO ? NT : 1];
#pragma unroll
  for (int t = 0; t < (WO ? NT : 1); ++t) acc[t] = f32x16{};
  // pk: the row's largest term of the running sum l_run, rescaled with it,
  // so that the peak probability pk / l rounds like the sum it divides
  float m_ref = -INFINITY, pk = 0.f, l_run = 0.f;
  const float sc = a.scale_log2;
  // exp2-domain headroom before the reference max moves; token modes keep
  // logits raw (x = S), pooled mode works on x = S*sc + log2 n_j directly
  const float thresh = POOLED ? 8.0f : 8.0f / sc;

  const float lb = POOLED ? log2f((float)a.b) : 0.f;   // the bias of a block of b rows
  auto softmax_pv = [&](int j, STile St) {
    f32x16* S = St.t;
    const int t0 = (t_begin + j) * BN;
    const bool uni = POOLED && pooled_uniform_tile(a, t_begin + j, ctx_tail);
    if (POOLED && !uni) {
      const float* bs = sbias[j % NSTAGE];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 bb = *(const f32x4*)(bs + 32 * ti + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) S[ti][4 * g + e] = fmaf(S[ti][4 * g + e], sc, bb[e]);
        }
    } else if (!POOLED && t0 + BN > n_valid) {
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3) >= n_valid) S[ti][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[ti][r]);
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float smax = mx;              // uniform tiles: the largest S
    if (uni) mx = fmaf(mx, sc, lb);     // the largest S*sc + log2 b (the fma is monotone in S)
    // each row moves its own reference (rows of a wave never influence one
    // another, so a row's result does not depend on how rows are grouped);
    // the branch is taken when any row of the wave needs it
    const bool move = mx > m_ref + thresh;
    if (__ballot(move)) {
      const float m_new = move ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(POOLED ? (m_ref - m_new) : (m_ref - m_new) * sc);
      l_run *= alpha;
      if constexpr (WP) pk *= alpha;
      if constexpr (WO) {
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      }
      m_ref = m_new;
    }
    const float msub = POOLED ? m_ref : m_ref * sc;
    const float lm = lb - m_ref;   // uniform pooled tiles: exponent S*sc + (log2 b - m_ref)
    // the tile's largest term, with the expression of its terms below
    if constexpr (WP) pk = fmaxf(pk, __builtin_amdgcn_exp2f(uni ? fmaf(smax, sc, lm) : mx - msub));
    Op pB[4];
    float psum = 0.f;  // tile-local sum first: fewer roundings at the running sum's scale
    if (uni) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[s >> 1][8 * (s & 1) + jj], sc, lm));
          psum += p;
          pB[s][jj] = (__bf16)p;
        }
      }
    } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float x = S[s >> 1][8 * (s & 1) + jj];
        const float p = __builtin_amdgcn_exp2f(POOLED ? x - msub : fmaf(x, sc, -msub));
        psum += p;
        pB[s][jj] = (__bf16)p;
      }
    }
    }
    l_run += psum;
    if constexpr (WO) {
      // addressing stays in the LDS address space so the constant offsets
      // fold into the instructions
      const lds_char* Vs = (const lds_char*)smem + (j % NSTAGE) * STAGE + vbase;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const lds_char* p = Vs + 16 * s * VRS + 32 * t * ES;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * VRS));
          const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[t] = mma32(__builtin_bit_cast(Op, v), pB[s], acc[t]);
        }
    }
  };

  // ---- prologue: tiles 0 .. PF-1 in LDS, the rows of tile PF looked up
  Rows ra = {}, rb = {};
  Staged gs = {};
  if (nt > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (p < nt) {
        const int tp = t_begin + p;
        store(p, load(lookup(tp), tp));
      }
    }
    ra = lookup(min(t_begin + PF, t_last));
    __syncthreads();
  }

  // Tile j: the rows of tile j+PF were looked up one tile earlier, those of
  // tile j+PF+1 are fetched now; loads past the last tile re-read it and are
  // never stored.  Stage (j+PF) % NSTAGE was last read in tile j-1, which
  // every wave finished before the barrier that closed it.
  for (int j = 0; j < nt; j += 2) {
    gs = load(ra, min(t_begin + j + PF, t_last));
    rb = lookup(min(t_begin + j + PF + 1, t_last));
    softmax_pv(j, qk(j % NSTAGE));
    if (j + PF < nt) store((j + PF) % NSTAGE, gs);
    __syncthreads();
    if (j + 1 < nt) {
      gs = load(rb, min(t_begin + j + 1 + PF, t_last));
      ra = lookup(min(t_begin + j + PF + 2, t_last));
      softmax_pv(j + 1, qk((j + 1) % NSTAGE));
      if (j + 1 + PF < nt) store((j + 1 + PF) % NSTAGE, gs);
      __syncthreads();
    }
  }

  // ---- epilogue
  const float l_tot = l_run + wave_shfl_xor(l_run, 32);
  if (a.nsplit == 1) {
    if (qrow >= 0) {
      const float inv = 1.0f / l_tot;
      if constexpr (WO) {
        bf16_t* op = (bf16_t*)a.O + rm_head(a.rmo, bh) + (long long)qrow * a.rmo.sn;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * t + 8 * g + 4 * h;
            *(u32x2*)(op + d0) = u32x2{pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                                       pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
          }
      }
      if constexpr (WP) {
        if (h == 0) a.peak[(long long)bh * a.Ns + qrow] = pk * inv;
      }
      if constexpr (WO) {
        // p = exp2(x - lse) with x = S*sc (tokens) or S*sc + log2 n_j (pooled)
        if (a.lse && h == 0) a.lse[(long long)bh * a.Ns + qrow] = (POOLED ? m_ref : m_ref * sc) + __builtin_log2f(l_tot);
      }
    }
  } else if constexpr (WO) {
    // split partial: this split's normalised output (bf16) and its (ref max, sum)
    const long long prow = ((long long)bh * a.row_tiles * BM + vrow) * a.nsplit + split;
    bf16_t* po = a.part_o + prow * D;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(u32x2*)(po + 32 * t + 8 * g + 4 * h) = u32x2{pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                                                       pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
    if (h == 0) *(float2*)(a.part_ml + prow * 2) = float2{m_ref, l_tot};
  }
}

// Ping-pong schedule for the token modes (full route, dense, context rows),
// d = 128 and d = 64.
//
// Two groups of four waves (waves w and w+4 share a SIMD) run the same tile
// loop one phase apart, so that one group's MFMA cluster overlaps the other
// group's softmax.  Each tile j takes two barrier-separated phases:
//   X_j  acc += V(j-1)^T P(j-1)^T, then S(j) = K(j) Q^T   (MFMA + LDS reads)
//   Y_j  direct global->LDS loads of K(j+3) and V(j+2) (and, gathering,
//        of the row-table entries of tile j+6); softmax of S(j) -> P(j)
// Group 0 runs X_j in phase 2j and Y_j in 2j+1, group 1 one phase later.
// Each group loads its own half (32 rows) of every K and V tile with
// global_load_lds_dwordx4 (each lane's 16 bytes land at the wave's LDS base
// + 16 x lane), so no tile passes through registers.  K and V rings have four
// stages: a stage is refilled (issue in phase 2t-5 or later) only after the
// last read of its previous tile (phase 2t-7 for K, 2t-5 for V), and each
// wave waits for its loads of Y_{j-1} before the barrier that closes Y_j, so
// every tile is in LDS two phases before its first read.
//
// LDS rows are 2d bytes, unpadded; the 16-byte chunk c of row r is stored
// at chunk c ^ f(r), f(r) = ((r & 3) << 2) | ((r >> 2) & 3) for 256-byte
// rows (lds_swz64 for 128-byte rows).  Sixteen consecutive rows at one chunk
// (the K operand reads) and four consecutive rows at four consecutive chunks
// (the V^T transpose reads) then fall on distinct banks.  A wave loads 8 rows
// of each tile: two loads of 4 rows (d = 128) or one of 8 (d = 64).  Operand
// addresses are per-lane offsets computed once.
// Numerics are those of isa_flash_kernel: the same per-row reference max,
// sums and bf16 roundings.
// (lds_swz, dma16x2 and pp_issue_order are in isa_device.h)

template <int KM, int RM, int D>
__global__ __launch_bounds__(512) void isa_flash_pp_kernel(FlashArgs a) {
  typedef bf16x8 Op;
  static_assert(D == 128 || D == 64, "head sizes of the ping-pong kernel");
  constexpr bool GATHER = KM == FK_GATHER;
  static_assert(KM != FK_POOLED, "token modes only");
  constexpr int BN = 64, BM = 256, NST = 4;
  constexpr int RB = D * 2;                      // row bytes (global and LDS)
  constexpr int TB = BN * RB;                    // tile bytes
  constexpr int NT = D / 32;
  constexpr int LPR = RB / 16;                   // lanes per row of one 16-byte load
  constexpr int NLD = LPR / 8;                   // loads per wave and tile (8 rows)
  static_assert(BM == kFlashRows, "tile mapping");
  auto swz = [](int r) { return D == 128 ? lds_swz(r) : lds_swz64(r); };

  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * TB];   // K ring, then V ring
  __shared__ __attribute__((aligned(16))) int stab[GATHER ? 8 : 1][4][64];   // per-wave key-table ring (gather)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  // Work items: gather mode (the full route), the items of stream-K
  // workgroup g (the logical id), as the persistent kernel takes them -- its
  // whole row tiles, then the row tiles that its range meets -- one after
  // the other, the pipeline drained between them; dense mode, row tile rt of
  // head bh (one key range).  Consecutive workgroups run on one XCD and share
  // its L2.
  int n_items = 1;
  SkItems sk = {};
  if constexpr (GATHER) {
    sk = sk_items(a, xcd_remap((int)blockIdx.x, (int)gridDim.x));
    n_items = sk.kdp + sk.nsk;
  }
#pragma unroll 1
  for (int item = 0; item < n_items; ++item) {
    int bh, rt, part = -1;   // part < 0: the whole row tile (output written here)
    int Rs = 0;              // else part `part` of range-phase row tile Rs (its partial buffer slot)
    int t_begin = 0, t_end = 0;   // key tiles of the item (gather)
    if constexpr (GATHER) {
      const SkItem it = sk_item(a, sk, item);
      bh = it.bh;
      rt = it.rt;
      t_begin = it.t_begin;
      t_end = it.t_begin + it.nt;
      if (it.part >= 0) {
        part = it.part & 7;
        Rs = it.part >> 3;
      }
      if (item > 0) __syncthreads();   // the previous item's LDS reads are done
    } else {
      const int lid = xcd_remap(blockIdx.x, a.n_wg);
      rt = lid % a.row_tiles;
      bh = lid / a.row_tiles;
    }

    const long long vrow = (long long)rt * BM + w * 32 + l32;
    int qrow;
    if constexpr (RM == FR_TABLE) qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
    else qrow = vrow < a.Ns ? (int)vrow : -1;
    Op qB[D / 16];
    {
      const bf16_t* qp = (const bf16_t*)a.Q + rm_head(a.rmq, bh) + (long long)(qrow < 0 ? 0 : qrow) * a.rmq.sn + 8 * h;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qB[s] = *(const Op*)(qp + 16 * s);
    }

    int n_keys, n_valid;
    if constexpr (GATHER) {
      n_keys = a.Ns + (int)a.ctx_tok;
      const bool tail_kept = a.kc > 0 && a.kept[(long long)bh * a.kc + a.kc - 1] == a.nb_c - 1;
      n_valid = n_keys - (tail_kept ? a.b - a.tail_c : 0);
    } else {
      n_keys = n_valid = a.Nk;
    }
    const int nt = GATHER ? t_end - t_begin : (n_keys + BN - 1) / BN;

    const char* Kg = (const char*)a.K + rm_head(a.rmk, bh) * 2;
    const char* Vg = (const char*)a.V + rm_head(a.rmv, bh) * 2;
    const unsigned krs = (unsigned)a.rmk.sn * 2u, vrs = (unsigned)a.rmv.sn * 2u;   // row steps in bytes (< 2^24)
    const int* tab = GATHER ? a.key_rows + (long long)bh * a.n_keytab : nullptr;

    // This wave loads rows 32*grp + 8*wg + 4*i + lane/16 (i = 0, 1) of each
    // tile (d = 64: rows 32*grp + 8*wg + lane/8), one 16-byte chunk each:
    // physical chunk lane%16 (lane%8) of the row, which holds logical chunk
    // (lane%16) ^ f(row).
    const int lrow0 = 32 * grp + 8 * wg + lane / LPR;
    struct Rows { int r[NLD]; };
    // Gather: the key-row table entries of the wave's 8 rows of tile t come to a
    // per-wave LDS ring (slot t % 4) by a direct load in step t-6, entry
    // 2q + i holding row 32*grp + 8*wg + q + 4i (d = 64: entry q row
    // 32*grp + 8*wg + q), are read into registers in step t-4 and used in
    // steps t-3 (K) and t-2 (V); so no load result is waited for inside the
    // tile loop.
    // (slots are indexed by the tile's position j in this workgroup's range)
    const unsigned stab_w = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_char*)&stab[0][0][0]) +
                            __builtin_amdgcn_readfirstlane(w) * (unsigned)sizeof(stab[0]);
    auto fetch_rows = [&](int j, int tile) {
      if constexpr (GATHER) {
        const int k = D == 128 ? 4 * (lane & 1) + ((lane >> 1) & 3) : (lane & 7);
        const int idx = tile * BN + 32 * grp + 8 * wg + k;
        dma4(stab_w + (unsigned)(j & 3) * (unsigned)sizeof(stab[0][0]), tab, (unsigned)idx * 4u);
      }
    };
    auto rows_of = [&](int j) -> Rows {
      Rows rows = {};
      if constexpr (GATHER) {
        if constexpr (D == 128) {
          const int2 v = *(const int2*)&stab[w][j & 3][2 * (lane >> 4)];
          rows.r[0] = v.x;
          rows.r[NLD - 1] = v.y;
        } else {
          rows.r[0] = stab[w][j & 3][lane >> 3];
        }
      }
      return rows;
    };
    const unsigned lds_k = (unsigned)(size_t)(lds_char*)smem;
    const unsigned lds_v = lds_k + NST * TB;
    // Lane part of the i-th load: row lrow0 + 4i (its offset within a tile,
    // in K and in V rows) and the 16-byte chunk that the swizzle puts at this
    // lane.
    unsigned lchunk[NLD], lrowk[NLD], lrowv[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      lchunk[i] = (unsigned)(((lane & (LPR - 1)) ^ swz(lrow0 + 4 * i)) * 16);
      lrowk[i] = __umul24((unsigned)(lrow0 + 4 * i), krs) + lchunk[i];
      lrowv[i] = __umul24((unsigned)(lrow0 + 4 * i), vrs) + lchunk[i];
    }
    // Global offsets of the wave's two loads of a tile (rows rs bytes apart;
    // lro: the lane parts for that tensor): gathered rows come from the
    // key-row table (whose padding reads row 0), dense tiles of valid rows
    // only are a contiguous row range (a uniform branch).
    auto src_offs = [&](Rows rows, int tile, unsigned* o, unsigned rs, const unsigned* lro) {
      const int t0 = tile * BN;
      if constexpr (GATHER) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) o[i] = __umul24((unsigned)rows.r[i], rs) + lchunk[i];
      } else {
        if (t0 + BN <= n_valid) {
#pragma unroll
          for (int i = 0; i < NLD; ++i) o[i] = (unsigned)t0 * rs + lro[i];
        } else {
#pragma unroll
          for (int i = 0; i < NLD; ++i) {
            const int t = t0 + lrow0 + 4 * i;
            o[i] = __umul24((unsigned)(t < n_valid ? t : 0), rs) + lchunk[i];
          }
        }
      }
    };
    // LDS base of this wave's first load into a ring stage (the second is 4
    // rows further)
    const unsigned wrow = __builtin_amdgcn_readfirstlane((32 * grp + 8 * wg) * RB);
    auto issue_tile = [&](unsigned ring, int stage, const char* base, Rows rows, int tile, unsigned rs,
                          const unsigned* lro) {
      unsigned o[NLD];
      src_offs(rows, tile, o, rs, lro);
      const unsigned d0 = ring + wrow + (unsigned)stage * TB;
      if constexpr (NLD == 2) dma16x2(d0, d0 + 4 * RB, base, o[0], o[NLD - 1]);
      else dma16(d0, base, o[0]);
    };
    auto issue = [&](int sk, Rows rk, int tk, int sv, Rows rv, int tv) {
      issue_tile(lds_k, sk, Kg, rk, tk, krs, lrowk);
      issue_tile(lds_v, sv, Vg, rv, tv, vrs, lrowv);
    };

    // operand offsets: K row 32*ti + l32, logical chunk 2s + h; V^T transpose
    // reads at key rows 16s + 4h + m/4 (+8), d = 32t + 16(g%2) + 4(m%4), with
    // g = lane/16, m = lane%16 (see isa_flash_kernel)
    int koff[D / 16], voff[NT][2];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] = l32 * RB + ((((2 * s + h) ^ swz(l32)) * 16));
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int m = lane & 15;
        const int kr = 4 * h + (m >> 2) + 8 * hi;
        const int c = 4 * t + 2 * ((lane >> 4) & 1) + ((m & 3) >> 1);
        voff[t][hi] = NST * TB + kr * RB + ((c ^ swz(kr)) * 16) + 8 * (m & 1);
      }

    struct STile { f32x16 t[2]; };
    struct PTile { Op p[4]; };
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.f;
    const float sc = a.scale_log2;
    const float thresh = 8.0f / sc;

    // X phase with both products as one pipeline of D/4 MFMAs (D/8 of P.V,
    // then D/8 of K.Q^T); the operand reads of each MFMA are issued LA MFMAs
    // ahead.
    auto pv_qk = [&](int vstage, const PTile& P, int kstage) -> STile {
      constexpr int LA = ISA_PP_LOOKAHEAD;
      constexpr int NM = D / 8;   // MFMAs of each product
      const lds_char* Vs = (const lds_char*)smem + vstage * TB;
      const lds_char* Ks = (const lds_char*)smem + kstage * TB;
      Op opv[NM], opk[NM];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + voff[t][0] + 16 * q * RB));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + voff[t][1] + 16 * q * RB));
          opv[4 * t + q] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
      for (int q = 0; q < D / 16; ++q)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) opk[2 * q + ti] = *(const Op*)(Ks + koff[q] + 32 * ti * RB);
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m >> 2] = mma32(opv[m], P.p[m & 3], acc[m >> 2]);
      STile S;
      S.t[0] = f32x16{};
      S.t[1] = f32x16{};
#pragma unroll
      for (int m = 0; m < NM; ++m) S.t[m & 1] = mma32(opk[m], qB[m >> 1], S.t[m & 1]);
      pp_issue_order<LA, NM, NM>();
      return S;
    };
    auto exp_tile = [&](const f32x16* S, PTile& P) -> float {
      const float msub = m_ref * sc;
      float psum = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[s >> 1][8 * (s & 1) + jj], sc, -msub));
          psum += p;
          P.p[s][jj] = (__bf16)p;
        }
      }
      return psum;
    };
    // Probabilities are first taken against the current reference max.  Any
    // probability above 2^8 (the point where isa_flash_kernel moves a row's
    // reference) makes the lane's tile sum exceed 2^7, so only then is the
    // row maximum formed and the move rule applied, and the tile recomputed:
    // the same references, sums and roundings as isa_flash_kernel.
    auto softmax = [&](int j, STile St) -> PTile {
      f32x16* S = St.t;
      const int t0 = (t_begin + j) * BN;
      if (t0 + BN > n_valid) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3) >= n_valid) S[ti][r] = -INFINITY;
      }
      PTile P;
      float psum = exp_tile(S, P);
      if (__ballot(!(psum <= 128.f))) {
        float mx = -INFINITY;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[ti][r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const bool move = mx > m_ref + thresh;
        if (__ballot(move)) {
          const float m_new = move ? mx : m_ref;
          const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * sc);
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] *= alpha;
          m_ref = m_new;
          psum = exp_tile(S, P);
        }
      }
      l_run += psum;
      return P;
    };

    // Barrier without a memory fence: the direct loads are waited for by
    // count (s_waitcnt vmcnt), every LDS read has been consumed by an MFMA
    // before the barrier, and the empty asm keeps the compiler from moving
    // memory accesses across it.
    auto phase_barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    // ---- tile loop, unrolled by four so that every ring stage is a
    // compile-time choice.  Positions past the last tile are clamped to it.
    auto cl = [&](int j) { return min(j, nt - 1); };
    auto tl = [&](int j) { return t_begin + cl(j); };
    if (nt > 0) {
      Rows rk, rv;   // rows of tiles j+3 (K) and j+2 (V) entering step j
      {
        fetch_rows(cl(0), tl(0));
        fetch_rows(cl(1), tl(1));
        fetch_rows(cl(2), tl(2));
        fetch_rows(cl(3), tl(3));
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        const Rows r0 = rows_of(cl(0)), r1 = rows_of(cl(1));
        rv = rows_of(cl(2));
        rk = rows_of(cl(3));
        issue(0, r0, tl(0), 0, r0, tl(0));
        issue(1, r1, tl(1), 1, r1, tl(1));
        // K(2) (V(2) is loaded again by the first step, into the same stage)
        issue(2, rv, tl(2), 2, rv, tl(2));
        fetch_rows(cl(4), tl(4));
        fetch_rows(cl(5), tl(5));
        // V stage 3 is first loaded in step 1; step 0 reads it as zeros
        u32x4* vz = (u32x4*)(smem + NST * TB + 3 * TB);
#pragma unroll
        for (int q = 0; q < TB / (16 * 512); ++q) vz[tid + 512 * q] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): prologue loads and the zero fill
      }
      phase_barrier();
      if (grp == 1) phase_barrier();   // group 1 runs one phase behind group 0
      STile S = {};
      PTile P = {};
      // Loads past the last tile re-read it (clamped) into the stage that the
      // schedule frees for tile j+3 / j+2 and are never read, so every step
      // issues the same loads and waits by the same count.
      auto step = [&](int j) {
        const int Z = j & 3;
        // X_j, at raised wave priority: the MFMA group's instructions issue
        // ahead of the softmax group's on the shared SIMD
        __builtin_amdgcn_s_setprio(3);
        // (step 0 multiplies the zeroed V stage 3 by P = 0, step nt computes
        // an S that is never used: every step runs the same pipeline)
        S = pv_qk((Z + 3) & 3, P, Z);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        phase_barrier();
        // Y_j
        issue((Z + 3) & 3, rk, tl(j + 3), (Z + 2) & 3, rv, tl(j + 2));
        const Rows rn = rows_of(cl(j + 4));   // used one step later: its LDS latency is hidden
        fetch_rows(cl(j + 6), tl(j + 6));
        if (j < nt) P = softmax(j, S);
        rv = rk;
        rk = rn;
        // the loads of Y_{j-1} have landed before the barrier that closes Y_j
        // (this step's: K and V, NLD each, and the table chunk)
        if constexpr (GATHER) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NLD + 1));   // vmcnt(5), d = 64 vmcnt(3)
        else __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NLD));                        // vmcnt(4), d = 64 vmcnt(2)
        phase_barrier();
      };
      for (int j = 0; j <= nt; ++j) step(j);
      __builtin_amdgcn_s_waitcnt(0x0f70);   // no load into this workgroup's LDS outlives it
      if (grp == 0) phase_barrier();   // balances group 1's extra barrier
    }

    // ---- epilogue (as isa_flash_kernel's).  16-byte chunk c = d / 8 of a
    // row has its halves in lanes l and l + 32; for the chunk pair (2k, 2k+1)
    // one permlane32 swap per word gives lane l all of chunk 2k and lane l + 32
    // all of chunk 2k + 1, so each store writes 32 bytes of a row, not 16.
    // (Both lanes of a row are active or inactive together.)
    auto store_row = [&](bf16_t* rowp, float inv) {
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        unsigned x[2], y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = 2 * k + u, t = c >> 2, g = c & 3;
          unsigned* dst = u ? y : x;
          dst[0] = pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
          dst[1] = pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const auto sw = __builtin_amdgcn_permlane32_swap(x[e], y[e], false, false);
          x[e] = sw[0];
          y[e] = sw[1];
        }
        *(u32x4*)(rowp + 8 * (2 * k + h)) = u32x4{x[0], x[1], y[0], y[1]};
      }
    };
    const float l_tot = l_run + wave_shfl_xor(l_run, 32);
    if (part < 0) {
      if (qrow >= 0) {
        store_row((bf16_t*)a.O + rm_head(a.rmo, bh) + (long long)qrow * a.rmo.sn, 1.0f / l_tot);
        if (a.lse && h == 0) a.lse[(long long)bh * a.Ns + qrow] = m_ref * sc + __builtin_log2f(l_tot);
      }
    } else {
      // part `part` of the row tile: [Rs][sk_P][BM][D] partial outputs
      const long long prow = ((long long)Rs * a.sk_P + part) * BM + w * 32 + l32;
      store_row(a.part_o + prow * D, l_tot > 0.f ? 1.0f / l_tot : 0.f);
      if (h == 0) *(float2*)(a.part_ml + prow * 2) = float2{m_ref, l_tot};
    }
  }  // items
}

// Persistent form of the full-route ping-pong kernel: workgroup g takes
// stream-K range g (units u = Ri * T + t, Ri = bh * row_tiles + rt, T key
// tiles per row tile), i.e. the row tiles it meets, each over its share of
// key tiles, and runs them as one sequence of steps s: the rings, the
// row-table ring and the wait counts are those of isa_flash_pp_kernel with
// the step index s in place of the tile index, and at an item boundary the
// pipeline does not drain.  Step s0, the first of item r + 1: X_{s0} ends
// the P.V sum of item r and starts S of item r + 1 (its queries were loaded
// in Y_{s0-1}); Y_{s0} writes item r's output or its partial (the same
// normalisation and stores as the epilogue of isa_flash_pp_kernel, through
// buffer stores, so that every wave issues the same nine stores and the load
// waits can count them), resets the running state and takes the softmax of
// item r + 1's first tile.  Used when a range meets at most kPpsMaxItems row
// tiles; the output is that of isa_flash_pp_kernel bit for bit.
constexpr int kPpsMaxItems = 8;
__global__ __launch_bounds__(512) void isa_flash_pps_kernel(FlashArgs a) {
  typedef bf16x8 Op;
  constexpr int D = 128, BN = 64, BM = 256, NST = 4;
  constexpr int RB = D * 2, TB = BN * RB, NT = D / 32;
  static_assert(BM == kFlashRows, "tile mapping");

  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * TB];   // K ring, then V ring
  __shared__ __attribute__((aligned(16))) int stab[8][4][64];         // per-wave key-table ring
  __shared__ int sq[8][kPpsMaxItems][64];                             // query row of each lane and item
  __shared__ int snv[kPpsMaxItems];                                   // valid keys of each item's head
  // per item: byte offsets of its head in Q, O and K (= V, whose row map is
  // K's here), and the Q and O row steps.  Read from LDS where an item starts
  // or ends, so that the strides hold no registers across the tile loop.
  __shared__ long long shead[3][kPpsMaxItems];
  __shared__ unsigned sstep[2];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const int n_keys = a.Ns + (int)a.ctx_tok;
  // This workgroup's items: whole row tiles (the workgroups of an XCD take
  // consecutive row tiles of its block), then the row tiles that its
  // stream-K range meets (ranges of consecutive g on one XCD)
  const SkItems sk = sk_items(a, xcd_remap((int)blockIdx.x, (int)gridDim.x));
  const int nr = sk.kdp + sk.nsk;
  typedef SkItem Item;
  auto item_of = [&](int r) -> Item { return sk_item(a, sk, r); };
  // per item: each lane's query row and the head's valid key count
  for (int r = 0; r < nr; ++r) {
    const Item it = item_of(r);
    const long long vrow = (long long)it.rt * BM + w * 32 + l32;
    sq[w][r][lane] = route_row(a.q_list + (long long)it.bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
    if (tid == 0) {
      const bool tail_kept = a.kc > 0 && a.kept[(long long)it.bh * a.kc + a.kc - 1] == a.nb_c - 1;
      snv[r] = n_keys - (tail_kept ? a.b - a.tail_c : 0);
      shead[0][r] = rm_head(a.rmq, it.bh) * 2;
      shead[1][r] = rm_head(a.rmo, it.bh) * 2;
      shead[2][r] = rm_head(a.rmk, it.bh) * 2;
    }
  }
  if (tid == 0) {
    sstep[0] = (unsigned)a.rmq.sn * 2u;
    sstep[1] = (unsigned)a.rmo.sn * 2u;
  }
  __syncthreads();

  // Positions of the step sequence: a cursor walks (item, tile) and stops at
  // the last tile, so that loads past the end re-read it (never used).
  struct Cursor { int r, k; Item it; };
  auto cursor0 = [&]() { return Cursor{0, 0, item_of(0)}; };
  auto advance = [&](Cursor& c) {
    if (c.k + 1 < c.it.nt) {
      ++c.k;
    } else if (c.r + 1 < nr) {
      ++c.r;
      c.k = 0;
      c.it = item_of(c.r);
    }
  };

  Op qB[D / 16];
  auto load_q = [&](int r) {
    const int qrow = sq[w][r][lane];
    const bf16_t* qp =
        (const bf16_t*)((const char*)a.Q + shead[0][r] + (long long)(qrow < 0 ? 0 : qrow) * sstep[0]) + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qB[s] = *(const Op*)(qp + 16 * s);
  };

  const int lrow0 = 32 * grp + 8 * wg + (lane >> 4);
  struct Rows { int r[2]; };
  const unsigned stab_w = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_char*)&stab[0][0][0]) +
                          __builtin_amdgcn_readfirstlane(w) * (unsigned)sizeof(stab[0]);
  // key-table entries of the wave's 8 rows of the tile at cursor c into slot pos % 4
  auto fetch_rows = [&](int pos, const Cursor& c) {
    const int k = 4 * (lane & 1) + ((lane >> 1) & 3);
    const int* tab = a.key_rows + (long long)c.it.bh * a.n_keytab;
    const int idx = (c.it.t_begin + c.k) * BN + 32 * grp + 8 * wg + k;
    dma4(stab_w + (unsigned)(pos & 3) * (unsigned)sizeof(stab[0][0]), tab, (unsigned)idx * 4u);
  };
  auto rows_of = [&](int pos) -> Rows {
    const int2 v = *(const int2*)&stab[w][pos & 3][2 * (lane >> 4)];
    return Rows{{v.x, v.y}};
  };
  const unsigned lds_k = (unsigned)(size_t)(lds_char*)smem;
  const unsigned lds_v = lds_k + NST * TB;
  unsigned lchunk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) lchunk[i] = (unsigned)(((lane & 15) ^ lds_swz(lrow0 + 4 * i)) * 16);
  const unsigned wrow = __builtin_amdgcn_readfirstlane((32 * grp + 8 * wg) * RB);
  // K and V share one row map here (the launch checks it): head hd's rows
  // start rm_head(mk, hd) elements into each, rs bytes apart
  const unsigned rs = (unsigned)a.rmk.sn * 2u;
  auto head_off = [&](int r) { return uniform64(shead[2][r]); };   // of item r
  auto issue_tile = [&](unsigned ring, int stage, const void* base, int r, Rows rows) {
    const char* G0 = (const char*)base + head_off(r);
    const unsigned d0 = ring + wrow + (unsigned)stage * TB;
    dma16x2(d0, d0 + 4 * RB, G0, __umul24((unsigned)rows.r[0], rs) + lchunk[0],
            __umul24((unsigned)rows.r[1], rs) + lchunk[1]);
  };

  // the loads of step s (stage Z = s mod 4): K tile s + 3 (head offset ko,
  // in bytes, rows rk), V tile s + 2 (head offset vo, rows rv), key-table
  // entries of position pos (cursor c)
  Rows rk, rv;
  auto issue_step = [&](int Z, long long ko, long long vo, int pos, const Cursor& c) {
    const int kt = 4 * (lane & 1) + ((lane >> 1) & 3);
    const int* tab = a.key_rows + (long long)c.it.bh * a.n_keytab;
    const int idx = (c.it.t_begin + c.k) * BN + 32 * grp + 8 * wg + kt;
    dma_kvt(lds_k + wrow + (unsigned)((Z + 3) & 3) * TB, lds_v + wrow + (unsigned)((Z + 2) & 3) * TB,
            (const char*)a.K + ko, (const char*)a.V + vo, rs, (unsigned)rk.r[0], (unsigned)rk.r[1],
            (unsigned)rv.r[0], (unsigned)rv.r[1], lchunk[0], lchunk[1],
            stab_w + (unsigned)(pos & 3) * (unsigned)sizeof(stab[0][0]), tab, (unsigned)idx * 4u);
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
      voff[t][hi] = NST * TB + kr * RB + ((c ^ lds_swz(kr)) * 16) + 8 * (m & 1);
    }

  struct STile { f32x16 t[2]; };
  struct PTile { Op p[4]; };
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;
  const float sc = a.scale_log2;
  const float thresh = 8.0f / sc;

  auto pv_qk = [&](int vstage, const PTile& P, int kstage) -> STile {
    constexpr int LA = ISA_PPS_LOOKAHEAD;
    const lds_char* Vs = (const lds_char*)smem + vstage * TB;
    const lds_char* Ks = (const lds_char*)smem + kstage * TB;
    Op opv[16], opk[16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + voff[t][0] + 16 * q * RB));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + voff[t][1] + 16 * q * RB));
        opv[4 * t + q] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) opk[2 * q + ti] = *(const Op*)(Ks + koff[q] + 32 * ti * RB);
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m >> 2] = mma32(opv[m], P.p[m & 3], acc[m >> 2]);
    STile S;
    S.t[0] = f32x16{};
    S.t[1] = f32x16{};
#pragma unroll
    for (int m = 0; m < 16; ++m) S.t[m & 1] = mma32(opk[m], qB[m >> 1], S.t[m & 1]);
    pp_issue_order<LA>();
    return S;
  };
  auto exp_tile = [&](const f32x16* S, PTile& P) -> float {
    const float msub = m_ref * sc;
    float psum;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[s >> 1][8 * (s & 1) + jj], sc, -msub));
        psum = s + jj == 0 ? p : psum + p;   // (p >= 0: the same sum as from 0)
        P.p[s][jj] = (__bf16)p;
      }
    }
    return psum;
  };
  // the softmax rule of isa_flash_pp_kernel; t0: first key of the tile
  auto softmax = [&](int t0, int n_valid, STile St) -> PTile {
    f32x16* S = St.t;
    if (t0 + BN > n_valid) {
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3) >= n_valid) S[ti][r] = -INFINITY;
    }
    PTile P;
    float psum = exp_tile(S, P);
    if (__ballot(!(psum <= 128.f))) {
      float mx = -INFINITY;
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[ti][r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const bool move = mx > m_ref + thresh;
      if (__ballot(move)) {
        const float m_new = move ? mx : m_ref;
        const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * sc);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] *= alpha;
        m_ref = m_new;
        psum = exp_tile(S, P);
      }
    }
    l_run += psum;
    return P;
  };
  // Output of item r (as the epilogue of isa_flash_pp_kernel) through
  // buffer stores: a lane with nothing to store gets an offset past its
  // buffer, which the hardware drops, so every wave issues 8 + 1 stores.
  constexpr unsigned kOut = 0x80000000u;
  // 16-byte chunk c = d / 8 of a row: lanes l and l + 32 hold its halves;
  // one permlane32 swap per word gives each lane a whole chunk
  auto store_rows = [&](__amdgpu_buffer_rsrc_t rs, unsigned off, float inv) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      unsigned x[2], y[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = 2 * k + u, t = c >> 2, g = c & 3;
        unsigned* dst = u ? y : x;
        dst[0] = pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
        dst[1] = pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto sw = __builtin_amdgcn_permlane32_swap(x[e], y[e], false, false);
        x[e] = sw[0];
        y[e] = sw[1];
      }
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{x[0], x[1], y[0], y[1]}, rs,
                                            off == kOut ? kOut : off + 16 * (2 * k + h), 0, 0);
    }
  };
  auto finish = [&](int r, const Item& it) {
    const float l_tot = l_run + wave_shfl_xor(l_run, 32);
    const int qrow = sq[w][r][lane];
    if (it.part < 0) {
      const auto rO = __builtin_amdgcn_make_buffer_rsrc((char*)a.O + uniform64(shead[1][r]), (short)0, a.o_span,
                                                        0x00020000);
      store_rows(rO, qrow >= 0 ? (unsigned)qrow * sstep[1] : kOut, 1.0f / l_tot);
      const auto rL = __builtin_amdgcn_make_buffer_rsrc(a.lse ? a.lse + (long long)it.bh * a.Ns : a.lse, (short)0,
                                                        a.lse ? a.Ns * 4 : 0, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_ref * sc + __builtin_log2f(l_tot)), rL,
                                           (qrow >= 0 && h == 0) ? (unsigned)qrow * 4 : kOut, 0, 0);
    } else {
      // part it.part & 7 of the row tile: [Rs][sk_P][BM][D] partial outputs
      const long long prow0 = (long long)(it.part >> 3) * a.sk_P * BM;   // its first partial row
      const int nrow = a.sk_P * BM;
      const int prow = (it.part & 7) * BM + w * 32 + l32;
      const auto rP = __builtin_amdgcn_make_buffer_rsrc(a.part_o + prow0 * D, (short)0, nrow * RB, 0x00020000);
      store_rows(rP, (unsigned)prow * RB, l_tot > 0.f ? 1.0f / l_tot : 0.f);
      const auto rM = __builtin_amdgcn_make_buffer_rsrc(a.part_ml + prow0 * 2, (short)0, nrow * 8, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(m_ref), __float_as_uint(l_tot)}, rM,
                                           h == 0 ? (unsigned)prow * 8 : kOut, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    m_ref = -INFINITY;
    l_run = 0.f;
  };
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nr == 0) return;   // (never: every range holds at least one unit)
  int total = 0;
  for (int r = 0; r < nr; ++r) total += item_of(r).nt;
  const Item it0 = item_of(0);
  load_q(0);
  auto cp = [&](int s) { return min(s, total - 1); };   // slot positions past the end clamp
  // cursors: compute (step s), K (s + 3), V (s + 2), table (s + 6)
  Cursor cc = cursor0(), ck = cursor0(), cv = cursor0(), ct = cursor0();
  {
    // tables of positions 0..3, then K(0..2), V(0..1), tables of 4, 5
    fetch_rows(0, ct); advance(ct);
    fetch_rows(1, ct); advance(ct);
    fetch_rows(2, ct); advance(ct);
    fetch_rows(3, ct); advance(ct);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    const Rows r0 = rows_of(0), r1 = rows_of(1);
    rv = rows_of(2);
    rk = rows_of(3);
    issue_tile(lds_k, 0, a.K, ck.r, r0); advance(ck);
    issue_tile(lds_v, 0, a.V, cv.r, r0); advance(cv);
    issue_tile(lds_k, 1, a.K, ck.r, r1); advance(ck);
    issue_tile(lds_v, 1, a.V, cv.r, r1); advance(cv);
    issue_tile(lds_k, 2, a.K, ck.r, rv); advance(ck);   // (V(2) is loaded by the first step)
    fetch_rows(4, ct); advance(ct);
    fetch_rows(5, ct); advance(ct);
    u32x4* vz = (u32x4*)(smem + NST * TB + 3 * TB);
#pragma unroll
    for (int q = 0; q < TB / (16 * 512); ++q) vz[tid + 512 * q] = u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  }
  phase_barrier();
  if (grp == 1) phase_barrier();   // group 1 runs one phase behind group 0
  STile S = {};
  PTile P = {};
  Item fin = it0;   // the item whose output the next boundary writes
  int fin_r = 0;
  // One step.  first: the first tile of an item (after item 0, the previous
  // item's output is written); last: its last tile (the next item's queries
  // are loaded for the step after it), both for a one-tile item (uniform
  // flags, not template arguments: a third copy of the step spills); INNER:
  // a tile whose K, V and table
  // positions (s + 3, s + 2, s + 6) lie in the same item, so that they are
  // offsets from the compute cursor and the other cursors are not moved
  // (they are set again after the inner run).  nv: valid keys of the item's
  // head, kept in a register for the item.
  auto step = [&](int s, bool first, bool last, auto inner_c, int nv, long long ho) {
    constexpr bool INNER = decltype(inner_c)::value;
    const int Z = s & 3;
    __builtin_amdgcn_s_setprio(3);
    S = pv_qk((Z + 3) & 3, P, Z);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    phase_barrier();
    // Y_s
    const bool boundary = !INNER && first && s > 0;
    if (boundary) {
      finish(fin_r, fin);
      fin = cc.it;
      fin_r = cc.r;
    }
    if constexpr (INNER) {
      issue_step(Z, ho, ho, s + 6, Cursor{cc.r, cc.k + 6, cc.it});
      const Rows rn = rows_of(s + 4);
      P = softmax((cc.it.t_begin + cc.k) * BN, nv, S);
      rv = rk;
      rk = rn;
      ++cc.k;
      __builtin_amdgcn_s_waitcnt(0x0f75);   // vmcnt(5)
    } else {
      issue_step(Z, head_off(ck.r), head_off(cv.r), cp(s + 6), ct);
      const Rows rn = rows_of(cp(s + 4));
      if (s < total) P = softmax((cc.it.t_begin + cc.k) * BN, nv, S);
      rv = rk;
      rk = rn;
      const bool next_item = last && cc.r + 1 < nr;
      if (next_item) load_q(cc.r + 1);
      advance(cc);
      advance(ck);
      advance(cv);
      advance(ct);
      // the loads of Y_{s-1} have landed before the barrier that closes Y_s
      // (this step's output stores or query loads were issued too)
      if (boundary && next_item) __builtin_amdgcn_s_waitcnt(0x4f76);   // vmcnt(22): a one-tile item
      else if (boundary) __builtin_amdgcn_s_waitcnt(0x0f7e);         // vmcnt(14)
      else if (next_item) __builtin_amdgcn_s_waitcnt(0x0f7d);        // vmcnt(13)
      else __builtin_amdgcn_s_waitcnt(0x0f75);                       // vmcnt(5)
    }
    phase_barrier();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int s = 0;
  for (int r = 0; r < nr; ++r) {
    const int ntr = cc.it.nt;   // >= 1
    const int nv = snv[r];
    const long long ho = head_off(r);   // the item's K and V rows (inner steps)
    step(s++, true, ntr == 1, F_{}, nv, ho);   // (a one-tile item: first and last)
    if (ntr == 1) continue;
    // K, V and table positions stay in the item while k + 6 < ntr
    if (ntr > 7) {
      for (int k = 1; k + 6 < ntr; ++k) step(s++, false, false, T_{}, nv, ho);
      ck = cc; advance(ck); advance(ck); advance(ck);
      cv = cc; advance(cv); advance(cv);
      ct = cc;
#pragma unroll 1
      for (int j = 0; j < 6; ++j) advance(ct);
    }
#pragma unroll 1
    for (int k = max(1, ntr - 6); k < ntr - 1; ++k) step(s++, false, false, F_{}, nv, ho);
    step(s++, false, true, F_{}, nv, ho);
  }
  step(s, false, false, F_{}, 0, 0);   // s == total: the last P.V (no softmax)
  finish(fin_r, fin);
  __builtin_amdgcn_s_waitcnt(0x0f70);   // no load into this workgroup's LDS outlives it
  if (grp == 0) phase_barrier();   // balances group 1's extra barrier
}

// Ping-pong schedule of the pooled pass (sharpness + Taylor output of every
// source row over the kept pooled blocks), d = 128, as a persistent kernel.
// The arithmetic is that of isa_flash_kernel in pooled mode (hi + lo key
// parts, additive log2 n_j bias, per-row reference max moved past 2^8, true
// running max for the peak probability).  The key set is short (a few
// tiles), so each workgroup takes row tiles g, g + G, ... (G workgroups) and
// runs their key tiles as one sequence of steps j: the loads of the next row
// tile start while the current one finishes, and a row tile's output is
// written in the Y phase that starts the next.  Schedule as in
// isa_flash_pp_kernel, with three-stage rings and every direct load issued
// by group 0:
//   X_j  acc += V(j-1)^T P(j-1)^T, then S(j) = Khi(j) Q^T + Klo(j) Q^T
//   Y_j  [row tile change: output of the finished row tile] bias + softmax
//        of S(j) -> P(j); group 0 also loads Khi, Klo and the bias of step
//        j+2 and V of step j+1, then waits for its loads of Y_{j-1}
// Group 0 runs Y_j in phase 2j+1: K(t) is issued in phase 2t-3 and has
// landed by the end of 2t-1 (first read in 2t); its stage was last read in
// X_{t-3} (phase 2t-5).  V(t) is issued in phase 2t-1, lands by 2t+1 and is
// first read in 2t+2; its stage was last read in X_{t-2} (phase 2t-3).
// The bias of step t is read in Y_t (phases 2t+1, 2t+2) and its slot was
// last read in Y_{t-3} (phase 2t-4).  The queries of the next row tile are
// loaded into spare registers two steps before they are used.
__global__ __launch_bounds__(512) void isa_flash_pp_pooled_kernel(FlashArgs a) {
  typedef bf16x8 Op;
  constexpr int D = 128, BN = 64, BM = 256, NST = 3;
  constexpr int RB = D * 2, TB = BN * RB, NT = D / 32;
  static_assert(BM == kFlashRows, "tile mapping");
  // Khi ring, Klo ring, V ring
  __shared__ __attribute__((aligned(1024))) char smem[3 * NST * TB];
  __shared__ __attribute__((aligned(256))) float sbias[NST][BN];
  // the Q and O row maps, read from LDS where a row tile starts or ends, so
  // that they hold no registers across the tile loop
  __shared__ RowMap smap[2];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  if (tid == 0) {
    smap[0] = a.rmq;
    smap[1] = a.rmo;
  }
  __syncthreads();
  const int G = gridDim.x;
  const int n_tiles = a.n_wg;                  // row tiles over all heads
  const int nr = n_tiles > (int)blockIdx.x ? (n_tiles - 1 - (int)blockIdx.x) / G + 1 : 0;
  const int ntk = a.mk_pad / BN;               // key tiles per row tile (>= 2; padding keys carry bias -inf)
  const int total = nr * ntk;                  // steps with a key tile
  auto tile_bh = [&](int ri) { return (int)(blockIdx.x + (unsigned)ri * G) / a.row_tiles; };
  auto tile_rt = [&](int ri) { return (int)(blockIdx.x + (unsigned)ri * G) % a.row_tiles; };
  auto query_row = [&](int ri) -> int {
    const long long v = (long long)tile_rt(ri) * BM + w * 32 + l32;
    return v < a.Ns ? (int)v : -1;
  };
  auto load_q = [&](int ri, Op* q) {
    const int qr = query_row(ri);
    const RowMap m = smap[0];
    const bf16_t* qp = (const bf16_t*)a.Q + rm_head(m, tile_bh(ri)) + (long long)(qr < 0 ? 0 : qr) * m.sn + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) q[s] = *(const Op*)(qp + 16 * s);
  };

  const unsigned lds_kh = (unsigned)(size_t)(lds_char*)smem;
  const unsigned lds_kl = lds_kh + NST * TB, lds_v = lds_kh + 2 * NST * TB;
  const unsigned lds_b = (unsigned)(size_t)(lds_char*)&sbias[0][0];
  // Key tile of step t: a cursor walks the steps in order, so the head of
  // a row tile (a division) is formed once per row tile, not per load.
  struct Cursor { int kt, ri; long long row0; };   // row0: first pooled row of the head
  auto cursor_at = [&](int t) -> Cursor {
    const int ri = t / ntk;
    return Cursor{t - ri * ntk, ri, (long long)tile_bh(ri) * a.mk_pad};
  };
  auto advance = [&](Cursor& c) {
    if (++c.kt == ntk) {
      c.kt = 0;
      ++c.ri;
      c.row0 = (long long)tile_bh(c.ri) * a.mk_pad;
    }
  };
  // group 0, wave wg: rows 16*wg + 4*i + lane/16 (i = 0..3) of the key tile
  const unsigned wrow = __builtin_amdgcn_readfirstlane(16 * wg * RB);
  unsigned loff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = 16 * wg + 4 * i + (lane >> 4);
    loff[i] = (unsigned)lr * RB + (unsigned)(((lane & 15) ^ lds_swz(lr)) * 16);
  }
  auto load_tile = [&](const void* base, unsigned ring, int stage, const Cursor& c) {
    const char* G0 = (const char*)base + (c.row0 + c.kt * BN) * RB;
    const unsigned d0 = ring + (unsigned)stage * TB + wrow;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(d0 + 4 * i * RB, G0, loff[i]);
  };
  auto load_k = [&](int stage, const Cursor& c) {   // Khi, Klo and the bias (wave 0)
    load_tile(a.pkhi, lds_kh, stage, c);
    load_tile(a.pklo, lds_kl, stage, c);
    if (w == 0) dma4(lds_b + stage * BN * 4, a.pbias + c.row0 + c.kt * BN, (unsigned)lane * 4u);
  };

  const int kb = l32 * RB + ((h ^ lds_swz(l32)) * 16);
  auto koff = [&](int s) -> int { return kb ^ (32 * s); };
  int voff[NT][2];
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
  // pk: the row's largest term of l_run, rescaled with it (as in isa_flash_kernel)
  float m_ref = -INFINITY, pk = 0.f, l_run = 0.f;
  const float sc = a.scale_log2;
  Op qB[D / 16], qN[D / 16];

  // X phase: 16 P.V MFMAs, then 32 K.Q^T MFMAs (hi, lo of each key step),
  // operand reads issued ISA_PP_LOOKAHEAD MFMAs ahead
  auto pv_qk = [&](int vstage, const PTile& P, int kstage) -> STile {
    const lds_char* Vs = (const lds_char*)smem + 2 * NST * TB + vstage * TB;
    const lds_char* Khs = (const lds_char*)smem + kstage * TB;
    const lds_char* Kls = (const lds_char*)smem + NST * TB + kstage * TB;
    Op opv[16], opk[32];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + voff[t][0] + 16 * q * RB));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + voff[t][1] + 16 * q * RB));
        opv[4 * t + q] = __builtin_bit_cast(Op, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        opk[4 * q + 2 * ti] = *(const Op*)(Khs + koff(q) + 32 * ti * RB);
        opk[4 * q + 2 * ti + 1] = *(const Op*)(Kls + koff(q) + 32 * ti * RB);
      }
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m >> 2] = mma32(opv[m], P.p[m & 3], acc[m >> 2]);
    STile S;
    S.t[0] = f32x16{};
    S.t[1] = f32x16{};
#pragma unroll
    for (int m = 0; m < 32; ++m) S.t[(m >> 1) & 1] = mma32(opk[m], qB[m >> 2], S.t[(m >> 1) & 1]);
    pp_issue_order<ISA_PP_LOOKAHEAD, 16, 32>();
    return S;
  };
  // uni: the key tile is uniform (pooled_uniform_tile), its bias log2 b in
  // every column
  const float lb = log2f((float)a.b);
  auto softmax = [&](int stage, STile St, bool uni) -> PTile {
    f32x16* S = St.t;
    if (!uni) {
      const float* bs = sbias[stage];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 bb = *(const f32x4*)(bs + 32 * ti + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) S[ti][4 * g + e] = fmaf(S[ti][4 * g + e], sc, bb[e]);
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[ti][r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float smax = mx;            // uniform tiles: the largest S
    if (uni) mx = fmaf(mx, sc, lb);   // the largest S*sc + log2 b (the fma is monotone in S)
    const bool move = mx > m_ref + 8.0f;
    if (__ballot(move)) {
      const float m_new = move ? mx : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
      pk *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      m_ref = m_new;
    }
    PTile P;
    float psum = 0.f;
    const float lm = lb - m_ref;
    // the tile's largest term, with the expression of its terms below
    pk = fmaxf(pk, __builtin_amdgcn_exp2f(uni ? fmaf(smax, sc, lm) : mx - m_ref));
    if (uni) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[s >> 1][8 * (s & 1) + jj], sc, lm));
          psum += p;
          P.p[s][jj] = (__bf16)p;
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(S[s >> 1][8 * (s & 1) + jj] - m_ref);
          psum += p;
          P.p[s][jj] = (__bf16)p;
        }
      }
    }
    l_run += psum;
    return P;
  };
  // Output of a finished row tile, then the running state of the next.  The
  // stores go through buffer descriptors: a row past Ns (or a lane that
  // does not store) gets an offset beyond the buffer, which the hardware
  // drops, so every wave issues the same number of stores (kRowStores) and
  // the load waits below can count them.
  auto finish_row = [&](int ri) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int qr = query_row(ri);
    const long long bh = tile_bh(ri);
    const float inv = 1.0f / l_tot;
    constexpr unsigned kOut = 0x80000000u;   // beyond every buffer below (each under 2^31 bytes)
    const RowMap m = smap[1];
    const auto rO = __builtin_amdgcn_make_buffer_rsrc((bf16_t*)a.O + uniform64(rm_head(m, bh)), (short)0, a.o_span,
                                                      0x00020000);
    const unsigned oo = qr >= 0 ? (unsigned)qr * ((unsigned)m.sn * 2u) : kOut;
    // 16-byte chunk c = d / 8 = 4t + g of the row: lanes l and l + 32 hold
    // its halves.  For the chunk pair (2k, 2k + 1) one permlane32 swap per
    // word gives lane l all of chunk 2k and lane l + 32 all of chunk 2k + 1,
    // so a store writes 32 bytes of each row instead of 16.
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      unsigned x[2], y[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = 2 * k + u, t = c >> 2, g = c & 3;
        unsigned* dst = u ? y : x;
        dst[0] = pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
        dst[1] = pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto sw = __builtin_amdgcn_permlane32_swap(x[e], y[e], false, false);
        x[e] = sw[0];
        y[e] = sw[1];
      }
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{x[0], x[1], y[0], y[1]}, rO, oo + 16 * (2 * k + h), 0, 0);
    }
    const unsigned po = (qr >= 0 && h == 0) ? (unsigned)qr * 4 : kOut;
    const auto rP = __builtin_amdgcn_make_buffer_rsrc(a.peak + bh * a.Ns, (short)0, a.Ns * 4, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pk * inv), rP, po, 0, 0);
    if (a.lse) {
      const auto rL = __builtin_amdgcn_make_buffer_rsrc(a.lse + bh * a.Ns, (short)0, a.Ns * 4, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_ref + __builtin_log2f(l_tot)), rL, po, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    m_ref = -INFINITY;
    pk = 0.f;
    l_run = 0.f;
  };
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  if (total > 0) {
    load_q(0, qB);
    if (grp == 0) {
      load_k(0, cursor_at(0));
      load_tile(a.pv, lds_v, 0, cursor_at(0));
      if (total > 1) load_k(1, cursor_at(1));
    }
    // V stage 2 is first loaded in step 1; step 0 reads it as zeros
    u32x4* vz = (u32x4*)(smem + 2 * NST * TB + 2 * TB);
#pragma unroll
    for (int q = 0; q < TB / (16 * 512); ++q) vz[tid + 512 * q] = u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    phase_barrier();
    if (grp == 1) phase_barrier();   // group 1 runs one phase behind group 0
    STile S = {};
    PTile P = {};
    Cursor ck = cursor_at(2), cv = cursor_at(1);   // K of step j+2, V of step j+1
    // the head of the current row tile keeps a short last context block
    bool ctx_tail = pooled_ctx_tail(a, tile_bh(0));
    auto step = [&](auto ph, int j) {
      constexpr int Z = decltype(ph)::value;   // j % 3
      const int kt = j % ntk, ri = j / ntk;
      if (kt == 0 && j > 0 && ri < nr) ctx_tail = pooled_ctx_tail(a, tile_bh(ri));
      const bool uni = pooled_uniform_tile(a, kt, ctx_tail);
      // X_j at raised wave priority (step `total` computes an S that is not used)
      if (kt == 0 && j > 0) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qB[s] = qN[s];
      }
      __builtin_amdgcn_s_setprio(3);
      S = pv_qk((Z + 2) % 3, P, Z);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
      // Y_j
      if (kt == 0 && j > 0) finish_row(ri - 1);
      // the queries of the next row tile, two steps ahead of their first use
      const bool more_q = kt == ntk - 2 && ri + 1 < nr;
      if (more_q) load_q(ri + 1, qN);
      if (grp == 0) {
        const bool more_k = j + 2 < total, more_v = j + 1 < total;
        if (more_k) load_k((Z + 2) % 3, ck);
        if (more_v) load_tile(a.pv, lds_v, (Z + 1) % 3, cv);
        if (j < total) P = softmax(Z, S, uni);
        // the loads of Y_{j-1} have landed before the barrier that closes Y_j
        // (this step's 8 query loads or 9-10 output stores, if any, were
        // issued before its tiles)
        if (more_k && kt == 0 && j > 0) {
          if (a.lse) {
            if (w == 0) __builtin_amdgcn_s_waitcnt(0x0f77 | (1 << 14));   // vmcnt(23)
            else __builtin_amdgcn_s_waitcnt(0x0f76 | (1 << 14));          // vmcnt(22)
          } else {
            if (w == 0) __builtin_amdgcn_s_waitcnt(0x0f76 | (1 << 14));   // vmcnt(22)
            else __builtin_amdgcn_s_waitcnt(0x0f75 | (1 << 14));          // vmcnt(21)
          }
        } else if (more_k && more_q) {
          if (w == 0) __builtin_amdgcn_s_waitcnt(0x0f75 | (1 << 14));   // vmcnt(21)
          else __builtin_amdgcn_s_waitcnt(0x0f74 | (1 << 14));          // vmcnt(20)
        } else if (more_k) {
          if (w == 0) __builtin_amdgcn_s_waitcnt(0x0f7d);   // vmcnt(13)
          else __builtin_amdgcn_s_waitcnt(0x0f7c);          // vmcnt(12)
        } else if (more_v) {
          __builtin_amdgcn_s_waitcnt(0x0f74);               // vmcnt(4)
        } else {
          __builtin_amdgcn_s_waitcnt(0x0f70);               // vmcnt(0)
        }
      } else {
        if (j < total) P = softmax(Z, S, uni);
      }
      // (outside the group branch, so that the cursors stay scalar)
      advance(ck);
      advance(cv);
      phase_barrier();
    };
    for (int j = 0; j <= total; j += 3) {
      step(std::integral_constant<int, 0>{}, j);
      if (j + 1 <= total) step(std::integral_constant<int, 1>{}, j + 1);
      if (j + 2 <= total) step(std::integral_constant<int, 2>{}, j + 2);
    }
    // (step `total` wrote the last row tile)
    __builtin_amdgcn_s_waitcnt(0x0f70);
    if (grp == 0) phase_barrier();   // balances group 1's extra barrier
  }
}

// Merges the split partials of each full-route query row, in part order.
template <int D>
__global__ __launch_bounds__(256) void isa_flash_merge_kernel(FlashArgs a) {
  constexpr int TPR = D / 8;           // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;       // rows per workgroup
  long long gid = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int e = (threadIdx.x % TPR) * 8;
  const long long rows_head = (long long)a.row_tiles * kFlashRows;
  // the row's np partials: rows prow + s * pstep
  int np;
  long long prow, pstep;
  if (a.sk_G > 0) {
    // stream-K: the launch covers the rows of the range phase's row tiles;
    // its row tile Rs met ranges first .. last; one range wrote it whole
    const long long Rs = gid / kFlashRows, ub = Rs * a.sk_T;
    if (ub >= a.sk_U) return;
    np = sk_range_of(a, ub + a.sk_T - 1) - sk_range_of(a, ub) + 1;
    if (np == 1) return;
    prow = Rs * a.sk_P * kFlashRows + (gid - Rs * kFlashRows);
    pstep = kFlashRows;
    gid += ((long long)sk_rest_row(a, (int)Rs) - Rs) * kFlashRows;
  } else {
    np = a.nsplit;
    prow = gid * a.nsplit;
    pstep = 1;
  }
  const long long bh = gid / rows_head;
  const long long vrow = gid - bh * rows_head;
  if (bh >= a.n_wg) return;  // n_wg carries BH here
  const int qrow = route_row(a.q_list + bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  if (qrow < 0) return;
  constexpr int MAXS = kMaxSplits;
  float2 ml[MAXS];
  u32x4 po[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < np) {
      ml[s] = *(const float2*)(a.part_ml + (prow + s * pstep) * 2);
      po[s] = *(const u32x4*)(a.part_o + (prow + s * pstep) * D + e);
    }
  }
  float mstar = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < np) mstar = fmaxf(mstar, ml[s].x);
  // split s weighs in with its sum rescaled to the common max
  float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s >= np || ml[s].x == -INFINITY) continue;
    const float wgt = __builtin_amdgcn_exp2f((ml[s].x - mstar) * a.scale_log2) * ml[s].y;
    l += wgt;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] += wgt * __uint_as_float(po[s][k] << 16);
      o[2 * k + 1] += wgt * __uint_as_float(po[s][k] & 0xffff0000u);
    }
  }
  const float inv = 1.0f / l;
  if (a.lse && e == 0) a.lse[bh * a.Ns + qrow] = mstar * a.scale_log2 + __builtin_log2f(l);
  bf16_t* op = (bf16_t*)a.O + rm_head(a.rmo, bh) + (long long)qrow * a.rmo.sn + e;
  *(u32x4*)op = u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                      pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
}

// ---------------------------------------------------------------------------

static FlashArgs flash_args(const Layout& L, const Bufs& B) {
  FlashArgs a = {};
  a.Q = B.Q; a.O = B.O; a.K = B.K; a.V = B.V;
  a.rmq = L.q; a.rmo = L.o; a.rmk = L.k; a.rmv = L.v;
  a.o_span = (int)span_bytes(L.o, L.Ns, L.d, 2);
  a.Ns = L.Ns; a.Nk = L.Nk;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)L.d));
  a.nsplit = 1;
  if (B.ws) {
    a.ctx_rows = (const int*)(B.ws + L.off_ctxrows);
    a.key_rows = (const int*)(B.ws + L.off_keyrows);
    a.kept = (const int*)(B.ws + L.off_kept);
    a.pkhi = B.ws + L.off_pkhi;
    a.pklo = B.ws + L.off_pklo;
    a.pv = B.ws + L.off_pv;
    a.pbias = (const float*)(B.ws + L.off_pbias);
    a.peak = (float*)(B.ws + L.off_peak);
    a.part_o = (bf16_t*)(B.ws + L.off_part_o);
    a.part_ml = (float*)(B.ws + L.off_part_ml);
    a.lse = (float*)(B.ws + L.off_lse);
  }
  a.ctx_tok = L.ctx_tok;
  a.n_keytab = L.n_keytab;
  a.kc = L.kc; a.nb_c = L.nb_c; a.b = L.b; a.tail_c = L.tail_c;
  a.mk_pad = L.mk_pad;
  a.mk = L.mk;
  a.tail_s = L.tail_s;
  a.nb_s = L.nb_s;
  return a;
}

// The full route (gather mode) on the stream-K split that the layout set:
// a.sk_K rounds of whole row tiles on a grid of a.sk_R0 workgroups, then
// a.sk_G ranges over the remaining row tiles' key tiles.
template <int D, int KM, int RM>
static hipError_t flash_launch_sk(FlashArgs a, int ntiles, long long BH, hipStream_t s) {
  const long long R = (long long)a.row_tiles * BH, grid = a.sk_R0;
  a.sk_R0 = (int)(grid * a.sk_K);
  a.sk_grid = (int)grid;
  a.sk_q = (int)(R / 8);
  a.sk_x = (int)(R % 8);
  a.sk_T = ntiles;
  a.sk_U = (R - a.sk_R0) * ntiles;
  if (grid <= 0 || grid % 8 != 0 || a.sk_K < 0 || a.sk_R0 > R || (a.sk_U > 0) != (a.sk_G > 0) || a.sk_U < a.sk_G ||
      a.sk_P < 1 || a.sk_P > kMaxSplits)
    return hipErrorInvalidValue;
  const unsigned nwg = (unsigned)(a.sk_K > 0 ? grid : a.sk_G);
  // persistent form, one workgroup per round slot and range, when a
  // workgroup meets at most kPpsMaxItems row tiles and K and V share one row
  // map
  long long items = a.sk_K;
  if (a.sk_G > 0) items += ((a.sk_U + a.sk_G - 1) / a.sk_G - 1 + ntiles - 1) / ntiles + 1;
  if constexpr (D == 128) {
    if (kUsePps && items <= kPpsMaxItems && a.rmk.sb == a.rmv.sb && a.rmk.sh == a.rmv.sh && a.rmk.sn == a.rmv.sn) {
      hipLaunchKernelGGL(isa_flash_pps_kernel, dim3(nwg), dim3(512), 0, s, a);
      return hipGetLastError();
    }
  }
  // else the per-item kernel on the same grid, each workgroup's items one
  // after the other (d = 64, or K and V with different row maps)
  hipLaunchKernelGGL((isa_flash_pp_kernel<KM, RM, D>), dim3(nwg), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int D, int KM, int RM, bool WO, bool WP>
static hipError_t flash_launch(FlashArgs a, long long n_rows, long long keys, long long BH, hipStream_t s) {
  a.n_rows = n_rows;
  a.row_tiles = (int)((n_rows + kFlashRows - 1) / kFlashRows);
  const int ntiles = (int)((keys + 63) / 64);
  a.tiles_per_split = (ntiles + a.nsplit - 1) / a.nsplit;
  const long long nwg = (long long)a.row_tiles * BH * a.nsplit;
  if (nwg == 0) return hipSuccess;
  a.n_wg = (int)nwg;
  if constexpr ((D == 128 || D == 64) && KM != FK_POOLED && WO && !WP && kFlashWaves == 8) {
    if constexpr (KM == FK_GATHER && RM == FR_TABLE) {
      // (without the stream-K split -- d = 64 with few key tiles per
      // workgroup -- isa_flash_kernel on full_splits equal parts, below)
      if (a.sk_R0 > 0) return flash_launch_sk<D, KM, RM>(a, ntiles, BH, s);
    } else {
      hipLaunchKernelGGL((isa_flash_pp_kernel<KM, RM, D>), dim3((unsigned)nwg), dim3(512), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((isa_flash_kernel<D, KM, RM, kFlashWaves, WO, WP>), dim3((unsigned)nwg),
                     dim3(kFlashWaves * 64), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t flash_t(const Layout& L, const Bufs& B, FlashWhat what, hipStream_t s) {
  FlashArgs a = flash_args(L, B);
  switch (what) {
    case FlashWhat::kDense:
      return flash_launch<D, FK_DENSE, FR_IDENTITY, true, false>(a, L.Ns, L.Nk, L.BH, s);
    case FlashWhat::kContext:
      // context query rows: Q and O hold Nc rows per head (L.q and L.o
      // describe them)
      a.Ns = L.Nc;
      a.o_span = (int)span_bytes(L.o, L.Nc, L.d, 2);
      return flash_launch<D, FK_DENSE, FR_IDENTITY, true, false>(a, L.Nc, L.Nk, L.BH, s);
    case FlashWhat::kFull:
      a.q_list = (const int*)(B.ws + L.off_fullq);
      a.q_k = L.kq;
      a.nsplit = L.full_splits;
      a.sk_R0 = L.sk_grid;   // (the launch sets sk_R0 = sk_grid * sk_K)
      a.sk_K = L.sk_rounds;
      a.sk_G = L.sk_G;
      a.sk_P = L.sk_P;
      return flash_launch<D, FK_GATHER, FR_TABLE, true, false>(a, L.full_rows, (long long)L.Ns + L.ctx_tok,
                                                                L.BH, s);
    case FlashWhat::kFullMerge: {
      // the stream-K split of the d = 128 ping-pong kernels, else full_splits equal parts
      const bool sk = (D == 128 || D == 64) && kFlashWaves == 8 && L.sk_grid > 0;
      if ((sk ? L.sk_P : L.full_splits) <= 1 || L.full_rows == 0) return hipSuccess;
      a.q_list = (const int*)(B.ws + L.off_fullq);
      a.q_k = L.kq;
      a.nsplit = L.full_splits;
      a.n_rows = L.full_rows;
      a.row_tiles = (int)((L.full_rows + kFlashRows - 1) / kFlashRows);
      a.n_wg = (int)L.BH;
      long long rows = (long long)a.row_tiles * kFlashRows * L.BH;
      if (sk) {
        // the rows of the row tiles past the whole rounds
        a.sk_G = L.sk_G;
        a.sk_P = L.sk_P;
        a.sk_T = (int)((L.Ns + L.ctx_tok + 63) / 64);
        a.sk_R0 = L.sk_grid * L.sk_rounds;
        a.sk_K = L.sk_rounds;
        a.sk_grid = L.sk_grid;
        a.sk_q = (int)((long long)a.row_tiles * L.BH / 8);
        a.sk_x = (int)((long long)a.row_tiles * L.BH % 8);
        a.sk_U = ((long long)a.row_tiles * L.BH - a.sk_R0) * a.sk_T;
        rows -= (long long)a.sk_R0 * kFlashRows;
      }
      constexpr int RPB = 256 / (D / 8);
      hipLaunchKernelGGL((isa_flash_merge_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a);
      return hipGetLastError();
    }
    case FlashWhat::kSharpTaylor:
      if constexpr (D == 128 && kFlashWaves == 8) {
        if (L.mk_pad >= 2 * 64) {
          // persistent: one workgroup per compute unit, row tiles dealt round-robin
          a.n_rows = L.Ns;
          a.row_tiles = (int)((L.Ns + kFlashRows - 1) / kFlashRows);
          a.n_wg = (int)(a.row_tiles * L.BH);   // row tiles over all heads
          if (a.n_wg == 0) return hipSuccess;
          const int grid = a.n_wg < kCUs ? a.n_wg : kCUs;
          hipLaunchKernelGGL(isa_flash_pp_pooled_kernel, dim3((unsigned)grid), dim3(512), 0, s, a);
          return hipGetLastError();
        }
      }
      return flash_launch<D, FK_POOLED, FR_IDENTITY, true, true>(a, L.Ns, L.mk_pad, L.BH, s);
    case FlashWhat::kSharp:
      return flash_launch<D, FK_POOLED, FR_IDENTITY, false, true>(a, L.Ns, L.mk_pad, L.BH, s);
    case FlashWhat::kTaylor:
      a.q_list = (const int*)(B.ws + L.off_taylq);
      a.q_k = L.nb_s - L.kq;
      return flash_launch<D, FK_POOLED, FR_TABLE, true, false>(a, L.taylor_rows, L.mk_pad, L.BH, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_flash(const Layout& L, const Bufs& B, FlashWhat what, hipStream_t s) {
  return L.d == 128 ? flash_t<128>(L, B, what, s) : flash_t<64>(L, B, what, s);
}

}  // namespace isa
