// Argument checks, counts and workspace layout (no HIP calls).
//
// Counts of the two selections (the context pruning and the query routing of
// Lightning Unified Video Editing via In-Context Sparse Attention, English
// abstract): keeping a fraction f of n items keeps ceil(f*n - 1e-9) of them,
// clipped to [0, n], evaluated in double.
#include "isa_layout.h"

#include <math.h>

namespace isa {

static int kept_count(double f, int n) {
  double c = ceil(f * (double)n - 1e-9);
  if (c < 0) c = 0;
  if (c > n) c = n;
  return (int)c;
}

int choose_splits(int64_t units, int ntiles) {
  if (units <= 0 || ntiles <= 1) return 1;
  int best = 1;
  double best_cost = 0;
  for (int s = 1; s <= kMaxSplits && s <= ntiles; ++s) {
    const int per = (ntiles + s - 1) / s;
    if ((int64_t)per * (s - 1) >= ntiles) continue;  // an empty split
    const double rounds = ceil((double)(units * s) / kCUs);
    const double cost = rounds * (per + 3.0) + (s > 1 ? 0.02 * ntiles : 0.0);
    if (s == 1 || cost < best_cost * 0.98) {
      if (s == 1 || cost < best_cost) {
        best = s;
        best_cost = cost;
      }
    }
  }
  return best;
}

static size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Row map of one tensor [B,H,rows,d] from its isa_strides (all zero:
// contiguous).  Checks the signs, the 16-byte alignment of every used
// stride and the 32-bit spans the kernels address a head with.
static isa_status make_map(const isa_strides& s, int B, int H, int rows, int d, int es, RowMap* m) {
  int64_t sb, sh, sn;
  if (s.b == 0 && s.h == 0 && s.n == 0) {
    sn = d;
    sh = (int64_t)rows * d;
    sb = (int64_t)H * sh;
  } else {
    if (s.b < 0 || s.h < 0 || s.n < 0) return ISA_ERR_INVALID_ARGUMENT;
    sb = s.b;
    sh = s.h;
    sn = s.n;
  }
  // magnitudes first, so that the products below cannot overflow
  if (sn >= kMaxRowStride || sb >= (int64_t(1) << 50) || sh >= (int64_t(1) << 50)) return ISA_ERR_UNSUPPORTED;
  if ((B > 1 && (sb * es) % 16) || (H > 1 && (sh * es) % 16) || (rows > 1 && (sn * es) % 16))
    return ISA_ERR_INVALID_ARGUMENT;
  if (sn * es >= kMaxRowStride) return ISA_ERR_UNSUPPORTED;
  m->sb = sb;
  m->sh = sh;
  m->sn = (int32_t)sn;
  m->H = H;
  m->hmul = H > 1 ? (uint32_t)(((uint64_t(1) << 32) + (uint64_t)H - 1) / (uint64_t)H) : 0u;
  m->pad = 0;
  if (span_bytes(*m, rows, d, es) >= kMaxSpan) return ISA_ERR_UNSUPPORTED;
  return ISA_OK;
}

bool map_disjoint(const RowMap& m, int B, int rows, int d) {
  // dimensions of more than one element, by stride: each stride must step
  // past the whole extent of the dimensions below it
  int64_t st[4] = {1, m.sn, m.sh, m.sb};
  int64_t n[4] = {d, rows, m.H, B};
  int k = 0;
  int64_t ss[4], nn[4];
  for (int i = 0; i < 4; ++i)
    if (n[i] > 1) {
      ss[k] = st[i];
      nn[k] = n[i];
      ++k;
    }
  for (int i = 1; i < k; ++i)
    for (int j = i; j > 0 && ss[j] < ss[j - 1]; --j) {
      int64_t t = ss[j]; ss[j] = ss[j - 1]; ss[j - 1] = t;
      t = nn[j]; nn[j] = nn[j - 1]; nn[j - 1] = t;
    }
  if (k > 0 && ss[0] < 1) return false;
  for (int i = 1; i < k; ++i)
    if (ss[i] < ss[i - 1] * nn[i - 1]) return false;
  return true;
}

isa_status context_maps(const isa_desc* desc, Layout* L) {
  if (!desc || !L) return ISA_ERR_INVALID_ARGUMENT;
  isa_status st;
  if ((st = make_map(desc->q, desc->B, desc->H, L->Nc, L->d, L->es, &L->q)) != ISA_OK) return st;
  if ((st = make_map(desc->o, desc->B, desc->H, L->Nc, L->d, L->es, &L->o)) != ISA_OK) return st;
  if (!map_disjoint(L->o, desc->B, L->Nc, L->d)) return ISA_ERR_INVALID_ARGUMENT;
  return ISA_OK;
}

isa_status check_tensors(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return ISA_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)ptrs[i] & 15u) != 0) return ISA_ERR_INVALID_ARGUMENT;
  }
  return ISA_OK;
}

isa_status check_workspace(const void* ws, size_t bytes, size_t need) {
  if (!ws) return ISA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)ws % kWsAlign) != 0 || bytes < need) return ISA_ERR_WORKSPACE;
  return ISA_OK;
}

isa_status make_layout(const isa_desc* desc, Layout* L) {
  if (!desc || !L) return ISA_ERR_INVALID_ARGUMENT;
  const isa_desc& D = *desc;
  if (D.B < 1 || D.H < 1 || D.Ns < 1 || D.Nc < 0 || D.b < 1) return ISA_ERR_INVALID_ARGUMENT;
  if (!(D.rho >= 0.0 && D.rho <= 1.0) || !(D.gamma >= 0.0 && D.gamma <= 1.0))
    return ISA_ERR_INVALID_ARGUMENT;  // also rejects NaN
  if (D.d != 64 && D.d != 128) return ISA_ERR_UNSUPPORTED;
  if (D.b > 256) return ISA_ERR_UNSUPPORTED;
  if (D.dtype != ISA_BF16 && D.dtype != ISA_F32) return ISA_ERR_UNSUPPORTED;
  if (D.reserved != 0) return ISA_ERR_INVALID_ARGUMENT;
  const int64_t nk = (int64_t)D.Ns + D.Nc;
  if (nk > kMaxRows) return ISA_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)D.B * D.H;
  if (bh > kMaxBH) return ISA_ERR_UNSUPPORTED;
  {
    const int es = D.dtype == ISA_BF16 ? 2 : 4;
    isa_status st;
    if ((st = make_map(D.q, D.B, D.H, D.Ns, D.d, es, &L->q)) != ISA_OK) return st;
    if ((st = make_map(D.k, D.B, D.H, (int)nk, D.d, es, &L->k)) != ISA_OK) return st;
    if ((st = make_map(D.v, D.B, D.H, (int)nk, D.d, es, &L->v)) != ISA_OK) return st;
    if ((st = make_map(D.o, D.B, D.H, D.Ns, D.d, es, &L->o)) != ISA_OK) return st;
    if (!map_disjoint(L->o, D.B, D.Ns, D.d)) return ISA_ERR_INVALID_ARGUMENT;
  }

  L->BH = bh;
  L->Ns = D.Ns;
  L->Nc = D.Nc;
  L->Nk = (int)nk;
  L->d = D.d;
  L->b = D.b;
  L->es = D.dtype == ISA_BF16 ? 2 : 4;
  L->nb_s = (D.Ns + D.b - 1) / D.b;
  L->nb_c = (D.Nc + D.b - 1) / D.b;
  L->M = L->nb_s + L->nb_c;
  L->kc = kept_count(D.rho, L->nb_c);
  L->kq = kept_count(D.gamma, L->nb_s);
  L->mk = L->nb_s + L->kc;
  L->mk_pad = (L->mk + kTileKeys - 1) / kTileKeys * kTileKeys;
  L->tail_s = D.Ns - (L->nb_s - 1) * D.b;
  L->tail_c = L->nb_c ? D.Nc - (L->nb_c - 1) * D.b : 0;
  L->sal_tiles = (L->nb_s + kSalRows - 1) / kSalRows;
  L->ctx_tok = (int64_t)L->kc * D.b;
  L->full_rows = (int64_t)L->kq * D.b;
  L->taylor_rows = (int64_t)(L->nb_s - L->kq) * D.b;
  {
    const int64_t row_tiles = (L->full_rows + kFlashRows - 1) / kFlashRows;
    const int ntiles = (int)((D.Ns + L->ctx_tok + 63) / 64);
    L->full_splits = L->es == 2 ? choose_splits(bh * row_tiles, ntiles) : 1;
    L->n_keytab = ntiles * kTileKeys;
    L->sk_grid = L->sk_rounds = L->sk_G = L->sk_P = 0;
    if (L->es == 2 && (D.d == 128 || D.d == 64) && row_tiles > 0) {
      // whole row tiles in at most 5 rounds of a multiple of the compute
      // unit count, the rest in ranges of equal length: at least
      // (T - 1) / (kMaxSplits - 1) units, so that a row tile of T units
      // meets at most kMaxSplits ranges, and min(8, T) (fixed costs); at
      // most one range per workgroup.  A range is then shorter than 2 T
      // units (or than T), so a workgroup meets at most 5 + 3 row tiles.
      const int64_t R = bh * row_tiles, T = ntiles;
      const int64_t G = kCUs * ((R + kCUs * 5 - 1) / (kCUs * 5));
      const int64_t rounds = R / G, rest = R - rounds * G, U = rest * T;
      L->sk_grid = (int)G;
      L->sk_rounds = (int)rounds;
      L->sk_P = 1;
      if (rest > 0) {
        int64_t wmin = T > 1 ? (T - 1 + kMaxSplits - 2) / (kMaxSplits - 1) : 1;
        if (wmin < 8) wmin = T < 8 ? T : 8;
        int64_t Gs = U / wmin < G ? U / wmin : G;
        if (Gs < 1) Gs = 1;
        const int64_t W = U / Gs;   // the shortest range
        L->sk_G = (int)Gs;
        L->sk_P = (int)((T - 1 + W - 1) / W + 1);
        if (L->sk_P > kMaxSplits) L->sk_P = kMaxSplits;   // (not reached: W >= wmin or Gs = 1)
        // Or, when that costs less, every remaining row tile cut into P equal
        // parts (rest * P ranges, aligned to the row tiles): a workgroup then
        // runs ceil(T / P) key tiles as one item, against the longest range's
        // key tiles and the items it meets.  Costs in key tiles, with
        // kItemCost per item (its queries, first tiles and output).
        const int64_t wmax = (U + Gs - 1) / Gs;
        const int64_t cost_ranges = wmax + kItemCost * ((wmax - 1 + T - 1) / T + 1);
        int64_t P = G / rest;
        if (P > kMaxSplits) P = kMaxSplits;
        if (P > T) P = T;
        if ((T + P - 1) / P + kItemCost <= cost_ranges) {
          L->sk_G = (int)(rest * P);
          L->sk_P = (int)P;
        }
      }
      // d = 64 with few key tiles per workgroup: the first-design kernel,
      // whose shorter start-up wins there, on full_splits equal parts
      const int64_t per_wg = rounds * T + (rest > 0 ? (U + L->sk_G - 1) / L->sk_G : 0);
      if (D.d == 64 && per_wg < kPpMinTiles64) L->sk_grid = L->sk_rounds = L->sk_G = L->sk_P = 0;
    }
  }

  const size_t d = (size_t)D.d;
  const size_t pk_es = L->es;  // packed pooled keys/values: bf16 or f32
  size_t o = 0;
  auto take = [&](size_t* off, size_t bytes) {
    *off = o;
    o = align_up(o + (bytes ? bytes : 1));
  };
  take(&L->off_qbar, bh * L->nb_s * d * 4);
  take(&L->off_kbar, bh * L->M * d * 4);
  take(&L->off_vbar, bh * L->M * d * 4);
  take(&L->off_salp, bh * L->sal_tiles * L->nb_c * 8);
  take(&L->off_sal, bh * L->nb_c * 8);
  take(&L->off_kept, bh * L->kc * 4);
  take(&L->off_pkhi, bh * L->mk_pad * d * pk_es);
  take(&L->off_pklo, L->es == 2 ? bh * L->mk_pad * d * 2 : 0);
  take(&L->off_pv, bh * L->mk_pad * d * pk_es);
  take(&L->off_pbias, bh * L->mk_pad * 4);
  take(&L->off_ctxrows, bh * L->ctx_tok * 4);
  take(&L->off_keyrows, bh * (size_t)L->n_keytab * 4);
  take(&L->off_peak, bh * D.Ns * 4);
  take(&L->off_sh, bh * L->nb_s * 8);
  take(&L->off_fullq, bh * L->kq * 4);
  take(&L->off_taylq, bh * (L->nb_s - L->kq) * 4);
  {
    // split partials: the FP8 variant and d = 64 split every row tile into
    // full_splits parts, the d = 128 full route the row tiles past the whole
    // rounds into up to sk_P
    const int64_t row_tiles = (L->full_rows + kFlashRows - 1) / kFlashRows;
    int64_t prow = L->full_splits > 1 ? bh * row_tiles * kFlashRows * L->full_splits : 0;
    const int64_t prow_sk =
        L->sk_P > 1 ? (bh * row_tiles - (int64_t)L->sk_rounds * L->sk_grid) * kFlashRows * L->sk_P : 0;
    if (prow_sk > prow) prow = prow_sk;
    take(&L->off_part_o, prow * d * 2);
    take(&L->off_part_ml, prow * 2 * 4);
  }
  take(&L->off_lse, bh * D.Ns * 4);
  L->total = o;
  return ISA_OK;
}

isa_status make_bwd_layout(const Layout& L, BwdLayout* B) {
  if (!B) return ISA_ERR_INVALID_ARGUMENT;
  if (L.es != 2) return ISA_ERR_UNSUPPORTED;
  const size_t bh = (size_t)L.BH, d = (size_t)L.d;
  B->dkv_key_tiles = (L.mk + kBwdKeys - 1) / kBwdKeys;
  // pooled dK/dV: split the Taylor rows so that about four workgroups per
  // compute unit exist, never more splits than row steps
  const int64_t steps = (L.taylor_rows + kBwdRows - 1) / kBwdRows;
  const int64_t units = (int64_t)bh * B->dkv_key_tiles;
  int64_t sp = units > 0 ? (4 * (int64_t)kCUs + units - 1) / units : 1;
  sp = sp < 1 ? 1 : sp;
  sp = sp > steps ? steps : sp;
  sp = sp > 64 ? 64 : sp;
  B->dkv_splits = (int)(sp < 1 ? 1 : sp);
  size_t o = 0;
  auto take = [&](size_t* off, size_t bytes) {
    *off = o;
    o = align_up(o + (bytes ? bytes : 1));
  };
  take(&B->off_delta, bh * L.Ns * 4);
  take(&B->off_part_dkv, (size_t)B->dkv_splits * bh * L.mk_pad * 2 * d * 4);
  take(&B->off_dkvbar, bh * L.mk_pad * 2 * d * 4);
  {
    // dQ partials: d = 64 splits every row tile into full_splits key ranges;
    // d = 128 cuts only the row tiles of a part-filled last round, into
    // dq_parts key ranges
    const int64_t row_tiles = (L.full_rows + kFlashRows - 1) / kFlashRows;
    const int64_t items = (int64_t)bh * row_tiles, ktiles = (L.Ns + L.ctx_tok + 63) / 64;
    B->dq_rounds = (int)(items / kCUs);
    B->dq_rest = (int)(items % kCUs);
    int64_t P = B->dq_rest > 0 ? kCUs / B->dq_rest : 0;
    if (P > kMaxSplits) P = kMaxSplits;
    if (P > ktiles) P = ktiles;
    B->dq_parts = (L.d == 128 && P >= 2) ? (int)P : 0;
    // (room for both: a build without the d = 128 ping-pong dQ kernel splits
    // every row tile)
    int64_t prow = L.full_splits > 1 ? (int64_t)bh * row_tiles * kFlashRows * L.full_splits : 0;
    const int64_t prow_cut = B->dq_parts ? (int64_t)B->dq_rest * B->dq_parts * kFlashRows : 0;
    if (prow_cut > prow) prow = prow_cut;
    take(&B->off_part_dq, prow * d * 4);
  }
  B->n_rowtab = (int)((L.full_rows + 63) / 64 * 64);
  {
    // the last round of the d = 128 full-route dK/dV items, when at most
    // half full, cut along the query tiles so that it fills the compute units
    const int64_t items = (int64_t)bh * ((L.Ns + L.ctx_tok + kBwdKeys - 1) / kBwdKeys);
    const int64_t qtiles = B->n_rowtab / 64;
    B->kv_rounds = (int)(items / kCUs);
    B->kv_rest = (int)(items % kCUs);
    int64_t P = B->kv_rest > 0 ? kCUs / B->kv_rest : 0;
    if (P > kBwdMaxParts) P = kBwdMaxParts;
    if (P > qtiles) P = qtiles;
    B->kv_parts = (L.d == 128 && P >= 2) ? (int)P : 0;
    take(&B->off_part_kv, (size_t)(B->kv_parts ? B->kv_rest * B->kv_parts : 0) * kBwdKeys * d * 4);
  }
  take(&B->off_rrow, bh * (size_t)B->n_rowtab * 4);
  take(&B->off_rlse, bh * (size_t)B->n_rowtab * 4);
  take(&B->off_rdel, bh * (size_t)B->n_rowtab * 4);
  B->total = o;
  return ISA_OK;
}

isa_status make_fp8_layout(const Layout& L, Fp8Layout* F) {
  if (!F) return ISA_ERR_INVALID_ARGUMENT;
  if (L.es != 2) return ISA_ERR_UNSUPPORTED;
  const size_t bh = (size_t)L.BH, d = (size_t)L.d;
  const int64_t nk = (int64_t)L.Ns + L.ctx_tok;
  F->ntile = (int)((nk + 63) / 64);
  F->nkp = F->ntile * 64;
  size_t o = 0;
  auto take = [&](size_t* off, size_t bytes) {
    *off = o;
    o = align_up(o + (bytes ? bytes : 1));
  };
  take(&F->off_k8, bh * F->nkp * d);
  take(&F->off_ks, bh * F->nkp * (d / 32));
  take(&F->off_v8t, bh * F->ntile * d * 64);
  take(&F->off_vs, bh * F->ntile * d * 2);
  F->total = o;
  return ISA_OK;
}

}  // namespace isa

extern "C" isa_status isa_fp8_workspace_size(const isa_desc* desc, size_t* bytes) {
  if (!bytes) return ISA_ERR_INVALID_ARGUMENT;
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  isa::Fp8Layout F;
  st = isa::make_fp8_layout(L, &F);
  if (st != ISA_OK) return st;
  *bytes = F.total;
  return ISA_OK;
}

extern "C" isa_status isa_backward_workspace_size(const isa_desc* desc, size_t* bytes) {
  if (!bytes) return ISA_ERR_INVALID_ARGUMENT;
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  isa::BwdLayout B;
  st = isa::make_bwd_layout(L, &B);
  if (st != ISA_OK) return st;
  *bytes = B.total;
  return ISA_OK;
}

extern "C" isa_status isa_get_counts(const isa_desc* desc, isa_counts* out) {
  if (!out) return ISA_ERR_INVALID_ARGUMENT;
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  out->nb_s = L.nb_s;
  out->nb_c = L.nb_c;
  out->kc = L.kc;
  out->kq = L.kq;
  out->m_kept = L.mk;
  out->reserved = 0;
  out->full_keys = (int64_t)L.Ns + L.ctx_tok;
  return ISA_OK;
}

extern "C" isa_status isa_workspace_size(const isa_desc* desc, size_t* bytes) {
  if (!bytes) return ISA_ERR_INVALID_ARGUMENT;
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  *bytes = L.total;
  return ISA_OK;
}

extern "C" isa_status isa_plan_views(const isa_desc* desc, void* workspace, size_t workspace_bytes,
                                     isa_plan_view* out) {
  if (!out || !workspace) return ISA_ERR_INVALID_ARGUMENT;
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  if (((uintptr_t)workspace % isa::kWsAlign) != 0 || workspace_bytes < L.total) return ISA_ERR_WORKSPACE;
  char* w = (char*)workspace;
  out->qbar = (const float*)(w + L.off_qbar);
  out->kbar = (const float*)(w + L.off_kbar);
  out->vbar = (const float*)(w + L.off_vbar);
  out->sal = (const double*)(w + L.off_sal);
  out->kept_ctx = (const int32_t*)(w + L.off_kept);
  out->sh = (const double*)(w + L.off_sh);
  out->full_q = (const int32_t*)(w + L.off_fullq);
  out->taylor_q = (const int32_t*)(w + L.off_taylq);
  return isa_get_counts(desc, &out->counts);
}

extern "C" const char* isa_status_string(isa_status s) {
  switch (s) {
    case ISA_OK: return "ISA_OK";
    case ISA_ERR_INVALID_ARGUMENT: return "ISA_ERR_INVALID_ARGUMENT: null pointer, misaligned pointer or value out of range";
    case ISA_ERR_UNSUPPORTED: return "ISA_ERR_UNSUPPORTED: d must be 64 or 128, b at most 256, dtype bf16 or f32";
    case ISA_ERR_WORKSPACE: return "ISA_ERR_WORKSPACE: workspace too small or not 256-byte aligned";
    case ISA_ERR_DEVICE: return "ISA_ERR_DEVICE: a kernel launch failed (see isa_last_error)";
  }
  return "unknown isa_status";
}
