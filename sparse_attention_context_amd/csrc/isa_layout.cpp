// Argument checks, counts and workspace layout (no HIP calls).
//
// Counts follow the reading of "prune redundant context" and "routes
// high-error queries to full attention" (Lightning Unified Video Editing via
// In-Context Sparse Attention, English abstract): a fraction f of n items
// keeps ceil(f*n - 1e-9) of them, clipped to [0, n], evaluated in double.
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

isa_status make_layout(const isa_desc* desc, Layout* L) {
  if (!desc || !L) return ISA_ERR_INVALID_ARGUMENT;
  const isa_desc& D = *desc;
  if (D.B < 1 || D.H < 1 || D.Ns < 1 || D.Nc < 0 || D.b < 1) return ISA_ERR_INVALID_ARGUMENT;
  if (!(D.rho >= 0.0 && D.rho <= 1.0) || !(D.gamma >= 0.0 && D.gamma <= 1.0))
    return ISA_ERR_INVALID_ARGUMENT;  // also rejects NaN
  if (D.d != 64 && D.d != 128) return ISA_ERR_UNSUPPORTED;
  if (D.b > 256) return ISA_ERR_UNSUPPORTED;
  if (D.dtype != ISA_BF16 && D.dtype != ISA_F32) return ISA_ERR_UNSUPPORTED;
  const int64_t nk = (int64_t)D.Ns + D.Nc;
  if (nk > (int64_t(1) << 30)) return ISA_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)D.B * D.H;
  if (bh > (int64_t(1) << 24)) return ISA_ERR_UNSUPPORTED;

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
    const int64_t prow = L->full_splits > 1 ? bh * ((L->full_rows + kFlashRows - 1) / kFlashRows) * kFlashRows * L->full_splits : 0;
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
    const int64_t prow = L.full_splits > 1 ? (int64_t)bh * ((L.full_rows + kFlashRows - 1) / kFlashRows) * kFlashRows * L.full_splits : 0;
    take(&B->off_part_dq, prow * d * 4);
  }
  B->n_rowtab = (int)((L.full_rows + 63) / 64 * 64);
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
