// C-ABI entry points declared in include/isa.h.  Each validates on the
// host, then enqueues the kernel chain on the caller's stream.
#include <stdio.h>

#include "isa_kernels.h"

namespace {

thread_local char g_last_error[256] = "";

}  // namespace

isa_status isa::device_status(hipError_t e) {
  if (e == hipSuccess) return ISA_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s (%d)", hipGetErrorString(e), (int)e);
  return ISA_ERR_DEVICE;
}

namespace {

using isa::device_status;

isa_status check_io(const void* Q, const void* K, const void* V, const void* O, bool need_o) {
  const void* p[4] = {Q, K, V, O};
  return isa::check_tensors(p, need_o ? 4 : 3);
}

isa_status check_ws(const isa::Layout& L, const void* ws, size_t bytes) {
  return isa::check_workspace(ws, bytes, L.total);
}

#define ISA_RUN(call)                             \
  do {                                            \
    isa_status st_ = device_status(call);         \
    if (st_ != ISA_OK) return st_;                \
  } while (0)

// Pooling, saliency, context pre-selection and packing of the kept set
// (with the pooling of the kept context blocks' V).
isa_status select_context(const isa::Layout& L, const isa::Bufs& B, hipStream_t s, isa::Tracer* tr = nullptr) {
  if (tr) tr->mark("pool");
  ISA_RUN(isa::launch_pool(L, B, s));
  if (tr) tr->mark("saliency");
  ISA_RUN(isa::launch_saliency(L, B, s));
  if (tr) tr->mark("select_ctx");
  ISA_RUN(isa::launch_select_ctx(L, B, s));
  if (tr) tr->mark("pool_kept_v");
  ISA_RUN(isa::launch_pool_pack(L, B, s));
  return ISA_OK;
}

}  // namespace

extern "C" isa_status isa_plan(const isa_desc* desc, const void* Q, const void* K, const void* V,
                               void* workspace, size_t workspace_bytes, void* stream) {
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  if ((st = check_io(Q, K, V, nullptr, false)) != ISA_OK) return st;
  if ((st = check_ws(L, workspace, workspace_bytes)) != ISA_OK) return st;
  const isa::Bufs B{Q, K, V, nullptr, (char*)workspace};
  hipStream_t s = (hipStream_t)stream;
  if ((st = select_context(L, B, s)) != ISA_OK) return st;
  ISA_RUN(isa::launch_pooled_attention(L, B, 1, s));
  ISA_RUN(isa::launch_select_q(L, B, s));
  return ISA_OK;
}

extern "C" isa_status isa_forward(const isa_desc* desc, const void* Q, const void* K, const void* V,
                                  void* O, void* workspace, size_t workspace_bytes, void* stream) {
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  if ((st = check_io(Q, K, V, O, true)) != ISA_OK) return st;
  if ((st = check_ws(L, workspace, workspace_bytes)) != ISA_OK) return st;
  const isa::Bufs B{Q, K, V, O, (char*)workspace};
  hipStream_t s = (hipStream_t)stream;
  if (L.taylor_rows > 0) ISA_RUN(isa::launch_pooled_attention(L, B, 2, s));
  if (L.kq > 0) {
    ISA_RUN(isa::launch_full_attention(L, B, false, s));
    ISA_RUN(isa::launch_full_merge(L, B, s));
  }
  return ISA_OK;
}

// The launches of isa_attention on validated arguments.
isa_status isa::run_attention(const isa::Layout& L, const isa::Bufs& B, hipStream_t s, bool trace) {
  isa::Tracer tr(trace ? s : nullptr, trace);
  isa_status st;
  if ((st = select_context(L, B, s, &tr)) != ISA_OK) return st;
  // sharpness of every row; unless every block goes to full attention the
  // same pass also writes the Taylor output of every row
  tr.mark(L.kq == L.nb_s ? "sharp" : "sharp_taylor");
  ISA_RUN(isa::launch_pooled_attention(L, B, L.kq == L.nb_s ? 1 : 0, s));
  tr.mark("select_q");
  ISA_RUN(isa::launch_select_q(L, B, s));
  if (L.kq > 0) {
    tr.mark("full");
    ISA_RUN(isa::launch_full_attention(L, B, false, s));
    tr.mark("full_merge");
    ISA_RUN(isa::launch_full_merge(L, B, s));
  }
  return ISA_OK;
}

extern "C" isa_status isa_attention(const isa_desc* desc, const void* Q, const void* K, const void* V,
                                    void* O, void* workspace, size_t workspace_bytes, void* stream) {
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  if ((st = check_io(Q, K, V, O, true)) != ISA_OK) return st;
  if ((st = check_ws(L, workspace, workspace_bytes)) != ISA_OK) return st;
  return isa::run_attention(L, isa::Bufs{Q, K, V, O, (char*)workspace}, (hipStream_t)stream);
}

extern "C" isa_status isa_dense_forward(const isa_desc* desc, const void* Q, const void* K, const void* V,
                                        void* O, void* stream) {
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  if ((st = check_io(Q, K, V, O, true)) != ISA_OK) return st;
  const isa::Bufs B{Q, K, V, O, nullptr};
  ISA_RUN(isa::launch_full_attention(L, B, true, (hipStream_t)stream));
  return ISA_OK;
}

namespace {

isa_status fp8_prepare(const isa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                       const void* ws, size_t ws_bytes, const void* fws, size_t fws_bytes, isa::Layout* L,
                       isa::Fp8Layout* F) {
  isa_status st = isa::make_layout(desc, L);
  if (st != ISA_OK) return st;
  // the FP8 full route at d = 128 takes the bf16 route's stream-K split; at
  // d = 64 it splits every row tile's keys into full_splits equal parts (the
  // workspace holds room for either split)
  if (L->d != 128) L->sk_grid = L->sk_rounds = L->sk_G = L->sk_P = 0;
  if ((st = isa::make_fp8_layout(*L, F)) != ISA_OK) return st;
  if ((st = check_io(Q, K, V, O, true)) != ISA_OK) return st;
  if ((st = check_ws(*L, ws, ws_bytes)) != ISA_OK) return st;
  return isa::check_workspace(fws, fws_bytes, F->total);
}

}  // namespace

extern "C" isa_status isa_attention_fp8(const isa_desc* desc, const void* Q, const void* K, const void* V, void* O,
                                        void* workspace, size_t workspace_bytes, void* fp8_workspace,
                                        size_t fp8_workspace_bytes, void* stream) {
  isa::Layout L;
  isa::Fp8Layout F;
  isa_status st = fp8_prepare(desc, Q, K, V, O, workspace, workspace_bytes, fp8_workspace, fp8_workspace_bytes, &L, &F);
  if (st != ISA_OK) return st;
  const isa::Bufs B{Q, K, V, O, (char*)workspace};
  hipStream_t s = (hipStream_t)stream;
  if ((st = select_context(L, B, s)) != ISA_OK) return st;
  ISA_RUN(isa::launch_pooled_attention(L, B, L.kq == L.nb_s ? 1 : 0, s));
  ISA_RUN(isa::launch_select_q(L, B, s));
  if (L.kq > 0) {
    ISA_RUN(isa::launch_fp8(L, F, B, (char*)fp8_workspace, true, s));
    ISA_RUN(isa::launch_fp8(L, F, B, (char*)fp8_workspace, false, s));
    ISA_RUN(isa::launch_full_merge(L, B, s));
  }
  return ISA_OK;
}

extern "C" isa_status isa_run_fp8_stage(const isa_desc* desc, int stage, const void* Q, const void* K, const void* V,
                                        void* O, void* workspace, size_t workspace_bytes, void* fp8_workspace,
                                        size_t fp8_workspace_bytes, void* stream) {
  if (stage < ISA_FP8_PACK || stage > ISA_FP8_FULL_MERGE) return ISA_ERR_INVALID_ARGUMENT;
  isa::Layout L;
  isa::Fp8Layout F;
  isa_status st = fp8_prepare(desc, Q, K, V, O, workspace, workspace_bytes, fp8_workspace, fp8_workspace_bytes, &L, &F);
  if (st != ISA_OK) return st;
  if (L.kq == 0) return ISA_OK;
  const isa::Bufs B{Q, K, V, O, (char*)workspace};
  hipStream_t s = (hipStream_t)stream;
  if (stage == ISA_FP8_FULL_MERGE) ISA_RUN(isa::launch_full_merge(L, B, s));
  else ISA_RUN(isa::launch_fp8(L, F, B, (char*)fp8_workspace, stage == ISA_FP8_PACK, s));
  return ISA_OK;
}

extern "C" isa_status isa_context_forward(const isa_desc* desc, const void* Qc, const void* K, const void* V,
                                          void* Oc, void* stream) {
  if (!desc) return ISA_ERR_INVALID_ARGUMENT;
  // Q and O hold the Nc context rows here: their strides are checked against
  // that row count by context_maps, not as source rows by make_layout
  isa_desc D = *desc;
  D.q = isa_strides{0, 0, 0};
  D.o = isa_strides{0, 0, 0};
  isa::Layout L;
  isa_status st = isa::make_layout(&D, &L);
  if (st != ISA_OK) return st;
  if (L.es != 2) return ISA_ERR_UNSUPPORTED;
  if ((st = isa::context_maps(desc, &L)) != ISA_OK) return st;
  if ((st = check_io(Qc, K, V, Oc, true)) != ISA_OK) return st;
  if (L.Nc == 0) return ISA_OK;
  const isa::Bufs B{Qc, K, V, Oc, nullptr};
  ISA_RUN(isa::launch_flash(L, B, isa::FlashWhat::kContext, (hipStream_t)stream));
  return ISA_OK;
}

extern "C" isa_status isa_run_stage(const isa_desc* desc, int stage, const void* Q, const void* K,
                                    const void* V, void* O, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  if (stage < ISA_STAGE_POOL || stage > ISA_STAGE_FULL_MERGE) return ISA_ERR_INVALID_ARGUMENT;
  const bool writes_o = stage == ISA_STAGE_SHARP_TAYLOR || stage == ISA_STAGE_TAYLOR || stage == ISA_STAGE_FULL ||
                        stage == ISA_STAGE_FULL_MERGE;
  if ((st = check_io(Q, K, V, O, writes_o)) != ISA_OK) return st;
  if ((st = check_ws(L, workspace, workspace_bytes)) != ISA_OK) return st;
  const isa::Bufs B{Q, K, V, O, (char*)workspace};
  hipStream_t s = (hipStream_t)stream;
  switch (stage) {
    case ISA_STAGE_POOL: ISA_RUN(isa::launch_pool(L, B, s)); break;
    case ISA_STAGE_SALIENCY: ISA_RUN(isa::launch_saliency(L, B, s)); break;
    case ISA_STAGE_SELECT_CTX: ISA_RUN(isa::launch_select_ctx(L, B, s)); break;
    case ISA_STAGE_POOL_KEPT_V: ISA_RUN(isa::launch_pool_pack(L, B, s)); break;
    case ISA_STAGE_PACK: break;   // packed by the launch of ISA_STAGE_POOL_KEPT_V
    case ISA_STAGE_SHARP_TAYLOR: ISA_RUN(isa::launch_pooled_attention(L, B, 0, s)); break;
    case ISA_STAGE_SHARP: ISA_RUN(isa::launch_pooled_attention(L, B, 1, s)); break;
    case ISA_STAGE_SELECT_Q: ISA_RUN(isa::launch_select_q(L, B, s)); break;
    case ISA_STAGE_TAYLOR: if (L.taylor_rows > 0) ISA_RUN(isa::launch_pooled_attention(L, B, 2, s)); break;
    case ISA_STAGE_FULL: if (L.kq > 0) ISA_RUN(isa::launch_full_attention(L, B, false, s)); break;
    case ISA_STAGE_FULL_MERGE: if (L.kq > 0) ISA_RUN(isa::launch_full_merge(L, B, s)); break;
  }
  return ISA_OK;
}

namespace {

// Validates the backward arguments; fills the two layouts.
isa_status bwd_prepare(const isa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                       const void* dO, const void* ws, size_t ws_bytes, void* bws, size_t bws_bytes, void* dQ,
                       void* dK, void* dV, isa::Layout* L, isa::BwdLayout* W) {
  isa_status st = isa::make_layout(desc, L);
  if (st != ISA_OK) return st;
  if ((st = isa::make_bwd_layout(*L, W)) != ISA_OK) return st;
  // dQ, dK, dV are written through the maps of Q, K, V
  if (!isa::map_disjoint(L->q, desc->B, L->Ns, L->d) || !isa::map_disjoint(L->k, desc->B, L->Nk, L->d) ||
      !isa::map_disjoint(L->v, desc->B, L->Nk, L->d))
    return ISA_ERR_INVALID_ARGUMENT;
  if ((st = check_io(Q, K, V, O, true)) != ISA_OK) return st;
  if ((st = check_io(dO, dQ, dK, dV, true)) != ISA_OK) return st;
  if ((st = check_ws(*L, ws, ws_bytes)) != ISA_OK) return st;
  return isa::check_workspace(bws, bws_bytes, W->total);
}

}  // namespace

extern "C" isa_status isa_run_backward_stage(const isa_desc* desc, int stage, const void* Q, const void* K,
                                             const void* V, const void* O, const void* dO, const void* workspace,
                                             size_t workspace_bytes, void* bwd_workspace, size_t bwd_workspace_bytes,
                                             void* dQ, void* dK, void* dV, void* stream) {
  if (stage < ISA_BWD_DELTA || stage > ISA_BWD_DQ_POOLED) return ISA_ERR_INVALID_ARGUMENT;
  isa::Layout L;
  isa::BwdLayout W;
  isa_status st = bwd_prepare(desc, Q, K, V, O, dO, workspace, workspace_bytes, bwd_workspace, bwd_workspace_bytes,
                              dQ, dK, dV, &L, &W);
  if (st != ISA_OK) return st;
  const isa::BwdBufs B{Q, K, V, O, dO, dQ, dK, dV, (const char*)workspace, (char*)bwd_workspace};
  static const isa::BwdWhat kWhat[] = {isa::BwdWhat::kDelta,   isa::BwdWhat::kDkPooled,   isa::BwdWhat::kDvPooled,
                                       isa::BwdWhat::kDkvReduce, isa::BwdWhat::kDkFull,   isa::BwdWhat::kDvFull,
                                       isa::BwdWhat::kZeroPruned, isa::BwdWhat::kDqFull,  isa::BwdWhat::kDqMerge,
                                       isa::BwdWhat::kDqPooled};
  ISA_RUN(isa::launch_backward(L, W, B, kWhat[stage], (hipStream_t)stream));
  return ISA_OK;
}

extern "C" isa_status isa_backward(const isa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const void* workspace, size_t workspace_bytes, void* bwd_workspace,
                                   size_t bwd_workspace_bytes, void* dQ, void* dK, void* dV, void* stream) {
  isa::Layout L;
  isa::BwdLayout W;
  isa_status st = bwd_prepare(desc, Q, K, V, O, dO, workspace, workspace_bytes, bwd_workspace, bwd_workspace_bytes,
                              dQ, dK, dV, &L, &W);
  if (st != ISA_OK) return st;
  const isa::BwdBufs B{Q, K, V, O, dO, dQ, dK, dV, (const char*)workspace, (char*)bwd_workspace};
  hipStream_t s = (hipStream_t)stream;
  // the pooled-key gradients must exist before the full dK/dV epilogue adds them
  for (isa::BwdWhat w : {isa::BwdWhat::kDelta, isa::BwdWhat::kDkPooled, isa::BwdWhat::kDvPooled,
                         isa::BwdWhat::kDkvReduce, isa::BwdWhat::kDkFull, isa::BwdWhat::kDvFull,
                         isa::BwdWhat::kZeroPruned, isa::BwdWhat::kDqFull, isa::BwdWhat::kDqMerge,
                         isa::BwdWhat::kDqPooled})
    ISA_RUN(isa::launch_backward(L, W, B, w, s));
  return ISA_OK;
}

extern "C" const char* isa_last_error(void) { return g_last_error; }
