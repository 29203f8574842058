/*
 * isa.h -- C-ABI of the MI355X (gfx950) In-context Sparse Attention library.
 *
 * The operation is the forward pass of In-context Sparse Attention (ISA) as
 * named in "Lightning Unified Video Editing via In-Context Sparse Attention"
 * (chatpaper.ai page), English abstract: source-video query tokens attend
 * over the source tokens concatenated with context (reference) tokens;
 * low-saliency context is pruned by a pre-selection step; query blocks are
 * grouped by query sharpness, the sharp (high-error) ones going to exact full
 * attention and the rest to 0-th order Taylor sparse attention over pooled
 * key blocks.  The abstract gives no formulas; this library computes:
 *
 *   blocks     each of the source rows [0,Ns) and context rows [Ns,Ns+Nc) is
 *              cut into blocks of b rows from its own start (last one short);
 *              block j has count n_j and mean key kbar_j, mean value vbar_j;
 *              pooled query qbar_i is the mean query of source block i.
 *   saliency   sal_c = sum_i P_i(c), P_i the n-weighted softmax of qbar_i
 *              over all key blocks: n_j exp(qbar_i.kbar_j/sqrt d) / sum.
 *   pre-select keep kc = ceil(rho*nb_c - 1e-9) context blocks, highest sal
 *              first, ties to the lower index.  Kept key set = all source
 *              blocks + kept context blocks.
 *   sharpness  sh_i = mean over queries q of block i of max_j P_j(q), the
 *              n-weighted softmax of q over the kept blocks.
 *   grouping   kq = ceil(gamma*nb_s - 1e-9) query blocks with the highest sh
 *              (ties to the lower index) take the full route, the rest Taylor.
 *   full       o = softmax(q K^T/sqrt d) V over every token of the kept set.
 *   Taylor     o = sum_j n_j e^{q.kbar_j/sqrt d} vbar_j / sum_j n_j e^{...}
 *              over the kept blocks (exp(q.k_t) ~ exp(q.kbar_j) inside j).
 *   merge      every source row of O is written by its block's route.
 *
 * Tensors (device memory, caller-owned, d unit-stride):
 *   Q [B,H,Ns,d], K and V [B,H,Ns+Nc,d] (rows [0,Ns) source, [Ns,Ns+Nc)
 *   context), O [B,H,Ns,d]; all of element type desc->dtype.  Each tensor is
 *   addressed through its own element strides of the batch, head and row
 *   dimensions (isa_desc.q, .k, .v, .o): row r of head h of batch x of Q
 *   starts at element x*q.b + h*q.h + r*q.n (likewise K, V, O).  A layout
 *   [B,N,H,d] (tokens before heads, as a fused QKV projection leaves it)
 *   has strides {N*H*d, d, H*d}; all three 0 means contiguous [B,H,rows,d].
 *   Pointers and every stride that is used (dimension larger than 1) must
 *   be 16-byte aligned in bytes; O's strides (for isa_backward also Q's, K's
 *   and V's, which address dQ, dK, dV) must not make two of its elements
 *   overlap; one head of a tensor must span less than 2^31 bytes
 *   and a row step less than 2^24 bytes.
 *   Context-token query rows are not computed.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Every call only enqueues work on that stream: no host
 * synchronisation, no device allocation, no printing.  Results are
 * deterministic (no floating-point atomics).
 *
 * Workspace: caller-owned device memory of isa_workspace_size() bytes,
 * 256-byte aligned.  isa_plan() leaves the plan (pooled blocks, scores and
 * index lists) in it; isa_forward() reads it and adds each source row's
 * log-sum-exp, which isa_backward() reads (bf16).  It must stay alive and
 * unmodified until the work that reads it has completed on the stream.
 *
 * Errors: every call validates its arguments on the host before enqueuing
 * anything, so a call that returns an error has launched no work and left O
 * untouched, except ISA_ERR_DEVICE, which reports a failed launch (the text
 * of the HIP error is then available from isa_last_error()).
 */
#ifndef ISA_H_
#define ISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum isa_status {
  ISA_OK = 0,
  ISA_ERR_INVALID_ARGUMENT = 1, /* null pointer, rho/gamma not in [0,1] or NaN,
                                   Ns < 1, Nc < 0, B or H < 1, b < 1, misaligned
                                   pointer or stride, negative stride, an output
                                   layout whose elements overlap, reserved != 0 */
  ISA_ERR_UNSUPPORTED = 2,      /* d not 64/128, b > 256, unknown dtype, B*H >
                                   65535, Ns + Nc >= 2^24, a head of a tensor
                                   spanning 2^31 bytes or more, a row step of
                                   2^24 bytes or more */
  ISA_ERR_WORKSPACE = 3,        /* workspace too small or not 256-byte aligned */
  ISA_ERR_DEVICE = 4            /* a kernel launch failed; see isa_last_error() */
} isa_status;

typedef enum isa_dtype { ISA_BF16 = 0, ISA_F32 = 1 } isa_dtype;

/* Element strides of the batch, head and row dimensions of one tensor
 * (the d dimension is unit-stride).  {0, 0, 0} = contiguous [B,H,rows,d]. */
typedef struct isa_strides {
  int64_t b;
  int64_t h;
  int64_t n;
} isa_strides;

/* Problem description.  rho and gamma are doubles so that the kept counts
 * ceil(f*n - 1e-9) are evaluated exactly as documented. */
typedef struct isa_desc {
  int32_t B;      /* batch, >= 1 */
  int32_t H;      /* heads, >= 1; B*H <= 65535 */
  int32_t Ns;     /* source (query) rows, >= 1 */
  int32_t Nc;     /* context rows, >= 0; Ns + Nc < 2^24 */
  int32_t d;      /* head width, 64 or 128 */
  int32_t b;      /* block size in tokens, 1..256 */
  double rho;     /* fraction of context blocks kept, in [0,1] */
  double gamma;   /* fraction of query blocks sent to full attention, in [0,1] */
  int32_t dtype;  /* isa_dtype of Q, K, V and O */
  int32_t reserved; /* must be 0 */
  isa_strides q;  /* Q (also dQ of isa_backward and Qc of isa_context_forward) */
  isa_strides k;  /* K (also dK) */
  isa_strides v;  /* V (also dV) */
  isa_strides o;  /* O (also dO of isa_backward and Oc of isa_context_forward) */
} isa_desc;

/* Derived counts (host values). */
typedef struct isa_counts {
  int32_t nb_s;        /* source (query) blocks, ceil(Ns/b) */
  int32_t nb_c;        /* context blocks, ceil(Nc/b) */
  int32_t kc;          /* kept context blocks */
  int32_t kq;          /* query blocks on the full route */
  int32_t m_kept;      /* kept key blocks, nb_s + kc */
  int32_t reserved;
  int64_t full_keys;   /* key tokens seen by a full-route query: Ns + kept context tokens
                          (an upper bound: a kept short tail block counts b) */
} isa_counts;

/* Device pointers into a planned workspace (isa_plan_views).  Shapes are
 * per (batch, head) slice, slices stored one after another in [B,H] order.
 * Lists are ascending int32. */
typedef struct isa_plan_view {
  const float* qbar;       /* [B,H,nb_s,d]      pooled source queries */
  const float* kbar;       /* [B,H,nb_s+nb_c,d] pooled keys, source blocks first */
  const float* vbar;       /* [B,H,nb_s+nb_c,d] pooled values (context entries of
                              blocks that are not kept are not computed) */
  const double* sal;       /* [B,H,nb_c]  context saliency */
  const int32_t* kept_ctx; /* [B,H,kc]    kept context block indices */
  const double* sh;        /* [B,H,nb_s]  query-block sharpness */
  const int32_t* full_q;   /* [B,H,kq]    query blocks on the full route */
  const int32_t* taylor_q; /* [B,H,nb_s-kq] query blocks on the Taylor route */
  isa_counts counts;
} isa_plan_view;

/* The steps of the layer, in the order isa_attention runs them.  Each stage
 * is one kernel launch and reads what the earlier stages left in the
 * workspace (same desc, same inputs); a stage with nothing to do for the
 * shape (e.g. saliency with Nc = 0) enqueues nothing. */
typedef enum isa_stage {
  ISA_STAGE_POOL = 0,         /* block means: source Q, every K block, source V (pooling) */
  ISA_STAGE_SALIENCY = 1,     /* per-workgroup column sums of the pooled softmax (saliency) */
  ISA_STAGE_SELECT_CTX = 2,   /* sal, kept_ctx (top-rho) and the context key-row table */
  ISA_STAGE_POOL_KEPT_V = 3,  /* block means of V for the kept context blocks, and in the same
                                 launch the packed kept set: pooled keys (bf16 hi/lo), values, log2 n_j */
  ISA_STAGE_PACK = 4,         /* no work of its own (the packing runs with POOL_KEPT_V); kept so that
                                 stage sequences stay valid */
  ISA_STAGE_SHARP_TAYLOR = 5, /* per-row peak probability + Taylor output of every row into O */
  ISA_STAGE_SHARP = 6,        /* per-row peak probability only (sharpness) */
  ISA_STAGE_SELECT_Q = 7,     /* sh, full_q / taylor_q (top-gamma) and the full-route key-row table */
  ISA_STAGE_TAYLOR = 8,       /* Taylor output of the Taylor-route rows into O */
  ISA_STAGE_FULL = 9,         /* full attention of the full-route rows: into O, or into
                                 split partials when the key range is split */
  ISA_STAGE_FULL_MERGE = 10   /* merges the full route's split partials into O (no-op unsplit) */
} isa_stage;

/* Runs one stage.  isa_plan = POOL, SALIENCY, SELECT_CTX, POOL_KEPT_V, PACK,
 * SHARP, SELECT_Q; isa_forward = TAYLOR, FULL, FULL_MERGE; isa_attention =
 * POOL .. PACK, SHARP_TAYLOR, SELECT_Q, FULL, FULL_MERGE.  O may be NULL for stages that do not
 * write it.  Unknown stage: ISA_ERR_INVALID_ARGUMENT. */
isa_status isa_run_stage(const isa_desc* desc, int stage, const void* Q, const void* K, const void* V,
                         void* O, void* workspace, size_t workspace_bytes, void* stream);

/* Counts implied by *desc (validates it).  Defined by the readings above. */
isa_status isa_get_counts(const isa_desc* desc, isa_counts* out);

/* Bytes of workspace isa_plan / isa_forward / isa_attention need for *desc. */
isa_status isa_workspace_size(const isa_desc* desc, size_t* bytes);

/* Selection half: pooling, context saliency and pre-selection, query
 * sharpness and grouping.  Reads Q, K, V; writes only the workspace. */
isa_status isa_plan(const isa_desc* desc, const void* Q, const void* K, const void* V,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Output half: given a workspace planned by isa_plan with the same desc and
 * inputs, writes every source row of O (Taylor rows, then full rows). */
isa_status isa_forward(const isa_desc* desc, const void* Q, const void* K, const void* V,
                       void* O, void* workspace, size_t workspace_bytes, void* stream);

/* The whole layer in one call: plan and forward, with the sharpness pass
 * also producing the Taylor output of every row, which the full route then
 * overwrites for its rows.  Same O and same plan contents as
 * isa_plan + isa_forward. */
isa_status isa_attention(const isa_desc* desc, const void* Q, const void* K, const void* V,
                         void* O, void* workspace, size_t workspace_bytes, void* stream);

/* Dense attention of all Ns source queries over all Ns+Nc keys with the same
 * flash-attention kernel as the full route (the library's own dense
 * baseline); rho, gamma and b are ignored.  Needs no workspace.  This is the
 * global self-attention softmax(q k^T / sqrt d) v of the intelliparadigm.com
 * page "深度学习注意力机制：全局与时间注意力的计算效率对比", section 1. */
isa_status isa_dense_forward(const isa_desc* desc, const void* Q, const void* K, const void* V,
                             void* O, void* stream);

/* ---- Backward pass (bf16 only) -------------------------------------------
 *
 * The pages give no backward pass.  These calls compute the derivatives of
 * the forward above for L = sum(dO * O) with the selection frozen: kept_ctx
 * and full_q are discrete decisions and get no gradient (nor do sal and sh),
 * the counts n_j are constants, a pooled key's (value's) gradient is shared
 * equally by the rows of its block (it is their mean), and rows of pruned
 * context blocks get zero gradient:
 *   full rows   ds = p (dO.v - D), D = dO.o;  dq = ds K/sqrt d,
 *               dk += ds^T q/sqrt d, dv += p^T dO over the kept tokens;
 *   Taylor rows the same over the kept pooled blocks (p n_j-weighted), then
 *               dk_t += dkbar_j/n_j, dv_t += dvbar_j/n_j for rows t of block j.
 *
 * workspace: the forward workspace of an isa_attention or isa_plan +
 * isa_forward call with the same desc and inputs (plan and per-row log-sum-
 * exp); read only.  bwd_workspace: caller-owned device memory of
 * isa_backward_workspace_size() bytes, 256-byte aligned.  O is the forward's
 * output and dO its gradient, both [B,H,Ns,d]; dQ [B,H,Ns,d], dK and dV
 * [B,H,Ns+Nc,d] are written entirely.  All of element type bf16; f32 gives
 * ISA_ERR_UNSUPPORTED.  Deterministic (no atomics). */

typedef enum isa_bwd_stage {
  ISA_BWD_DELTA = 0,        /* D = rowsum(dO * O) of every source row */
  ISA_BWD_DK_POOLED = 1,    /* Taylor rows: per-split partial gradients of the kept pooled keys */
  ISA_BWD_DV_POOLED = 2,    /* Taylor rows: per-split partial gradients of the kept pooled values */
  ISA_BWD_DKV_REDUCE = 3,   /* sums those partials in split order (zero without Taylor rows) */
  ISA_BWD_DK_FULL = 4,      /* full rows: dK of every source and kept context row, plus the pooled
                               share of its block (d = 128: a part-filled last round of key tiles is
                               cut into query-tile parts, merged within the stage) */
  ISA_BWD_DV_FULL = 5,      /* the same for dV */
  ISA_BWD_ZERO_PRUNED = 6,  /* zeroes dK, dV rows of pruned context blocks */
  ISA_BWD_DQ_FULL = 7,      /* full rows: dQ, or split partials when the key range is split */
  ISA_BWD_DQ_MERGE = 8,     /* merges the dQ split partials (no-op unsplit) */
  ISA_BWD_DQ_POOLED = 9     /* Taylor rows: dQ */
} isa_bwd_stage;

/* Bytes of backward workspace isa_backward needs for *desc. */
isa_status isa_backward_workspace_size(const isa_desc* desc, size_t* bytes);

/* dQ, dK, dV of the layer planned in `workspace` (stages DELTA .. DQ_POOLED
 * in order). */
isa_status isa_backward(const isa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const void* workspace, size_t workspace_bytes, void* bwd_workspace,
                        size_t bwd_workspace_bytes, void* dQ, void* dK, void* dV, void* stream);

/* One backward stage (one kernel launch); same arguments as isa_backward.
 * Unknown stage: ISA_ERR_INVALID_ARGUMENT. */
isa_status isa_run_backward_stage(const isa_desc* desc, int stage, const void* Q, const void* K, const void* V,
                                  const void* O, const void* dO, const void* workspace, size_t workspace_bytes,
                                  void* bwd_workspace, size_t bwd_workspace_bytes, void* dQ, void* dK, void* dV,
                                  void* stream);

/* Context-token query rows (bf16): the other half of the in-context layer.
 * The pages define pruning and query grouping for the source (editing)
 * queries only and say nothing of context queries; they are read here as
 * ordinary attention: every context row attends over all Ns+Nc keys,
 * softmax(q K^T / sqrt d) V.  Qc and Oc are [B,H,Nc,d] (the context rows of
 * the concatenated queries), K and V [B,H,Ns+Nc,d].  Same flash kernel as
 * isa_dense_forward; needs no workspace; Nc = 0 enqueues nothing; f32 gives
 * ISA_ERR_UNSUPPORTED. */
isa_status isa_context_forward(const isa_desc* desc, const void* Qc, const void* K, const void* V, void* Oc,
                               void* stream);

/* ---- FP8 variant of the full route (bf16 inputs) ------------------------
 *
 * The first page's list of attention speed-ups names 8-bit quantisation.
 * isa_attention_fp8 runs the same layer as isa_attention, with the full
 * route's operands in OCP e4m3 under power-of-two block scales (MX: a shared
 * 2^e per 32 elements, e the smallest with max|x| / 2^e <= 448): Q per (query,
 * 32 d), K per (key, 32 d), V per (d, 32 consecutive keys of the full
 * route's key list: source rows, then the tokens of the kept context blocks),
 * and the probabilities exp2(x - m) unscaled, with the reference maximum m a
 * whole number in the exp2 domain.  Products on v_mfma_scale_f32_32x32x64_
 * f8f6f4 with fp32 accumulation; everything else as isa_attention.  The
 * error against exact attention is that of the rounding (a few percent of
 * the output norm on N(0,1) data); the plan is identical to isa_attention's.
 * fp8_workspace: isa_fp8_workspace_size() bytes, 256-byte aligned (the key
 * list in e4m3 and its scales). */
typedef enum isa_fp8_stage {
  ISA_FP8_PACK = 0,         /* quantises the full route's key list into the FP8 workspace */
  ISA_FP8_FULL = 1,         /* FP8 full attention: O rows, or split partials */
  ISA_FP8_FULL_MERGE = 2    /* merges the split partials (as ISA_STAGE_FULL_MERGE) */
} isa_fp8_stage;

isa_status isa_fp8_workspace_size(const isa_desc* desc, size_t* bytes);

isa_status isa_attention_fp8(const isa_desc* desc, const void* Q, const void* K, const void* V, void* O,
                             void* workspace, size_t workspace_bytes, void* fp8_workspace,
                             size_t fp8_workspace_bytes, void* stream);

/* One stage of the FP8 full route (after the plan stages of isa_attention,
 * POOL .. SELECT_Q, have run on the workspace); nothing when kq = 0. */
isa_status isa_run_fp8_stage(const isa_desc* desc, int stage, const void* Q, const void* K, const void* V, void* O,
                             void* workspace, size_t workspace_bytes, void* fp8_workspace,
                             size_t fp8_workspace_bytes, void* stream);

/* ---- Without allocation --------------------------------------------------
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * isa_attention with its workspace in a fixed scratch array inside the
 * library (isa_noalloc_scratch_bytes() = 128 MiB per device, held by each
 * device the library runs on until the process ends) instead of caller
 * memory.  Same arguments, output and errors as isa_attention without the
 * workspace; ISA_ERR_WORKSPACE when isa_workspace_size(desc) exceeds the
 * scratch.  The plan is not kept for the caller (isa_plan_views and
 * isa_backward need isa_attention's workspace).  No allocation, no host
 * synchronisation.  Every call on a device shares that device's scratch:
 * calls that overlap on one device race, so the caller orders them (one
 * stream, or stream order); each call writes every scratch word it reads. */
isa_status isa_attention_noalloc(const isa_desc* desc, const void* Q, const void* K, const void* V, void* O,
                                 void* stream);

/* Bytes of the scratch array of isa_attention_noalloc. */
size_t isa_noalloc_scratch_bytes(void);

/* Device pointers to the plan held in a workspace (no device access). */
isa_status isa_plan_views(const isa_desc* desc, void* workspace, size_t workspace_bytes,
                          isa_plan_view* out);

/* One stage of a traced call: its name ("pool", "saliency", "select_ctx",
 * "pool_kept_v", "sharp_taylor" or "sharp", "select_q", "full",
 * "full_merge"; static strings owned by the library) and the milliseconds
 * between the events recorded on the stream before it and before the next
 * stage (after the last). */
typedef struct isa_trace_entry {
  const char* stage;
  float ms;
} isa_trace_entry;

/* Per-stage timestamps of the last isa_attention call made while the
 * environment variable ISA_TRACE was set (to a value other than "" or "0";
 * read at every call; isa_attention_noalloc never traces, since the first
 * traced call creates HIP events).  Such a call
 * records a HIP event on its stream before each kernel and one after the
 * last, into a set of events that every traced call reuses: only the last
 * call is kept, calls from several threads at once interleave, and a call on
 * a stream under graph capture records nothing.  Waits for the last event,
 * then writes up to max_entries stages to out and their number to
 * *n_entries.  ISA_ERR_INVALID_ARGUMENT when n_entries is NULL, out is NULL
 * with max_entries > 0, or no traced call has completed its recording;
 * ISA_ERR_DEVICE when an event query fails. */
isa_status isa_trace_read(isa_trace_entry* out, int max_entries, int* n_entries);

/* Static text for a status code. */
const char* isa_status_string(isa_status status);

/* Text of the last device error seen by this thread ("" if none). */
const char* isa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ISA_H_ */
