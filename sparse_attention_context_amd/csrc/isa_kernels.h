// Launchers of the ISA kernels (host side).  Each enqueues on `stream` and
// returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include "isa_layout.h"

namespace isa {

// Pointers of one call: inputs, output and the carved workspace.
struct Bufs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  char* ws;
};

// ISA_OK, or ISA_ERR_DEVICE with the text of e kept for isa_last_error().
isa_status device_status(hipError_t e);

// The kernel sequence of isa_attention on validated arguments (B.ws: a
// workspace of at least L.total bytes); trace: record the stage timestamps
// when ISA_TRACE is set.
isa_status run_attention(const Layout& L, const Bufs& B, hipStream_t s, bool trace = true);

// Stage timestamps of a layer call when the ISA_TRACE environment variable
// is set (isa_trace.hip): mark(stage) records an event on the stream before
// the stage's launch, the destructor one after the last; isa_trace_read
// reports them.  Does nothing without ISA_TRACE or under stream capture.
class Tracer {
 public:
  Tracer(hipStream_t s, bool allowed = true);
  ~Tracer();
  void mark(const char* stage);

 private:
  hipStream_t s_;
  bool on_ = false;
};

// Block mean-pool of the source query blocks, every key block and the
// source value blocks.
hipError_t launch_pool(const Layout& L, const Bufs& B, hipStream_t s);

// After the context selection: block means of V for the kept context
// blocks, and the packed kept key set of the pooled attention (keys as bf16
// hi/lo, values, log2 n_j; padding rows zero with bias -inf).
hipError_t launch_pool_pack(const Layout& L, const Bufs& B, hipStream_t s);

// Context saliency partial column sums, one workgroup per kSalRows pooled
// queries of one head.
hipError_t launch_saliency(const Layout& L, const Bufs& B, hipStream_t s);

// Context top-rho: sums the partials into sal, selects kept_ctx and writes
// the full-route context row table.
hipError_t launch_select_ctx(const Layout& L, const Bufs& B, hipStream_t s);

// Query top-gamma: block means of the per-row peaks into sh, selects full_q /
// taylor_q and writes both query row tables.
hipError_t launch_select_q(const Layout& L, const Bufs& B, hipStream_t s);

// Pooled attention over the kept blocks.  mode 0: every source row, writes
// O (Taylor output) and the per-row peak probability; mode 1: every source
// row, peak only; mode 2: Taylor-route rows only, writes O.
hipError_t launch_pooled_attention(const Layout& L, const Bufs& B, int mode, hipStream_t s);

// Exact attention.  dense=false: full-route rows over the kept key tokens
// (bf16: the flash kernel, writing split partials when split; the merge is
// launch_full_merge); dense=true: every source row over every key row (no
// workspace needed).
hipError_t launch_full_attention(const Layout& L, const Bufs& B, bool dense, hipStream_t s);

// Merges the full route's split-K partials into O (nothing when unsplit or f32).
hipError_t launch_full_merge(const Layout& L, const Bufs& B, hipStream_t s);

// The bf16 flash kernel family (isa_flash.hip).
enum class FlashWhat { kDense, kContext, kFull, kFullMerge, kSharpTaylor, kSharp, kTaylor };
hipError_t launch_flash(const Layout& L, const Bufs& B, FlashWhat what, hipStream_t s);

// Backward pass (isa_flash_bwd.hip): inputs, forward output, its gradient,
// the three gradients, the planned forward workspace (read only) and the
// backward workspace.
struct BwdBufs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  const char* ws;
  char* bws;
};
// FP8 variant of the full route (isa_flash_fp8.hip): pack=true quantises the
// key list into the FP8 workspace, pack=false runs the attention (O rows, or
// split partials that the bf16 merge combines).
hipError_t launch_fp8(const Layout& L, const Fp8Layout& F, const Bufs& B, char* fp8_ws, bool pack, hipStream_t s);

enum class BwdWhat {
  kDelta, kDkPooled, kDvPooled, kDkvReduce, kDkFull, kDvFull, kZeroPruned, kDqFull, kDqMerge, kDqPooled
};
hipError_t launch_backward(const Layout& L, const BwdLayout& W, const BwdBufs& B, BwdWhat what, hipStream_t s);

}  // namespace isa
