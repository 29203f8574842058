// Per-stage timestamps of the last isa_attention call (ISA_TRACE).  The
// entry point without allocations (isa_attention_noalloc) never traces: the
// first traced call creates the events.
//
// With the environment variable ISA_TRACE set to a value other than "" or
// "0" at the time of a call, the layer's launch chain records a
// HIP event on the caller's stream before each kernel and one after the
// last; isa_trace_read turns them into per-stage milliseconds.  The events
// are created once per device (hipEventCreate, no memory allocation) and
// reused by every call, so only the last call is kept.  A call on a stream
// that is being captured into a graph records nothing (and clears the
// previous trace).  Without ISA_TRACE a call reads the variable once and
// takes one branch per stage.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "isa_kernels.h"

namespace {

constexpr int kMaxMarks = 16;

struct TraceState {
  std::mutex mu;
  int device = -1;
  hipEvent_t ev[kMaxMarks] = {};
  const char* name[kMaxMarks] = {};
  int n = 0;          // events recorded by the last traced call
  bool done = false;  // the last traced call recorded its closing event
};

TraceState& state() {
  static TraceState s;
  return s;
}

// (read at every call, so that a process can switch tracing on and off)
bool enabled() {
  const char* v = getenv("ISA_TRACE");
  return v && v[0] && strcmp(v, "0") != 0;
}

}  // namespace

namespace isa {

Tracer::Tracer(hipStream_t s, bool allowed) : s_(s) {
  if (!allowed || !enabled()) return;
  TraceState& t = state();
  std::lock_guard<std::mutex> g(t.mu);
  t.n = 0;
  t.done = false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  if (t.device != dev) {
    for (int i = 0; i < kMaxMarks; ++i) {
      if (t.ev[i]) (void)hipEventDestroy(t.ev[i]);
      t.ev[i] = nullptr;
    }
    for (int i = 0; i < kMaxMarks; ++i)
      if (hipEventCreate(&t.ev[i]) != hipSuccess) return;
    t.device = dev;
  }
  on_ = true;
}

void Tracer::mark(const char* stage) {
  if (!on_) return;
  TraceState& t = state();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.n >= kMaxMarks || hipEventRecord(t.ev[t.n], s_) != hipSuccess) {
    on_ = false;
    return;
  }
  t.name[t.n++] = stage;
}

Tracer::~Tracer() {
  if (!on_) return;
  mark(nullptr);   // closing event
  TraceState& t = state();
  std::lock_guard<std::mutex> g(t.mu);
  t.done = on_;
}

}  // namespace isa

extern "C" isa_status isa_trace_read(isa_trace_entry* out, int max_entries, int* n_entries) {
  if (!n_entries || max_entries < 0 || (max_entries > 0 && !out)) return ISA_ERR_INVALID_ARGUMENT;
  *n_entries = 0;
  TraceState& t = state();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.done || t.n < 2) return ISA_ERR_INVALID_ARGUMENT;
  isa_status st = isa::device_status(hipEventSynchronize(t.ev[t.n - 1]));
  if (st != ISA_OK) return st;
  int k = 0;
  for (int i = 0; i + 1 < t.n && k < max_entries; ++i, ++k) {
    float ms = 0.f;
    if ((st = isa::device_status(hipEventElapsedTime(&ms, t.ev[i], t.ev[i + 1]))) != ISA_OK) return st;
    out[k].stage = t.name[i];
    out[k].ms = ms;
  }
  *n_entries = k;
  return ISA_OK;
}
