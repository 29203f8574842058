// isa_attention_noalloc: isa_attention with its workspace in a file-scope
// device array instead of caller memory, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Nothing here allocates: the array is part of the library's
// code object, and each device that runs it holds its own copy until the
// process ends.
//
// The host never uses the array's name as an address (in host code it is a
// stand-in symbol, not device memory): the first call on a device, with that
// device current, asks the runtime for the device address of that device's
// copy (hipGetSymbolAddress) and keeps it; kernels get that pointer as their
// workspace, exactly as isa_attention gets the caller's.
//
// No part of the workspace has to start at zero: every kernel of the layer
// writes each workspace word before a later kernel reads it, so a call does
// not depend on what an earlier call left.  Calls that overlap on one device
// share the array and race; the caller serialises them (one stream, or
// stream order).
#include <mutex>
#include <vector>

#include "isa_kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // 128 MiB: the video-DiT and multi-reference layers fit

__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::mutex g_mu;
std::vector<void*> g_ptr;   // device address of `scratch`, per device

// Device address of this device's copy of the scratch array.
isa_status scratch_for_current_device(void** out) {
  int dev = -1;
  isa_status st = isa::device_status(hipGetDevice(&dev));
  if (st != ISA_OK) return st;
  if (dev < 0) return ISA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((size_t)dev >= g_ptr.size()) g_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    st = isa::device_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (st != ISA_OK) return st;
    if (!p || ((uintptr_t)p % isa::kWsAlign) != 0) return ISA_ERR_DEVICE;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return ISA_OK;
}

}  // namespace

extern "C" size_t isa_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" isa_status isa_attention_noalloc(const isa_desc* desc, const void* Q, const void* K, const void* V,
                                            void* O, void* stream) {
  isa::Layout L;
  isa_status st = isa::make_layout(desc, &L);
  if (st != ISA_OK) return st;
  const void* p[4] = {Q, K, V, O};
  if ((st = isa::check_tensors(p, 4)) != ISA_OK) return st;
  if (L.total > kScratchBytes) return ISA_ERR_WORKSPACE;   // the layer needs more than the fixed scratch
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != ISA_OK) return st;
  return isa::run_attention(L, isa::Bufs{Q, K, V, O, (char*)ws}, (hipStream_t)stream, false);
}
