// fm_attn_fwd_static: the forward entry point for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid allocation).
//
// fm_attn_fwd takes a caller workspace for its classification (block min/max, queues,
// counts, costs, the LPT order and the sort's scratch).  This variant runs the same
// kernels on a library-owned workspace instead: `scratch`, a file-scope device array of
// FM_STATIC_WORKSPACE_BYTES that every GPU the library runs on holds until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory, so the
// array is only ever used through the device address hipGetSymbolAddress returns for it,
// taken once per device (with that device current) on the first call there and kept.
//
// Nothing in the forward's workspace has to start at zero: the classification writes
// every entry it later reads, and the block-sparse zero vectors are cleared by a fill
// kernel.  The array keeps the last call's contents.  All calls on one GPU share its
// copy, so calls that overlap on one GPU (on different streams, without ordering between
// them) race on it; calls on one stream are ordered and safe.
#include <mutex>

#include "fm.h"
#include "fm_internal.h"

namespace {

static_assert(FM_STATIC_WORKSPACE_BYTES % 256 == 0, "static workspace size");

__device__ __align__(256) unsigned char scratch[FM_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's address of `scratch`, resolved on the first call on that device.
fm_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return FM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FM_OK;
}

}  // namespace

extern "C" fm_status fm_attn_fwd_static(const fm_problem* p, const void* q, const void* k,
                                        const void* v, const fm_mask* m, void* o, float* lse,
                                        void* stream, const fm_kernel_events* events) {
  size_t need = 0;
  fm_status st = fm_workspace_size(p, FM_OP_FWD, 0, 0, &need);
  if (st != FM_OK) return st;
  if (need > (size_t)FM_STATIC_WORKSPACE_BYTES) return FM_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != FM_OK) return st;
  return fm_attn_fwd(p, q, k, v, m, o, lse, ws, FM_STATIC_WORKSPACE_BYTES, stream, events);
}
