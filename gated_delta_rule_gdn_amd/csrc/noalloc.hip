// gdn_backward_noalloc: gdn_backward with its workspace in a file-scope
// device array instead of caller memory, for callers that cannot allocate.
//
// Each GPU the library runs on holds its own copy of `scratch` (kScratchBytes)
// from module load until the process ends.  Host code never passes the
// array's name to a kernel or a copy: the name is a host-side stand-in, so the
// device address of the current GPU's copy is looked up once per device
// (hipGetSymbolAddress, with that device current) and that address is what
// the backward receives as its workspace.  Every call on one GPU shares that
// GPU's copy; calls that overlap on one GPU (other streams, other host
// threads) race on it.  The backward writes every workspace element it reads,
// so nothing has to start at zero.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Device address of the current GPU's copy of `scratch`.
hipError_t scratch_on_current_device(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch[dev];
  return g_status[dev];
}

}  // namespace

extern "C" {

size_t gdn_backward_noalloc_max_bytes(void) { return kScratchBytes; }

gdn_status gdn_backward_noalloc(const gdn_bwd_desc* desc, const void* q, const void* k,
                                const void* v, const void* beta_or_b, const void* w,
                                const void* g, const float* state_in, const void* d_o,
                                const float* d_state_out, float* dq, float* dk, float* dv,
                                float* db, float* dw, float* dg, float* d_state_in,
                                void* stream) {
  if (!desc) return GDN_ERR_INVALID_ARG;
  // 0 means an invalid descriptor or no token: gdn_backward decides which
  // (and needs no workspace for the latter)
  if (gdn_backward_workspace_size(desc) > kScratchBytes) return GDN_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess || !ws) return GDN_ERR_HIP;
  return gdn_backward(desc, q, k, v, beta_or_b, w, g, state_in, d_o, d_state_out, ws,
                      kScratchBytes, dq, dk, dv, db, dw, dg, d_state_in, stream);
}

}  // extern "C"
