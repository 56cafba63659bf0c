// kda_fwd_noalloc: the forward with its workspace in a static device array, for callers
// that cannot allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation).  Declaration and contract in include/kda.h.
//
// `scratch` below is a file-scope device array: every GPU that runs this library holds
// its own copy (KDA_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code its name
// is only a stand-in, never a device address: the address of the current device's copy is
// looked up once per device with hipGetSymbolAddress and that pointer is what the kernels
// receive.  Nothing in the workspace has to start at zero (the fused kernel's flags are
// compared with a per-launch value), so nothing is cleared between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"

static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the first call
// made with that device current.
hipError_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status_t kda_fwd_noalloc(const kda_problem_t* prob, const void* q, const void* k, const void* v,
                                        const float* g, const void* beta, const float* h0,
                                        const int32_t* cu_seqlens, float scale, void* out, float* ht,
                                        void* stream) {
  if (!prob) return KDA_ERR_NULL;
  // problems whose workspace exceeds the array are rejected before anything is enqueued
  // (an invalid problem sizes to 0 here and gets kda_fwd's own error below)
  if (kda_fwd_workspace_size(prob) > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess || ws == nullptr) return KDA_ERR_HIP;
  return kda_fwd(prob, q, k, v, g, beta, h0, cu_seqlens, scale, out, ht, ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES,
                 stream);
}
