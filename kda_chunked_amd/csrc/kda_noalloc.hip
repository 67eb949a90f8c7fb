// kda_fwd_noalloc: the forward of kda_fwd with its scratch workspace taken
// from a fixed device array of the library instead of a caller buffer, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc). Nothing here allocates.
//
// Each GPU holds its own copy of `scratch` from module load until the process
// ends. The host never passes the array's name to a kernel: the name is a host
// stand-in, so the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept. The
// forward writes every scratch byte it reads in the same call (the chunk table
// and, without a saved set, the per-chunk set), so nothing needs clearing
// between calls; calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on its first use).
kda_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return kda::fail(KDA_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return kda::fail(KDA_ERR_UNSUPPORTED, "device %d: the no-alloc scratch serves devices 0..%d",
                     dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return kda::fail(KDA_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_fwd_noalloc(const kda_problem* p, const void* q, const void* k,
                                      const void* v, const void* beta, const void* g_or_a,
                                      const float* A_log, const float* dt_bias,
                                      const int32_t* cu_seqlens, void* o, void* saved,
                                      void* stream) {
  const size_t need = kda_workspace_bytes(p, 0, saved == nullptr);
  if (need == 0)   // an invalid problem: kda_fwd reports it before anything else
    return kda_fwd(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, o, saved, nullptr, 0,
                   stream);
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
    return kda::fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                     "kda_fwd_noalloc: this call needs %zu bytes of scratch; the library's fixed "
                     "scratch holds %zu (pass a saved set, or use kda_fwd with a workspace)",
                     need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const kda_status st = scratch_of_current_device(&ws);
  if (st != KDA_OK) return st;
  return kda_fwd(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, o, saved, ws,
                 (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}
