// noalloc.hip -- the forward pass with the library's own scratch, for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid allocation).
//
// The scratch is one file-scope device array of kScratchBytes per GPU, part
// of the code object: every GPU the library runs on holds it until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol); its device address comes from
// hipGetSymbolAddress, once per device, with that device current, and is
// kept per device.
//
// Nothing in the scratch has to start at zero: the forward kernels tag their
// chunk-to-chunk flags and their status word with a per-call value and never
// read anything else they did not write in the same call.  Calls share the
// scratch of their GPU, so calls that overlap on one GPU (other streams,
// other threads) race; callers serialise them.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdio>
#include <mutex>

#include "../../include/ssd.h"

namespace ssd {
ssd_status fwd_check_scratch(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                             const float* dt, const float* A, const void* B, const void* C,
                             const float* D, const float* init_state, void* y,
                             float* final_state, size_t* need);
ssd_status report(ssd_status st, const char* msg);
}  // namespace ssd

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {nullptr};

// The device address of this device's scratch, looked up once per device.
ssd_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ssd::report(SSD_ERR_HIP, "no-alloc forward: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return ssd::report(SSD_ERR_UNSUPPORTED, "no-alloc forward: device index beyond 63");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return ssd::report(SSD_ERR_HIP, "no-alloc forward: hipGetSymbolAddress of the scratch failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SSD_OK;
}

}  // namespace

namespace ssd {
// This device's scratch when the no-alloc entry point has set it up, else NULL.
void* noalloc_scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_scratch[dev];
}
}  // namespace ssd

extern "C" ssd_status ssd_fwd_noalloc(const ssd_problem* prob, const ssd_dt_transform* dtx,
                                      const void* x, const float* dt, const float* A,
                                      const void* B, const void* C, const float* D,
                                      const float* init_state, void* y, float* final_state,
                                      void* stream) {
  try {
    size_t need = 0;
    ssd_status st = ssd::fwd_check_scratch(prob, dtx, x, dt, A, B, C, D, init_state, y,
                                           final_state, &need);
    if (st != SSD_OK) return st;
    if (need > kScratchBytes) {
      char msg[160];
      snprintf(msg, sizeof(msg),
               "no-alloc forward: the problem needs %zu bytes of scratch, the built-in scratch "
               "holds %zu",
               need, kScratchBytes);
      return ssd::report(SSD_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != SSD_OK) return st;
    return ssd_fwd_ex(prob, dtx, x, dt, A, B, C, D, init_state, y, final_state, ws, kScratchBytes,
                      stream);
  } catch (...) {
    return ssd::report(SSD_ERR_INTERNAL, "unexpected exception");
  }
}
