// The allocation-free split-key forward: attn_jvp_fwd_split with its
// workspace in a fixed device array owned by the library, for callers that
// cannot allocate (graph capture, serving loops, harnesses that forbid it).
//
// `scratch` is a file-scope device array: every device the library runs on
// holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device
// memory); on the first call on a device, with that device current, its
// device address is fetched once with hipGetSymbolAddress and kept per
// device, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace attnjvp {
namespace {

constexpr uint64_t kScratchBytes = ATTN_JVP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (fetched once per device
// with the device current).  NULL if the address cannot be obtained.
void *scratch_on(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();  // leave no sticky error behind
      return nullptr;
    }
    g_ptr[device] = ptr;
  }
  return g_ptr[device];
}

}  // namespace
}  // namespace attnjvp

extern "C" int attn_jvp_fwd_split_noalloc(const attn_jvp_args *a, const attn_jvp_mask *m,
                                          int32_t max_splits, void *hip_stream) {
  if (!a || !m) return ATTN_JVP_ERR_NULL;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return ATTN_JVP_ERR_HIP;
  void *ws = attnjvp::scratch_on(device);
  if (!ws) return ATTN_JVP_ERR_HIP;
  return attnjvp::fwd_split(a, m, max_splits, ws, attnjvp::kScratchBytes, hip_stream, true);
}
