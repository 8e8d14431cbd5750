// Kernel launchers for a host-only (sanitizer) link of the library's C++
// sources, which leaves out the .hip files.  A host without a HIP device
// never reaches them (the entry points stop at hipGetDevice); if one were
// reached it reports a launch failure.
#include "internal.h"

namespace attnjvp {

int launch_bf16(const KernelParams &, int, bool, void *) { return hipErrorInvalidDeviceFunction; }
int launch_f32(const KernelParams &, int, bool, void *) { return hipErrorInvalidDeviceFunction; }
int launch_merge(const MergeParams &, int, bool, bool, void *) {
  return hipErrorInvalidDeviceFunction;
}
int launch_bwd_bf16_wide(const BwdParams &, int, void *) { return hipErrorInvalidDeviceFunction; }
int launch_bwd_f32(const BwdParams &, int, void *) { return hipErrorInvalidDeviceFunction; }

}  // namespace attnjvp
