// Backward kernels (identity straight-through at both QDQ sites).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

hipError_t launch_bwd(const BwdConfig&, const BwdKernelArgs&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gdn
