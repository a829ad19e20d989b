// fa_bwd.hip -- placeholder until the backward kernels land.
#include <hip/hip_runtime.h>
#include "fa_kernels.hpp"
namespace fa {
hipError_t launch_bwd(const BwdArgs&) { return hipErrorNotSupported; }
}  // namespace fa
