// gdr_bwd.hip -- backward kernels (placeholder until the reverse pass lands).
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {
hipError_t launch_dstate(DType, int, int, const DStateParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_grads(DType, int, const GradParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdr
