// Compiled instances of the RMSNorm kernels (one translation unit per operator
// so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_rmsnorm(const rr_plan &p, const Args &a, void *stream) { return launch_op<kRmsNorm>(p, a, stream); }

}  // namespace rowred
