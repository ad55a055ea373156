// Compiled instances of the RMSNorm kernels on float rows (one translation
// unit per operator and storage type so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_rmsnorm(const rr_plan &p, const Args &a, void *stream) { return launch_op<kRmsNorm, float>(p, a, stream); }

}  // namespace rowred
