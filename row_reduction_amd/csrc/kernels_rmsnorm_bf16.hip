// Compiled instances of the RMSNorm kernels on bfloat16 rows (float arithmetic).
#include "device.h"

namespace rowred {

int launch_rmsnorm_bf16(const rr_plan &p, const Args &a, void *stream) { return launch_op<kRmsNorm, bf16_t>(p, a, stream); }

}  // namespace rowred
