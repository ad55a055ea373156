// Compiled instances of the cross-entropy kernels on bfloat16 rows (float arithmetic).
#include "device.h"

namespace rowred {

int launch_cross_entropy_bf16(const rr_plan &p, const Args &a, void *stream) { return launch_op<kCrossEntropy, bf16_t>(p, a, stream); }

}  // namespace rowred
