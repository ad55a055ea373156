// Compiled instances of the softmax kernels on bfloat16 rows (float arithmetic).
#include "device.h"

namespace rowred {

int launch_softmax_bf16(const rr_plan &p, const Args &a, void *stream) { return launch_op<kSoftmax, bf16_t>(p, a, stream); }

}  // namespace rowred
