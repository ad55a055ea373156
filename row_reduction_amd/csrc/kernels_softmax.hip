// Compiled instances of the softmax kernels (one translation unit per operator
// so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_softmax(const rr_plan &p, const Args &a, void *stream) { return launch_op<kSoftmax>(p, a, stream); }

}  // namespace rowred
