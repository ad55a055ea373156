// Compiled instances of the cross-entropy kernels (one translation unit per operator
// so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_cross_entropy(const rr_plan &p, const Args &a, void *stream) { return launch_op<kCrossEntropy>(p, a, stream); }

}  // namespace rowred
