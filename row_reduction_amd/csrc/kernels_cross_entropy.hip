// Compiled instances of the cross-entropy kernels on float rows (one translation
// unit per operator and storage type so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_cross_entropy(const rr_plan &p, const Args &a, void *stream) { return launch_op<kCrossEntropy, float>(p, a, stream); }

}  // namespace rowred
