// Compiled instances of the softmax kernels on float rows (one translation
// unit per operator and storage type so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_softmax(const rr_plan &p, const Args &a, void *stream) { return launch_op<kSoftmax, float>(p, a, stream); }

}  // namespace rowred
