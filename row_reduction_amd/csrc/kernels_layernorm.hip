// Compiled instances of the LayerNorm kernels (one translation unit per operator
// so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_layernorm(const rr_plan &p, const Args &a, void *stream) { return launch_op<kLayerNorm>(p, a, stream); }

}  // namespace rowred
