// Compiled instances of the residual LayerNorm kernels on float rows (one translation
// unit per operator and storage type so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_residual_layernorm(const rr_plan &p, const Args &a, void *stream) { return launch_op<kResidualLayerNorm, float>(p, a, stream); }

}  // namespace rowred
