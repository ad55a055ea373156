// Compiled instances of the LayerNorm kernels on bfloat16 rows (float arithmetic).
#include "device.h"

namespace rowred {

int launch_layernorm_bf16(const rr_plan &p, const Args &a, void *stream) { return launch_op<kLayerNorm, bf16_t>(p, a, stream); }

}  // namespace rowred
