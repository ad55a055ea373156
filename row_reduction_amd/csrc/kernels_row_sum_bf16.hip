// Compiled instances of the row sum kernels on bfloat16 rows (float arithmetic).
#include "device.h"

namespace rowred {

int launch_row_sum_bf16(const rr_plan &p, const Args &a, void *stream) { return launch_op<kSum, bf16_t>(p, a, stream); }

}  // namespace rowred
