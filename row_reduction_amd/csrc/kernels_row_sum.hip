// Compiled instances of the row sum kernels on float rows (one translation
// unit per operator and storage type so the instances build in parallel).
#include "device.h"

namespace rowred {

int launch_row_sum(const rr_plan &p, const Args &a, void *stream) { return launch_op<kSum, float>(p, a, stream); }

}  // namespace rowred
