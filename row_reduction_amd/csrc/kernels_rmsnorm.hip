// Compiled instances of the RMSNorm kernels on float rows (one translation
// unit per operator and storage type so the instances build in parallel),
// and the static device buffer of the allocation-free RMSNorm entry point.
#include <mutex>

#include "device.h"

namespace rowred {

int launch_rmsnorm(const rr_plan &p, const Args &a, void *stream) { return launch_op<kRmsNorm, float>(p, a, stream); }

namespace {

// rmsnorm_f32_noalloc keeps its split-row partials in this array instead of a
// workspace the caller allocates. Each device the library runs on holds its
// own copy from the first kernel load until the process ends. In host code
// `scratch` names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device is passed to kernels.
static __device__ __align__(256) unsigned char scratch[RR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_addr[kMaxDevices];  // written once per device, under its once_flag

}  // namespace

int noalloc_scratch(void *stream, void **out) {
    // The kernels run on the stream's device, so the buffer is that
    // device's copy (the null stream: the calling thread's current device).
    int dev = -1;
    const hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                           : hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return RR_ERR_INVALID_ARGUMENT;
    }
    if (dev < 0 || dev >= kMaxDevices) return RR_ERR_UNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        // The lookup answers for the current device: make it `dev` for the
        // call and restore the caller's afterwards.
        int prev = -1;
        void *addr = nullptr;
        if (hipGetDevice(&prev) == hipSuccess && (prev == dev || hipSetDevice(dev) == hipSuccess)) {
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_addr[dev] = addr;
            if (prev != dev) (void)hipSetDevice(prev);
        }
        (void)hipGetLastError();  // a failed lookup must not fail the caller's later launches
    });
    if (g_scratch_addr[dev] == nullptr) return RR_ERR_LAUNCH;
    *out = g_scratch_addr[dev];
    return RR_OK;
}

}  // namespace rowred
