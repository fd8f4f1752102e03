// plan_scratch.hip -- the library's own device memory for plans built by
// moe_prefill_plan_device_noalloc (callers that cannot allocate: code under
// HIP graph capture, tight serving loops, harnesses that forbid it).
//
// One file-scope array per device holds the plan workspace.  Host code never
// passes the array's name to a kernel or a copy (in host code it is only a
// stand-in for the symbol): its device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and that address is
// what the launches take.  Every plan built this way on a device lives in
// the same array, so a new one overwrites the previous one; calls that
// overlap on one device race.
#include "internal.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace moe {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kScratchMaxDevices = 64;

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kScratchMaxDevices] = {};

// Offsets of experts at a constant stride: off[e] = first + e * stride.
__global__ __launch_bounds__(256) void stride_offsets_kernel(uint64_t *gu_off, uint64_t gu_first,
                                                             uint64_t gu_stride, uint64_t *dn_off,
                                                             uint64_t dn_first, uint64_t dn_stride,
                                                             int n_expert) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= n_expert) return;
    gu_off[e] = gu_first + uint64_t(e) * gu_stride;
    dn_off[e] = dn_first + uint64_t(e) * dn_stride;
}

}  // namespace

hipError_t scratch_workspace(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        // the current device is `dev`: this is its copy of the array
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_stride_offsets(uint64_t *gu_off, uint64_t gu_first, uint64_t gu_stride,
                                 uint64_t *dn_off, uint64_t dn_first, uint64_t dn_stride,
                                 int n_expert, hipStream_t stream) {
    if (n_expert <= 0) return hipSuccess;
    hipLaunchKernelGGL(stride_offsets_kernel, dim3((n_expert + 255) / 256), dim3(256), 0, stream, gu_off,
                       gu_first, gu_stride, dn_off, dn_first, dn_stride, n_expert);
    return hipGetLastError();
}

}  // namespace moe
