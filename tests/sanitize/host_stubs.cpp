// host_stubs.cpp -- the device launchers of libmoe_prefill.so replaced by
// stubs, so that the host side (moe_prefill.cpp: argument checks, host plans,
// queries, the ABI's exports) can be built with g++ and the address and
// undefined-behaviour sanitizers and exercised on a machine without a GPU.
// Every stub reports an error: no CPU test reaches a launch.
#include "../../quantized_moe_expert_scatter_amd/csrc/internal.h"

namespace moe {

hipError_t launch_quantize_scatter(const float *, int, int, int, const int32_t *, uint8_t *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_swiglu_q8(const float *, int, int, uint8_t *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_expert_product(const ProductArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_expert_small(const ProductArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_device_plan(const int32_t *, int, int, int, int, int, uint8_t *, const PlanLayout &,
                              hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_combine(const float *, const float *, int, int, int, float *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_weight_pack(const uint8_t *, uint8_t *, uint64_t, int, int, int, int, bool, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t scratch_workspace(void **) { return hipErrorNotSupported; }
hipError_t launch_stride_offsets(uint64_t *, uint64_t, uint64_t, uint64_t *, uint64_t, uint64_t, int,
                                 hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
