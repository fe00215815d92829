// hip_stubs.cpp -- CPU stand-ins for the HIP runtime calls and kernel
// launchers that the host code of libattn_mi355x.so makes, so that
// attn_api.cpp and l2norm_api.cpp can be built with gcc under AddressSanitizer
// and UndefinedBehaviorSanitizer and driven without a GPU.  Every launcher
// records the parameter block it was given; the
// runtime stubs report a configurable device (compute units, XCDs) and keep
// a HIP error state that a test can make sticky.  Like the real launchers,
// each stub returns hipGetLastError() after its "launch", so an error left
// by earlier work shows up unless the caller cleared it first.
#include <hip/hip_runtime.h>

#include "../../online_softmax_fusion_amd/csrc/attn_kernels.h"
#include "stub_state.h"

StubState g_stub;

extern "C" {

hipError_t hipGetDevice(int *device) {
    *device = g_stub.device;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int device) {
    if (device != g_stub.device) return hipErrorInvalidDevice;
    if (attr == hipDeviceAttributeMultiprocessorCount) {
        *value = g_stub.cus;
        return hipSuccess;
    }
    if (attr == hipDeviceAttributeNumberOfXccs) {
        *value = g_stub.xcds;
        return hipSuccess;
    }
    return hipErrorInvalidValue;
}

hipError_t hipGetLastError(void) {
    const hipError_t e = g_stub.last_error;
    g_stub.last_error = hipSuccess;
    return e;
}

}  // extern "C"

namespace attn {

hipError_t launch_prefill_bf16(const FwdParams &p, hipStream_t) {
    g_stub.fwd = p;
    g_stub.launches.push_back("prefill_bf16");
    return hipGetLastError();
}
hipError_t launch_prefill_part_bf16(const FwdParams &p, hipStream_t) {
    g_stub.fwd = p;
    g_stub.launches.push_back("prefill_part_bf16");
    return hipGetLastError();
}
hipError_t launch_decode_bf16(const FwdParams &p, hipStream_t) {
    g_stub.fwd = p;
    g_stub.launches.push_back("decode_bf16");
    return hipGetLastError();
}
hipError_t launch_rows_f32(const FwdParams &p, int partial, hipStream_t) {
    g_stub.fwd = p;
    g_stub.launches.push_back(partial ? "rows_f32_partial" : "rows_f32");
    return hipGetLastError();
}
hipError_t launch_combine(const CombineParams &c, hipStream_t) {
    g_stub.combine = c;
    g_stub.launches.push_back("combine");
    return hipGetLastError();
}
hipError_t launch_l2norm(const L2Params &p, hipStream_t) {
    g_stub.l2 = p;
    g_stub.launches.push_back("l2norm");
    return hipGetLastError();
}
hipError_t launch_bwd_bf16(const BwdParams &p, hipStream_t) {
    g_stub.fwd = p.f;
    g_stub.launches.push_back("bwd_bf16");
    return hipGetLastError();
}

}  // namespace attn
