// stub_state.h -- what the CPU stand-ins of hip_stubs.cpp report and record.
#pragma once

#include <string>
#include <vector>

#include "../../online_softmax_fusion_amd/csrc/attn_kernels.h"

struct StubState {
    int device = 0;
    int cus = 256;
    int xcds = 8;
    hipError_t last_error = hipSuccess;   // the thread's HIP error state
    attn::FwdParams fwd{};
    attn::CombineParams combine{};
    attn::L2Params l2{};
    std::vector<std::string> launches;
};

extern StubState g_stub;
