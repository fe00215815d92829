// noalloc.hip -- attn_fwd_noalloc: the planned forward with its split-plan
// partials in a fixed device array of this library instead of a workspace.
//
// The array is a file-scope __device__ variable, so every device the library
// runs on holds its own copy (ATTN_NOALLOC_SCRATCH_BYTES) from the first use
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host that name is a stand-in, not a device address): the
// first call on a device looks up that device's copy with
// hipGetSymbolAddress, with the device current, and every later call on the
// device reuses that address.  Nothing in the array needs to start at zero:
// the split kernels write every partial (empty chunks included) before the
// combine reads it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/attn.h"

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// This device's copy of scratch; `device` must be the current device.
attn_status scratch_address(int device, void **out) {
    if (device < 0 || device >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
    void *ptr = g_scratch_ptr[device].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return ATTN_ERR_HIP;
        }
        // concurrent first calls store the same address
        g_scratch_ptr[device].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_fwd_noalloc(const attn_fwd_args *a, void *stream) {
    attn_status st = attn_validate_prefill(a);
    if (st != ATTN_OK) return st;
    if (a->B * a->Hq * a->Lq == 0) return ATTN_OK;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_ERR_HIP;
    }
    attn_fwd_plan plan;
    st = attn_fwd_choose_plan(a, attn_device_cu_count(device), &plan);
    if (st != ATTN_OK) return st;
    if (plan.method == ATTN_PLAN_PREFILL) return attn_fwd_prefill(a, stream);
    if (plan.workspace_bytes > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((st = scratch_address(device, &ws)) != ATTN_OK) return st;
    return attn_fwd(a, ws, (size_t)ATTN_NOALLOC_SCRATCH_BYTES, stream);
}
