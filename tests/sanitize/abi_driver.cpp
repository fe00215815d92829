// abi_driver.cpp -- drives every entry point of include/attn.h and
// include/l2norm.h on the CPU (kernel launchers and HIP runtime stubbed by
// hip_stubs.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer:
// valid arguments, every kind of invalid argument, and sizes far past what
// the kernels hold (which must be refused without signed overflow).  Prints
// one line per failed check and exits non-zero if any failed.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "../../include/l2norm.h"
#include "stub_state.h"

namespace {

int g_failed = 0;
int g_checked = 0;

#define CHECK(cond)                                                              \
    do {                                                                         \
        ++g_checked;                                                             \
        if (!(cond)) {                                                           \
            ++g_failed;                                                          \
            std::printf("FAILED line %d: %s\n", __LINE__, #cond);                \
        }                                                                        \
    } while (0)

alignas(16) char g_buf[1 << 16];   // stands in for device memory (never dereferenced by the host code)

attn_fwd_args small_args() {
    attn_fwd_args a;
    std::memset(&a, 0, sizeof(a));
    a.B = 2; a.Hq = 8; a.Hkv = 2; a.Lq = 100; a.Lk = 300; a.D = 128;
    a.dtype = ATTN_BF16; a.o_dtype = ATTN_BF16;
    a.q = g_buf; a.k = g_buf; a.v = g_buf; a.o = g_buf;
    const int64_t q_st[3] = {8 * 100 * 128, 100 * 128, 128};
    const int64_t kv_st[3] = {2 * 300 * 128, 300 * 128, 128};
    std::memcpy(a.q_strides, q_st, sizeof(q_st));
    std::memcpy(a.o_strides, q_st, sizeof(q_st));
    std::memcpy(a.k_strides, kv_st, sizeof(kv_st));
    std::memcpy(a.v_strides, kv_st, sizeof(kv_st));
    a.scale = 0.0883883f;
    a.lse = reinterpret_cast<float *>(g_buf);
    return a;
}

void test_valid_calls() {
    attn_fwd_args a = small_args();
    g_stub.launches.clear();
    CHECK(attn_validate_prefill(&a) == ATTN_OK);
    CHECK(attn_fwd_prefill(&a, nullptr) == ATTN_OK);
    CHECK(!g_stub.launches.empty() && g_stub.launches.back() == "prefill_bf16");
    CHECK(g_stub.fwd.num_cus == 256 && g_stub.fwd.num_xcds == 8);
    CHECK(g_stub.fwd.G == 4 && g_stub.fwd.Lk == 300);

    // the device's topology reaches the kernels' parameters
    g_stub.device = 1; g_stub.cus = 32; g_stub.xcds = 1;
    CHECK(attn_fwd_prefill(&a, nullptr) == ATTN_OK);
    CHECK(g_stub.fwd.num_cus == 32 && g_stub.fwd.num_xcds == 1);
    CHECK(attn_device_cu_count(1) == 32 && attn_device_xcd_count(1) == 1);
    g_stub.device = 0; g_stub.cus = 256; g_stub.xcds = 8;

    float *part = reinterpret_cast<float *>(g_buf);
    CHECK(attn_validate_decode(&a, 4, part, part, part) == ATTN_OK);
    CHECK(attn_fwd_decode_splitk(&a, 4, part, part, part, nullptr) == ATTN_OK);
    CHECK(g_stub.launches.back() == "decode_bf16" && g_stub.fwd.chunk == 96);
    CHECK(attn_fwd_prefill_splitk(&a, 2, part, part, part, nullptr) == ATTN_OK);
    CHECK(g_stub.launches.back() == "prefill_part_bf16" && g_stub.fwd.chunk == 192);
    CHECK(attn_splitk_combine(part, part, part, 2, 8, 100, 128, 4, g_buf, ATTN_BF16, a.o_strides, a.lse, nullptr) ==
          ATTN_OK);
    CHECK(g_stub.launches.back() == "combine" && g_stub.combine.S == 4);

    attn_fwd_plan plan;
    CHECK(attn_fwd_choose_plan(&a, 256, &plan) == ATTN_OK);
    CHECK(attn_fwd(&a, g_buf, 0, nullptr) == (plan.method == ATTN_PLAN_PREFILL ? ATTN_OK : ATTN_ERR_WORKSPACE));

    a.dtype = ATTN_F32;
    CHECK(attn_fwd_prefill(&a, nullptr) == ATTN_OK && g_stub.launches.back() == "rows_f32");
    a.dtype = ATTN_BF16;

    attn_bwd_args g;
    std::memset(&g, 0, sizeof(g));
    g.fwd = a;
    g.dout = g_buf; g.dq = g_buf; g.dk = g_buf; g.dv = g_buf;
    std::memcpy(g.dout_strides, a.q_strides, sizeof(a.q_strides));
    std::memcpy(g.dq_strides, a.q_strides, sizeof(a.q_strides));
    std::memcpy(g.dk_strides, a.k_strides, sizeof(a.k_strides));
    std::memcpy(g.dv_strides, a.k_strides, sizeof(a.k_strides));
    g.grad_dtype = ATTN_BF16;
    g.workspace = reinterpret_cast<float *>(g_buf);
    CHECK(attn_validate_bwd(&g) == ATTN_OK);
    CHECK(attn_bwd(&g, nullptr) == ATTN_OK && g_stub.launches.back() == "bwd_bf16");
    CHECK(attn_bwd_workspace_bytes(2, 8, 100) == 2 * 1600 * sizeof(float));

    l2norm_args x;
    std::memset(&x, 0, sizeof(x));
    x.rows = 4; x.H = 4096; x.x = g_buf; x.x_stride = 4096; x.x_dtype = ATTN_BF16;
    x.y = g_buf; x.y_stride = 4096; x.y_dtype = ATTN_BF16; x.norm = reinterpret_cast<float *>(g_buf);
    CHECK(l2norm_validate(&x, 1) == ATTN_OK);
    CHECK(l2norm_rows(&x, 1, nullptr, 0, nullptr) == ATTN_OK && g_stub.launches.back() == "l2norm");
    CHECK(l2norm_rows(&x, 4, g_buf, l2norm_workspace_bytes(4, 4), nullptr) == ATTN_OK);
    CHECK(l2norm_rows(&x, 4, g_buf, 8, nullptr) == ATTN_ERR_WORKSPACE);
}

void test_sticky_error_is_not_reported() {
    // an error left by earlier, unrelated work on the thread
    attn_fwd_args a = small_args();
    g_stub.last_error = hipErrorOutOfMemory;
    CHECK(attn_fwd_prefill(&a, nullptr) == ATTN_OK);
    g_stub.last_error = hipErrorOutOfMemory;
    float *part = reinterpret_cast<float *>(g_buf);
    CHECK(attn_fwd_decode_splitk(&a, 4, part, part, part, nullptr) == ATTN_OK);
    g_stub.last_error = hipErrorOutOfMemory;
    CHECK(attn_splitk_combine(part, part, part, 2, 8, 100, 128, 4, g_buf, ATTN_BF16, a.o_strides, nullptr,
                              nullptr) == ATTN_OK);
    g_stub.last_error = hipErrorOutOfMemory;
    l2norm_args x;
    std::memset(&x, 0, sizeof(x));
    x.rows = 4; x.H = 4096; x.x = g_buf; x.x_stride = 4096; x.x_dtype = ATTN_BF16; x.norm = a.lse;
    CHECK(l2norm_rows(&x, 1, nullptr, 0, nullptr) == ATTN_OK);
    CHECK(g_stub.last_error == hipSuccess);
}

void test_invalid_arguments() {
    CHECK(attn_validate_prefill(nullptr) == ATTN_ERR_INVALID_ARG);
    CHECK(attn_fwd_prefill(nullptr, nullptr) == ATTN_ERR_INVALID_ARG);
    CHECK(attn_bwd(nullptr, nullptr) == ATTN_ERR_INVALID_ARG);
    CHECK(l2norm_rows(nullptr, 1, nullptr, 0, nullptr) == ATTN_ERR_INVALID_ARG);
    attn_fwd_args a = small_args();
    a.Hq = 7;
    CHECK(attn_validate_prefill(&a) == ATTN_ERR_INVALID_ARG);   // Hq % Hkv
    a = small_args(); a.D = 96;
    CHECK(attn_validate_prefill(&a) == ATTN_ERR_UNSUPPORTED);
    a = small_args(); a.q = g_buf + 2;
    CHECK(attn_validate_prefill(&a) == ATTN_ERR_UNSUPPORTED);
    a = small_args(); a.k = nullptr;
    CHECK(attn_validate_prefill(&a) == ATTN_ERR_INVALID_ARG);
    a = small_args(); a.scale = 1.0f / 0.0f;
    CHECK(attn_validate_prefill(&a) == ATTN_ERR_INVALID_ARG);
    a = small_args(); a.bias_kind = 7;
    CHECK(attn_validate_prefill(&a) == ATTN_ERR_INVALID_ARG);
    a = small_args(); a.q_strides[1] = -128;
    CHECK(attn_validate_prefill(&a) == ATTN_ERR_INVALID_ARG);
    a = small_args();
    float *part = reinterpret_cast<float *>(g_buf);
    CHECK(attn_validate_decode(&a, 0, part, part, part) == ATTN_ERR_INVALID_ARG);
    CHECK(attn_validate_decode(&a, 70000, part, part, part) == ATTN_ERR_INVALID_ARG);
    CHECK(attn_fwd_decode_splitk(&a, 4, nullptr, part, part, nullptr) == ATTN_ERR_INVALID_ARG);
    attn_fwd_plan plan;
    CHECK(attn_fwd_choose_plan(&a, 256, nullptr) == ATTN_ERR_INVALID_ARG);
    CHECK(attn_fwd_choose_plan(nullptr, 256, &plan) == ATTN_ERR_INVALID_ARG);
    CHECK(std::strlen(attn_status_str(static_cast<attn_status>(99))) > 0);
}

void test_huge_sizes() {
    const int64_t big[] = {(int64_t)1 << 31, (int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX};
    float *part = reinterpret_cast<float *>(g_buf);
    for (int64_t v : big) {
        for (int field = 0; field < 6; ++field) {
            attn_fwd_args a = small_args();
            int64_t *dims[6] = {&a.B, &a.Hq, &a.Hkv, &a.Lq, &a.Lk, &a.D};
            *dims[field] = v;
            if (field == 1) a.Hq = v - v % a.Hkv;   // keep Hq % Hkv == 0
            if (field == 2) a.Hq = v;
            const attn_status st = attn_validate_prefill(&a);
            if (st != ATTN_ERR_UNSUPPORTED) std::printf("field %d value %lld: status %d\n", field, (long long)v, st);
            CHECK(st == ATTN_ERR_UNSUPPORTED);
            CHECK(attn_fwd_prefill(&a, nullptr) == st);
            CHECK(attn_validate_decode(&a, 4, part, part, part) == st);
            attn_fwd_plan plan;
            CHECK(attn_fwd_choose_plan(&a, 256, &plan) == st);
        }
        // all of them at once
        attn_fwd_args a = small_args();
        a.B = v; a.Hq = v; a.Hkv = v; a.Lq = v; a.Lk = v;
        CHECK(attn_validate_prefill(&a) == ATTN_ERR_UNSUPPORTED);
        // products of in-range sizes past the grids
        a = small_args();
        a.B = 0x7fffffff; a.Hq = 0x7fffffff; a.Hkv = 1; a.Lq = 0x3fffffff;
        CHECK(attn_validate_prefill(&a) == ATTN_ERR_UNSUPPORTED);
        // pure host functions: no overflow, results in range
        CHECK(attn_decode_partial_bytes(v, v, v, 128, 4) == 0);
        CHECK(attn_bwd_workspace_bytes(v, v, v) == 0);
        const int32_t s1 = attn_decode_choose_splits(v, v, 1, v, v, 256);
        CHECK(s1 >= 1 && s1 <= 65535);
        const int32_t s2 = attn_prefill_choose_splits(v, v, v, v, 256);
        CHECK(s2 >= 1 && s2 <= 65535);
        CHECK(attn_splitk_combine(part, part, part, v, v, v, 128, 4, g_buf, ATTN_BF16, small_args().o_strides,
                                  nullptr, nullptr) == ATTN_ERR_UNSUPPORTED);
        l2norm_args x;
        std::memset(&x, 0, sizeof(x));
        x.rows = v; x.H = v; x.x = g_buf; x.x_stride = v; x.x_dtype = ATTN_F32; x.norm = part;
        CHECK(l2norm_validate(&x, 4) == ATTN_ERR_UNSUPPORTED);
        x.rows = 4; x.H = 4096; x.x_stride = v;
        CHECK(l2norm_validate(&x, 4) == (v > ((int64_t)1 << 40) ? ATTN_ERR_UNSUPPORTED : ATTN_OK));
        if (v >= ((int64_t)1 << 62)) CHECK(l2norm_workspace_bytes(v, 65535) == 0);
        const int32_t s3 = l2norm_choose_splits(v, v, ATTN_F32, 256);
        CHECK(s3 >= 1 && s3 <= 65535);
    }
}

}  // namespace

int main() {
    test_valid_calls();
    test_sticky_error_is_not_reported();
    test_invalid_arguments();
    test_huge_sizes();
    std::printf("%d checks, %d failed\n", g_checked, g_failed);
    return g_failed == 0 ? 0 : 1;
}
