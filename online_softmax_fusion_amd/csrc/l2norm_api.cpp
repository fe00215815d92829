// l2norm_api.cpp -- the C ABI of include/l2norm.h: argument checks on the host,
// split choice, launches on the caller's stream.
#include "../../include/l2norm.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_kernels.h"

namespace {

constexpr int64_t kMaxOnepassVecs = 16 * 64;   // 16-byte vectors of a row the one-pass kernel holds

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t elem_bytes(int32_t dt) { return dt == ATTN_BF16 ? 2 : 4; }
bool valid_dtype(int32_t dt) { return dt == ATTN_F32 || dt == ATTN_BF16; }

// 16-byte vectors per chunk of a split-K call
int64_t chunk_vecs(int64_t H, int32_t dt, int32_t S) {
    const int64_t nvec = H * elem_bytes(dt) / 16;
    return (nvec + S - 1) / S;
}

}  // namespace

extern "C" {

int64_t l2norm_max_onepass(int32_t x_dtype) { return kMaxOnepassVecs * 16 / elem_bytes(x_dtype); }

size_t l2norm_workspace_bytes(int64_t rows, int32_t num_splits) {
    size_t n;
    if (rows <= 0 || num_splits <= 1 || __builtin_mul_overflow((size_t)rows, (size_t)num_splits * 8u, &n)) return 0;
    return n;
}

int32_t l2norm_choose_splits(int64_t rows, int64_t H, int32_t x_dtype, int32_t cu_count) {
    if (rows <= 0 || H <= l2norm_max_onepass(x_dtype)) return 1;
    const int64_t cu = cu_count > 0 ? cu_count : 256;
    int64_t S = 4 * cu / rows + (4 * cu % rows != 0);        // four workgroups per compute unit
    if (H > INT64_MAX / 4) H = INT64_MAX / 4;
    const int64_t max_by_len = H * elem_bytes(x_dtype) / 4096; // at least 4096 bytes per chunk
    if (S > max_by_len) S = max_by_len;
    if (S < 2) S = 2;                                       // the row does not fit one pass
    if (S > 65535) S = 65535;
    return (int32_t)S;
}

attn_status l2norm_validate(const l2norm_args *a, int32_t num_splits) {
    if (a == nullptr) return ATTN_ERR_INVALID_ARG;
    if (a->rows < 0 || a->H < 0 || !valid_dtype(a->x_dtype)) return ATTN_ERR_INVALID_ARG;
    if (a->y != nullptr && !valid_dtype(a->y_dtype)) return ATTN_ERR_INVALID_ARG;
    if (num_splits < 1) return ATTN_ERR_INVALID_ARG;
    // sizes the kernels hold (this also keeps the products below from overflowing)
    if (a->rows > 0x7fffffff || a->H > ((int64_t)1 << 40) || a->x_stride > ((int64_t)1 << 40) ||
        a->y_stride > ((int64_t)1 << 40))
        return ATTN_ERR_UNSUPPORTED;
    if (a->x_stride < a->H || (a->y != nullptr && a->y_stride < a->H)) return ATTN_ERR_INVALID_ARG;
    if (a->rows > 0 && a->H > 0 && a->x == nullptr) return ATTN_ERR_INVALID_ARG;
    if (a->rows > 0 && a->y == nullptr && a->norm == nullptr) return ATTN_ERR_INVALID_ARG;   // nothing to write
    if (a->norm != nullptr && (reinterpret_cast<uintptr_t>(a->norm) & 3u)) return ATTN_ERR_INVALID_ARG;
    // 16-byte vectors of x and y
    const int64_t vx = 16 / elem_bytes(a->x_dtype);
    if (!aligned16(a->x) || a->H % vx || a->x_stride % vx) return ATTN_ERR_UNSUPPORTED;
    if (a->y != nullptr) {
        // each input vector of vx elements is stored as one piece of vx * (y element) bytes
        // (two 16-byte pieces for bf16 -> fp32): that piece's alignment
        const int64_t piece = vx * elem_bytes(a->y_dtype) < 16 ? vx * elem_bytes(a->y_dtype) : 16;
        if ((reinterpret_cast<uintptr_t>(a->y) & (uintptr_t)(piece - 1)) ||
            (a->y_stride * elem_bytes(a->y_dtype)) % piece)
            return ATTN_ERR_UNSUPPORTED;
    }
    if (num_splits == 1 && a->H > l2norm_max_onepass(a->x_dtype)) return ATTN_ERR_UNSUPPORTED;
    if (a->H * elem_bytes(a->x_dtype) / 16 > 0x7fffffff || a->rows * (int64_t)num_splits > 0x7fffffff ||
        (a->rows + 3) / 4 > 0x7fffffff)
        return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

attn_status l2norm_rows(const l2norm_args *a, int32_t num_splits, void *workspace, size_t workspace_bytes,
                        void *stream) {
    attn_status st = l2norm_validate(a, num_splits);
    if (st != ATTN_OK) return st;
    if (a->rows == 0) return ATTN_OK;
    if (num_splits > 1) {
        if (workspace == nullptr || workspace_bytes < l2norm_workspace_bytes(a->rows, num_splits))
            return ATTN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
    }
    attn::L2Params p{};
    p.x = a->x;
    p.x_stride = a->x_stride;
    p.y = a->y;
    p.y_stride = a->y_stride;
    p.norm = a->norm;
    p.rows = a->rows;
    p.H = a->H;
    p.x_bf16 = a->x_dtype == ATTN_BF16;
    p.y_bf16 = a->y_dtype == ATTN_BF16;
    p.S = num_splits;
    p.chunk_vecs = (int)chunk_vecs(a->H, a->x_dtype, num_splits);
    p.ws = workspace;
    (void)hipGetLastError();   // report this call's launch error only
    const hipError_t err = attn::launch_l2norm(p, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t l2norm_args_size(void) { return sizeof(l2norm_args); }

}  // extern "C"
