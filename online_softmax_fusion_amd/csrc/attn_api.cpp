// attn_api.cpp -- the C ABI of include/attn.h: argument checks on the host,
// choice of kernel instantiation, and launches on the caller's stream.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "attn_kernels.h"

using attn::FwdParams;

namespace {

constexpr int64_t kIntMax = 0x7fffffff;

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

int64_t elem_size(int32_t dt) { return dt == ATTN_BF16 ? 2 : 4; }

bool valid_dtype(int32_t dt) { return dt == ATTN_F32 || dt == ATTN_BF16; }

// a * b * c, false when the product of these non-negative values leaves int64
bool mul3(int64_t a, int64_t b, int64_t c, int64_t &out) {
    int64_t t;
    return !__builtin_mul_overflow(a, b, &t) && !__builtin_mul_overflow(t, c, &out);
}

// ceil(a / b) for 0 <= a and b >= 1, without forming a + b - 1
int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

// a * b for non-negative values, saturating at INT64_MAX
int64_t sat_mul(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

// Launches `fn` with the HIP error state cleared first, so that a launch
// error reported afterwards belongs to this call and not to earlier,
// unrelated work on the thread.
template <class F>
attn_status launch(F fn) {
    (void)hipGetLastError();
    return fn() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Checks shared by prefill and decode.
attn_status check_common(const attn_fwd_args *a) {
    if (a == nullptr) return ATTN_ERR_INVALID_ARG;
    if (a->B < 0 || a->Hq < 1 || a->Hkv < 1 || a->Lq < 0 || a->Lk < 0 || a->D < 1)
        return ATTN_ERR_INVALID_ARG;
    if (a->Hq % a->Hkv != 0) return ATTN_ERR_INVALID_ARG;
    if (!valid_dtype(a->dtype)) return ATTN_ERR_INVALID_ARG;
    if (a->causal != 0 && a->causal != 1) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(a->scale)) return ATTN_ERR_INVALID_ARG;
    for (int t = 0; t < 3; ++t)
        if (a->q_strides[t] < 0 || a->k_strides[t] < 0 || a->v_strides[t] < 0) return ATTN_ERR_INVALID_ARG;
    if (a->bias_kind != ATTN_BIAS_NONE && a->bias_kind != ATTN_BIAS_DENSE && a->bias_kind != ATTN_BIAS_ALIBI)
        return ATTN_ERR_INVALID_ARG;
    // every size is held in 32 bits by the kernels; bounding each one first
    // also keeps the products below from overflowing
    if (a->B > kIntMax || a->Hq > kIntMax || a->Hkv > kIntMax || a->Lq > kIntMax || a->Lk > kIntMax ||
        a->D > kIntMax)
        return ATTN_ERR_UNSUPPORTED;
    int64_t rows = 0, kv_rows = 0;
    if (!mul3(a->B, a->Hq, a->Lq, rows) || !mul3(a->B, a->Hkv, a->Lk, kv_rows)) return ATTN_ERR_UNSUPPORTED;
    const bool any_q = rows > 0;
    const bool any_kv = kv_rows > 0;
    if (any_q && a->q == nullptr) return ATTN_ERR_INVALID_ARG;
    if (any_q && any_kv && (a->k == nullptr || a->v == nullptr)) return ATTN_ERR_INVALID_ARG;
    if (a->bias_kind == ATTN_BIAS_DENSE) {
        if (any_q && any_kv && a->bias == nullptr) return ATTN_ERR_INVALID_ARG;
        if (!valid_dtype(a->bias_dtype)) return ATTN_ERR_INVALID_ARG;
        for (int t = 0; t < 4; ++t)
            if (a->bias_strides[t] < 0) return ATTN_ERR_INVALID_ARG;
        if (!aligned(a->bias, (uintptr_t)elem_size(a->bias_dtype))) return ATTN_ERR_UNSUPPORTED;
    }
    if (a->bias_kind == ATTN_BIAS_ALIBI && any_q && a->alibi_slopes == nullptr) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(a->softcap) || a->softcap < 0.f) return ATTN_ERR_INVALID_ARG;
    if (a->window != 0 && a->window != 1) return ATTN_ERR_INVALID_ARG;

    // implemented shapes
    if (a->D != 64 && a->D != 128) return ATTN_ERR_UNSUPPORTED;
    if (a->Lq > kIntMax / 2 || a->Lk > kIntMax / 2 || a->B * a->Hq > kIntMax || rows > kIntMax)
        return ATTN_ERR_UNSUPPORTED;
    // 16-byte vector loads of q, k, v rows
    const int64_t vec = 16 / elem_size(a->dtype);
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16)) return ATTN_ERR_UNSUPPORTED;
    for (int t = 0; t < 3; ++t)
        if (a->q_strides[t] % vec || a->k_strides[t] % vec || a->v_strides[t] % vec) return ATTN_ERR_UNSUPPORTED;
    // key rows are addressed with 32-bit offsets inside a tile of keys
    if (a->k_strides[2] > (1 << 24) || a->v_strides[2] > (1 << 24)) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

FwdParams make_params(const attn_fwd_args *a) {
    FwdParams p{};
    p.q = a->q; p.k = a->k; p.v = a->v;
    p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_sl = a->q_strides[2];
    p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_sl = a->k_strides[2];
    p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_sl = a->v_strides[2];
    p.o = a->o;
    p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1]; p.o_sl = a->o_strides[2];
    p.o_bf16 = a->o_dtype == ATTN_BF16;
    p.lse = a->lse;
    p.B = (int)a->B; p.Hq = (int)a->Hq; p.Hkv = (int)a->Hkv; p.G = (int)(a->Hq / a->Hkv);
    p.Lq = (int)a->Lq; p.Lk = (int)a->Lk; p.D = (int)a->D;
    p.causal = a->causal;
    p.scale = a->scale;
    p.scale_log2 = a->scale * 1.4426950408889634f;
    p.bias = a->bias;
    p.bias_sb = a->bias_strides[0]; p.bias_sh = a->bias_strides[1];
    p.bias_si = a->bias_strides[2]; p.bias_sj = a->bias_strides[3];
    p.slopes = a->alibi_slopes;
    if (a->bias_kind == ATTN_BIAS_ALIBI)
        p.bias_kind = attn::kBiasAlibi;
    else if (a->bias_kind == ATTN_BIAS_DENSE)
        p.bias_kind = a->bias_dtype == ATTN_BF16 ? attn::kBiasDenseBf16 : attn::kBiasDenseF32;
    else
        p.bias_kind = attn::kBiasNone;
    if (a->softcap > 0.f) {
        p.bias_kind = p.bias_kind == attn::kBiasNone ? (int)attn::kBiasNoneCap : p.bias_kind + 5;
        p.softcap = a->softcap;
        p.cap_l2 = a->softcap * 1.4426950408889634f;
        p.cap_k = 2.f / a->softcap;
        p.cap_inv = 1.f / p.cap_l2;
        // the polynomial form for raw scores s with |s scale / softcap| <= 1/2:
        // capped (log2) = s scale_log2 P(k s^2), k = (scale / softcap)^2
        if (a->scale > 0.f) {
            const double k = ((double)a->scale / a->softcap) * ((double)a->scale / a->softcap);
            double kp = 1.0;
            bool finite = true;
            for (int i = 0; i < 4; ++i, kp *= k) {
                p.cap_q[i] = (float)((double)p.scale_log2 * attn::kTanhPoly[i] * kp);
                finite = finite && std::isfinite(p.cap_q[i]);
            }
            // a cap so small against the scale that the coefficients leave the
            // float range: every tile takes the exp form (|s| > -1 always)
            p.cap_s0 = finite ? (float)(0.5 * a->softcap / a->scale) : -1.f;
        }
    }
    p.window = a->window;
    p.win_left = a->window_left;
    p.win_right = a->window_right;
    return p;
}

// Compute units and XCDs of the current device, for the kernels' work order
// and the launch rules that depend on how many workgroups the device holds.
attn_status device_topology(FwdParams &p) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return ATTN_ERR_HIP;
    const int32_t cus = attn_device_cu_count(device);
    const int32_t xcds = attn_device_xcd_count(device);
    if (cus <= 0 || xcds <= 0) return ATTN_ERR_HIP;
    p.num_cus = cus;
    p.num_xcds = xcds;
    return ATTN_OK;
}

// rows of one workspace array, rounded up to 16 bytes
int64_t bwd_rows_padded(int64_t rows) { return (rows + 3) / 4 * 4; }

int32_t chunk_len(int64_t Lk, int32_t S) {
    const int64_t per = ceil_div(Lk, (int64_t)S * 32);
    return (int32_t)(per < 1 ? 32 : per * 32);
}

// split prefill: enough (query tile, key chunk) workgroups for kPrefillSplitSlots
// per compute unit, with at least kPrefillSplitMinKeys keys per chunk; on a
// prefill grid that already gives every compute unit a workgroup, only chunks
// of kPrefillSplitLongChunk keys or more (the combine's cost is paid per row)
constexpr int64_t kPrefillSplitSlots = 2;
constexpr int64_t kPrefillSplitMinKeys = 1024;
constexpr int64_t kPrefillSplitLongChunk = 8192;
// grouped split-K only for decode-like query lengths
constexpr int64_t kSplitKMaxLq = 16;

// keys per chunk of the split prefill: whole 64-key tiles
int64_t prefill_chunk_len(int64_t Lk, int32_t num_splits) {
    const int64_t per = ceil_div(Lk, 64 * (int64_t)num_splits);
    return 64 * (per > 0 ? per : 1);
}

}  // namespace

extern "C" {

attn_status attn_validate_prefill(const attn_fwd_args *a) {
    attn_status st = check_common(a);
    if (st != ATTN_OK) return st;
    if (!valid_dtype(a->o_dtype)) return ATTN_ERR_INVALID_ARG;
    for (int t = 0; t < 3; ++t)
        if (a->o_strides[t] < 0) return ATTN_ERR_INVALID_ARG;
    if (a->B * a->Hq * a->Lq > 0) {
        if (a->o == nullptr) return ATTN_ERR_INVALID_ARG;
        const int64_t vec = 16 / elem_size(a->o_dtype);
        if (!aligned(a->o, 16)) return ATTN_ERR_UNSUPPORTED;
        for (int t = 0; t < 3; ++t)
            if (a->o_strides[t] % vec) return ATTN_ERR_UNSUPPORTED;
        if (a->lse != nullptr && !aligned(a->lse, 4)) return ATTN_ERR_INVALID_ARG;
    }
    return ATTN_OK;
}

attn_status attn_validate_decode(const attn_fwd_args *a, int32_t num_splits, const float *o_part,
                                 const float *m_part, const float *l_part) {
    attn_status st = check_common(a);
    if (st != ATTN_OK) return st;
    if (num_splits < 1 || num_splits > 65535) return ATTN_ERR_INVALID_ARG;
    if (a->B * a->Hq * a->Lq > 0) {
        if (o_part == nullptr || m_part == nullptr || l_part == nullptr) return ATTN_ERR_INVALID_ARG;
        if (!aligned(o_part, 16) || !aligned(m_part, 4) || !aligned(l_part, 4)) return ATTN_ERR_INVALID_ARG;
    }
    const int64_t G = a->Hq / a->Hkv;
    if (a->B * a->Hkv > 65535 || (G * a->Lq + 31) / 32 > 65535) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

attn_status attn_fwd_prefill(const attn_fwd_args *a, void *stream) {
    attn_status st = attn_validate_prefill(a);
    if (st != ATTN_OK) return st;
    if (a->B * a->Hq * a->Lq == 0) return ATTN_OK;
    FwdParams p = make_params(a);
    if ((st = device_topology(p)) != ATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launch([&] { return a->dtype == ATTN_BF16 ? attn::launch_prefill_bf16(p, s) : attn::launch_rows_f32(p, 0, s); });
}

attn_status attn_fwd_decode_splitk(const attn_fwd_args *a, int32_t num_splits, float *o_part, float *m_part,
                                   float *l_part, void *stream) {
    attn_status st = attn_validate_decode(a, num_splits, o_part, m_part, l_part);
    if (st != ATTN_OK) return st;
    if (a->B * a->Hq * a->Lq == 0) return ATTN_OK;
    FwdParams p = make_params(a);
    p.num_splits = num_splits;
    p.chunk = chunk_len(a->Lk, num_splits);
    p.o_part = o_part;
    p.m_part = m_part;
    p.l_part = l_part;
    if ((st = device_topology(p)) != ATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launch([&] { return a->dtype == ATTN_BF16 ? attn::launch_decode_bf16(p, s) : attn::launch_rows_f32(p, 1, s); });
}

attn_status attn_fwd_prefill_splitk(const attn_fwd_args *a, int32_t num_splits, float *o_part, float *m_part,
                                    float *l_part, void *stream) {
    attn_status st = check_common(a);   // o, o_strides and lse are not used
    if (st != ATTN_OK) return st;
    if (num_splits < 1 || num_splits > 65535) return ATTN_ERR_INVALID_ARG;
    if (a->B * a->Hq * a->Lq > 0) {
        if (o_part == nullptr || m_part == nullptr || l_part == nullptr) return ATTN_ERR_INVALID_ARG;
        if (!aligned(o_part, 16) || !aligned(m_part, 4) || !aligned(l_part, 4)) return ATTN_ERR_INVALID_ARG;
    }
    if (a->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (a->B * a->Hq * a->Lq == 0) return ATTN_OK;
    const int64_t chunk = prefill_chunk_len(a->Lk, num_splits);
    if (chunk > kIntMax) return ATTN_ERR_UNSUPPORTED;   // the kernel holds key positions in 32 bits
    FwdParams p = make_params(a);
    p.num_splits = num_splits;
    p.chunk = (int)chunk;
    p.o_part = o_part;
    p.m_part = m_part;
    p.l_part = l_part;
    if ((st = device_topology(p)) != ATTN_OK) return st;
    return launch([&] { return attn::launch_prefill_part_bf16(p, static_cast<hipStream_t>(stream)); });
}

int32_t attn_prefill_choose_splits(int64_t B, int64_t Hq, int64_t Lq, int64_t Lk, int32_t cu_count) {
    if (B < 1 || Hq < 1 || Lq < 1 || Lk < 1) return 1;
    const int64_t cu = cu_count > 0 ? cu_count : 256;
    const int64_t blocks = sat_mul(sat_mul(B, Hq), ceil_div(Lq, 128));
    int64_t S = ceil_div(kPrefillSplitSlots * cu, blocks);
    const int64_t max_by_len = Lk / kPrefillSplitMinKeys;
    if (S > max_by_len) S = max_by_len;
    if (S > 65535) S = 65535;
    if (S < 2) return 1;
    if (blocks >= cu && prefill_chunk_len(Lk, (int32_t)S) < kPrefillSplitLongChunk) return 1;
    return (int32_t)S;
}

attn_status attn_splitk_combine(const float *o_part, const float *m_part, const float *l_part, int64_t B,
                                int64_t Hq, int64_t Lq, int64_t D, int32_t num_splits, void *o, int32_t o_dtype,
                                const int64_t o_strides[3], float *lse, void *stream) {
    if (B < 0 || Hq < 1 || Lq < 0 || D < 1 || num_splits < 1 || num_splits > 65535) return ATTN_ERR_INVALID_ARG;
    if (!valid_dtype(o_dtype) || o_strides == nullptr) return ATTN_ERR_INVALID_ARG;
    for (int t = 0; t < 3; ++t)
        if (o_strides[t] < 0) return ATTN_ERR_INVALID_ARG;
    int64_t rows = 0;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (!mul3(B, Hq, Lq, rows) || rows > kIntMax / 4) return ATTN_ERR_UNSUPPORTED;
    if (rows == 0) return ATTN_OK;
    if (o_part == nullptr || m_part == nullptr || l_part == nullptr || o == nullptr) return ATTN_ERR_INVALID_ARG;
    if (!aligned(o_part, 4) || !aligned(m_part, 4) || !aligned(l_part, 4) || !aligned(o, (uintptr_t)elem_size(o_dtype)))
        return ATTN_ERR_INVALID_ARG;
    if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_INVALID_ARG;
    attn::CombineParams c{};
    c.o_part = o_part; c.m_part = m_part; c.l_part = l_part;
    c.o = o; c.o_sb = o_strides[0]; c.o_sh = o_strides[1]; c.o_sl = o_strides[2];
    c.lse = lse;
    c.B = (int)B; c.Hq = (int)Hq; c.Lq = (int)Lq; c.D = (int)D; c.S = num_splits;
    c.o_bf16 = o_dtype == ATTN_BF16;
    return launch([&] { return attn::launch_combine(c, static_cast<hipStream_t>(stream)); });
}

int32_t attn_decode_choose_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int32_t cu_count) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Hq % Hkv != 0 || Lk <= 256) return 1;
    const int64_t cu = cu_count > 0 ? cu_count : 256;
    const int64_t rblocks = (sat_mul(Hq / Hkv, Lq) - 1) / 32 + 1;
    const int64_t units = sat_mul(sat_mul(B, Hkv), rblocks);
    const int64_t target = cu;                   // one workgroup per compute unit (the decode
                                                 // kernel's LDS stages hold one per CU at D = 128)
    int64_t S = ceil_div(target, units);
    const int64_t max_by_len = Lk / 256;         // at least 256 keys per chunk
    if (S > max_by_len) S = max_by_len;
    if (S > 65535) S = 65535;
    if (S < 1) S = 1;
    return (int32_t)S;
}

size_t attn_decode_partial_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int32_t num_splits) {
    if (B < 0 || Hq < 0 || Lq < 0 || D < 0 || num_splits < 1) return 0;
    size_t rows, bytes;
    if (__builtin_mul_overflow((size_t)B, (size_t)Hq, &rows) || __builtin_mul_overflow(rows, (size_t)Lq, &rows) ||
        __builtin_mul_overflow(rows, (size_t)num_splits, &rows) ||
        __builtin_mul_overflow(rows, ((size_t)D + 2) * sizeof(float), &bytes))
        return 0;
    return bytes;
}

int32_t attn_device_cu_count(int32_t device) {
    static std::atomic<int32_t> cache[64];
    if (device < 0) return -1;
    if (device < 64) {
        const int32_t c = cache[device].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return -1;
    if (device < 64) cache[device].store(v, std::memory_order_relaxed);
    return v;
}

int32_t attn_device_xcd_count(int32_t device) {
    static std::atomic<int32_t> cache[64];
    if (device < 0) return -1;
    if (device < 64) {
        const int32_t c = cache[device].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, device) != hipSuccess) return -1;
    if (v < 1) v = 1;
    if (device < 64) cache[device].store(v, std::memory_order_relaxed);
    return v;
}

size_t attn_fwd_args_size(void) { return sizeof(attn_fwd_args); }

size_t attn_bwd_args_size(void) { return sizeof(attn_bwd_args); }

size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq) {
    int64_t rows = 0;
    if (B < 0 || Hq < 0 || Lq < 0 || !mul3(B, Hq, Lq, rows) || rows > INT64_MAX / 16) return 0;
    return 2 * (size_t)bwd_rows_padded(rows) * sizeof(float);
}

attn_status attn_validate_bwd(const attn_bwd_args *a) {
    if (a == nullptr) return ATTN_ERR_INVALID_ARG;
    const attn_fwd_args *f = &a->fwd;
    attn_status st = check_common(f);
    if (st != ATTN_OK) return st;
    if (!valid_dtype(f->o_dtype) || !valid_dtype(a->grad_dtype) || a->reserved != 0) return ATTN_ERR_INVALID_ARG;
    for (int t = 0; t < 3; ++t)
        if (f->o_strides[t] < 0 || a->dout_strides[t] < 0 || a->dq_strides[t] < 0 || a->dk_strides[t] < 0 ||
            a->dv_strides[t] < 0)
            return ATTN_ERR_INVALID_ARG;
    const bool any_q = f->B * f->Hq * f->Lq > 0;
    const bool any_kv = f->B * f->Hkv * f->Lk > 0;
    if (any_q && (f->o == nullptr || f->lse == nullptr || a->dout == nullptr || a->dq == nullptr ||
                  a->workspace == nullptr))
        return ATTN_ERR_INVALID_ARG;
    if (any_kv && (a->dk == nullptr || a->dv == nullptr)) return ATTN_ERR_INVALID_ARG;
    if (f->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    // one-dimensional grids of 128-row (query or key) tiles
    if (f->B * f->Hq * ((f->Lq + 127) / 128) > kIntMax || f->B * f->Hkv * ((f->Lk + 127) / 128) > kIntMax)
        return ATTN_ERR_UNSUPPORTED;
    // 16-byte rows of o, dout and the gradients; 4-byte lse; 16-byte workspace
    const int64_t ov = 16 / elem_size(f->o_dtype), gv = 16 / elem_size(a->grad_dtype), dv = 16 / elem_size(f->dtype);
    if (any_q) {
        if (!aligned(f->o, 16) || !aligned(a->dout, 16) || !aligned(a->dq, 16)) return ATTN_ERR_UNSUPPORTED;
        if (!aligned(f->lse, 4) || !aligned(a->workspace, 16)) return ATTN_ERR_INVALID_ARG;
        for (int t = 0; t < 3; ++t)
            if (f->o_strides[t] % ov || a->dout_strides[t] % dv || a->dq_strides[t] % gv) return ATTN_ERR_UNSUPPORTED;
        if (a->dout_strides[2] > (1 << 24) || f->q_strides[2] > (1 << 24)) return ATTN_ERR_UNSUPPORTED;
    }
    if (any_kv) {
        if (!aligned(a->dk, 16) || !aligned(a->dv, 16)) return ATTN_ERR_UNSUPPORTED;
        for (int t = 0; t < 3; ++t)
            if (a->dk_strides[t] % gv || a->dv_strides[t] % gv) return ATTN_ERR_UNSUPPORTED;
    }
    return ATTN_OK;
}

attn_status attn_fwd_choose_plan(const attn_fwd_args *a, int32_t cu_count, attn_fwd_plan *plan) {
    if (plan == nullptr) return ATTN_ERR_INVALID_ARG;
    attn_status st = attn_validate_prefill(a);
    if (st != ATTN_OK) return st;
    const int64_t cu = cu_count > 0 ? cu_count : 256;
    const int64_t G = a->Hq / a->Hkv;
    const int64_t rblocks = (G * a->Lq + 31) / 32;
    const int64_t R = a->B * a->Hkv * rblocks;
    plan->method = ATTN_PLAN_PREFILL;
    plan->num_splits = 0;
    plan->workspace_bytes = 0;
    if (a->dtype != ATTN_BF16 || a->Lk <= 0 || R <= 0) return ATTN_OK;
    const bool splitk_fits = R <= cu && a->B * a->Hkv <= 65535 && rblocks <= 65535;
    const int32_t PS = a->Lq > kSplitKMaxLq || !splitk_fits
                           ? attn_prefill_choose_splits(a->B, a->Hq, a->Lq, a->Lk, (int32_t)cu)
                           : 1;
    if (PS >= 2) {
        plan->method = ATTN_PLAN_PREFILL_SPLIT;
        plan->num_splits = PS;
        plan->workspace_bytes = attn_decode_partial_bytes(a->B, a->Hq, a->Lq, a->D, PS);
    } else if (splitk_fits) {
        const int32_t S = attn_decode_choose_splits(a->B, a->Hq, a->Hkv, a->Lq, a->Lk, (int32_t)cu);
        plan->method = ATTN_PLAN_SPLITK;
        plan->num_splits = S;
        plan->workspace_bytes = attn_decode_partial_bytes(a->B, a->Hq, a->Lq, a->D, S);
    }
    return ATTN_OK;
}

attn_status attn_fwd(const attn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
    attn_status st = attn_validate_prefill(a);
    if (st != ATTN_OK) return st;
    if (a->B * a->Hq * a->Lq == 0) return ATTN_OK;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return ATTN_ERR_HIP;
    attn_fwd_plan plan;
    st = attn_fwd_choose_plan(a, attn_device_cu_count(device), &plan);
    if (st != ATTN_OK) return st;
    if (plan.method == ATTN_PLAN_PREFILL) return attn_fwd_prefill(a, stream);
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_INVALID_ARG;
    const int64_t parts = a->B * a->Hq * a->Lq * (int64_t)plan.num_splits;
    float *o_part = static_cast<float *>(workspace);
    float *m_part = o_part + parts * a->D;
    float *l_part = m_part + parts;
    st = plan.method == ATTN_PLAN_SPLITK ? attn_fwd_decode_splitk(a, plan.num_splits, o_part, m_part, l_part, stream)
                                         : attn_fwd_prefill_splitk(a, plan.num_splits, o_part, m_part, l_part, stream);
    if (st != ATTN_OK) return st;
    return attn_splitk_combine(o_part, m_part, l_part, a->B, a->Hq, a->Lq, a->D, plan.num_splits, a->o, a->o_dtype,
                               a->o_strides, a->lse, stream);
}

attn_status attn_bwd(const attn_bwd_args *a, void *stream) {
    attn_status st = attn_validate_bwd(a);
    if (st != ATTN_OK) return st;
    const attn_fwd_args *f = &a->fwd;
    if (f->B * f->Hq * f->Lq == 0 && f->B * f->Hkv * f->Lk == 0) return ATTN_OK;
    attn::BwdParams p{};
    p.f = make_params(f);
    p.dout = a->dout;
    p.do_sb = a->dout_strides[0]; p.do_sh = a->dout_strides[1]; p.do_sl = a->dout_strides[2];
    p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
    p.dq_sb = a->dq_strides[0]; p.dq_sh = a->dq_strides[1]; p.dq_sl = a->dq_strides[2];
    p.dk_sb = a->dk_strides[0]; p.dk_sh = a->dk_strides[1]; p.dk_sl = a->dk_strides[2];
    p.dv_sb = a->dv_strides[0]; p.dv_sh = a->dv_strides[1]; p.dv_sl = a->dv_strides[2];
    p.delta = a->workspace;
    p.lse_l2 = a->workspace + bwd_rows_padded(f->B * f->Hq * f->Lq);
    p.grad_bf16 = a->grad_dtype == ATTN_BF16;
    if ((st = device_topology(p.f)) != ATTN_OK) return st;
    return launch([&] { return attn::launch_bwd_bf16(p, static_cast<hipStream_t>(stream)); });
}

const char *attn_status_str(attn_status s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID_ARG: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_WORKSPACE: return "workspace too small";
        case ATTN_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

}  // extern "C"
