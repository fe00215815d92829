// l2norm.hip -- numerically stable row-wise L2 norm on gfx950, in one pass
// (rolling update) or split over the row (split-K), with the repair algebra of
// "Neptune论文浅读" section 4 applied to the sum of squares.
//
// State of a partial reduction: a reference exponent e and s = sum (x * 2^-e)^2.
// Adding a 16-byte vector: if the vector's largest magnitude has an exponent
// more than kSlack above e, the reference moves up and s is repaired by
// 4^(e_old - e_new) (exact: a power of two); then s += (x * 2^-e)^2 for each
// element (v_ldexp_f32 and one FMA).  Merging two partials: e = max, each s
// repaired to it, added.  Because the scaling is by powers of two, no square
// overflows or underflows in fp32 for any finite input, and the result is as
// accurate as the unscaled sum.  The reference only moves when it must
// (values up to 2^kSlack times 2^e are taken as they are, their squares stay
// far below the fp32 range), so the common path has no compare-and-rescale
// per element.
//
// l2norm_onepass_kernel: one wave per row (four rows per workgroup); the row
// is loaded once into registers (NV 16-byte vectors per lane, consecutive
// lanes on consecutive vectors), reduced per lane, merged across the wave by
// xor shuffles, and written back scaled by 2^-e / sqrt(s).
// l2norm_partial_kernel / l2norm_scale_kernel: one workgroup per (row, chunk);
// the first writes (e, s) of its chunk, the second merges the row's partials
// and scales its chunk (the row is read twice).
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kNoExp = -100000;   // exponent of an empty partial (s = 0)
constexpr int kSlack = 30;        // values up to 2^(e + 30) are squared without moving e

struct Part {
    int e;
    float s;
};

__device__ __forceinline__ int exp_of(float a) { return __builtin_amdgcn_frexp_expf(a); }
__device__ __forceinline__ float scale2(float x, int k) { return __builtin_amdgcn_ldexpf(x, k); }

// 16 bytes of a row as floats
template <bool BF16>
struct Vec {
    static constexpr int N = BF16 ? 8 : 4;
    float v[N];
    __device__ __forceinline__ void load(const void *p) {
        const u32x4 w = load16(p);
        if (BF16) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v[2 * t] = bf16_bits_to_f32(w[t] & 0xffffu);
                v[2 * t + 1] = bf16_bits_to_f32(w[t] >> 16);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = __uint_as_float(w[t]);
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int t = 0; t < N; ++t) v[t] = 0.f;
    }
};

// the scaled values of input vector vi (8 or 4 floats times f * 2^-e) to row yr
// of the output: 16 bytes per vector for equal element types, 32 for bf16 ->
// fp32, 8 for fp32 -> bf16
template <bool XB, bool YB>
__device__ __forceinline__ void store_vec(char *yr, int vi, const float *v, int e, float f) {
    if (XB && YB) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(scale2(v[2 * t], -e) * f, scale2(v[2 * t + 1], -e) * f);
        store16(yr + (int64_t)vi * 16, u32x4{w[0], w[1], w[2], w[3]});
    } else if (XB && !YB) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            store16(yr + (int64_t)vi * 32 + 16 * h,
                    u32x4{__float_as_uint(scale2(v[4 * h], -e) * f), __float_as_uint(scale2(v[4 * h + 1], -e) * f),
                          __float_as_uint(scale2(v[4 * h + 2], -e) * f), __float_as_uint(scale2(v[4 * h + 3], -e) * f)});
    } else if (!XB && YB) {
        *reinterpret_cast<u32x2 *>(yr + (int64_t)vi * 8) =
            u32x2{pack_bf16x2(scale2(v[0], -e) * f, scale2(v[1], -e) * f),
                  pack_bf16x2(scale2(v[2], -e) * f, scale2(v[3], -e) * f)};
    } else {
        store16(yr + (int64_t)vi * 16, u32x4{__float_as_uint(scale2(v[0], -e) * f), __float_as_uint(scale2(v[1], -e) * f),
                                             __float_as_uint(scale2(v[2], -e) * f), __float_as_uint(scale2(v[3], -e) * f)});
    }
}

template <int N>
__device__ __forceinline__ void part_add(Part &a, const float (&v)[N]) {
    float mx = 0.f;
#pragma unroll
    for (int t = 0; t < N; ++t) mx = fmaxf(mx, fabsf(v[t]));
    if (mx > 0.f) {
        const int ev = exp_of(mx);
        if (ev > a.e + kSlack) {   // the reference must move up: repair the partial sum
            a.s = scale2(a.s, 2 * max(a.e - ev, -512));
            a.e = ev;
        }
    }
#pragma unroll
    for (int t = 0; t < N; ++t) {
        const float u = scale2(v[t], -a.e);
        a.s = fmaf(u, u, a.s);
    }
}

__device__ __forceinline__ Part part_merge(Part a, Part b) {
    const int e = max(a.e, b.e);
    return Part{e, scale2(a.s, 2 * max(a.e - e, -512)) + scale2(b.s, 2 * max(b.e - e, -512))};
}

__device__ __forceinline__ Part wave_merge(Part a) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Part o;
        o.e = __shfl_xor(a.e, m, 64);
        o.s = __shfl_xor(a.s, m, 64);
        a = part_merge(a, o);
    }
    return a;
}

// merge across the NW waves of a workgroup; every thread gets the result
template <int NW>
__device__ __forceinline__ Part block_merge(Part a, Part *lds, int wave, int lane) {
    a = wave_merge(a);
    if (lane == 0) lds[wave] = a;
    __syncthreads();
    Part r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = part_merge(r, lds[w]);
    __syncthreads();
    return r;
}

// norm and the factor 1/sqrt(s) applied after the 2^-e scaling
__device__ __forceinline__ void finish(const Part &a, float &norm, float &f) {
    if (a.s > 0.f) {
        const float r = sqrtf(a.s);
        norm = scale2(r, a.e);
        f = 1.f / r;
    } else {
        norm = 0.f;
        f = 0.f;
    }
}

template <bool XB, bool YB, int NV>
__global__ __launch_bounds__(256) void l2norm_onepass_kernel(L2Params p) {
    using V = Vec<XB>;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= p.rows) return;   // whole wave; no barrier in this kernel
    const int nvec = (int)(p.H / V::N);
    const char *xr = static_cast<const char *>(p.x) + row * p.x_stride * (XB ? 2 : 4);
    V v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vi = lane + 64 * i;
        if (vi < nvec)
            v[i].load(xr + (int64_t)vi * 16);
        else
            v[i].zero();
    }
    Part a{kNoExp, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) part_add(a, v[i].v);
    a = wave_merge(a);
    float norm, f;
    finish(a, norm, f);
    if (p.norm != nullptr && lane == 0) p.norm[row] = norm;
    if (p.y != nullptr) {
        char *yr = static_cast<char *>(p.y) + row * p.y_stride * (YB ? 2 : 4);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int vi = lane + 64 * i;
            if (vi < nvec) store_vec<XB, YB>(yr, vi, v[i].v, a.e, f);
        }
    }
}

// (e, s) of chunk c of row r: vectors [c * chunk, min((c + 1) * chunk, nvec))
template <bool XB>
__global__ __launch_bounds__(256) void l2norm_partial_kernel(L2Params p) {
    using V = Vec<XB>;
    __shared__ Part lds[4];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t r = blockIdx.x / p.S;
    const int c = (int)(blockIdx.x - r * p.S);
    const int nvec = (int)(p.H / V::N);
    const int v0 = c * p.chunk_vecs;
    const int v1 = min(v0 + p.chunk_vecs, nvec);
    const char *xr = static_cast<const char *>(p.x) + r * p.x_stride * (XB ? 2 : 4);
    Part a{kNoExp, 0.f};
    constexpr int U = 4;   // loads in flight per thread
    int vi = v0 + (int)threadIdx.x;
    for (; vi + 256 * (U - 1) < v1; vi += 256 * U) {
        V v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u].load(xr + (int64_t)(vi + 256 * u) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u) part_add(a, v[u].v);
    }
    for (; vi < v1; vi += 256) {
        V v;
        v.load(xr + (int64_t)vi * 16);
        part_add(a, v.v);
    }
    a = block_merge<4>(a, lds, wave, lane);
    if (threadIdx.x == 0) {
        int *w = reinterpret_cast<int *>(p.ws) + 2 * (r * p.S + c);
        w[0] = a.e;
        w[1] = __float_as_int(a.s);
    }
}

// merge row r's partials, write its norm (chunk 0), scale chunk c
template <bool XB, bool YB>
__global__ __launch_bounds__(256) void l2norm_scale_kernel(L2Params p) {
    using V = Vec<XB>;
    __shared__ Part lds[4];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t r = blockIdx.x / p.S;
    const int c = (int)(blockIdx.x - r * p.S);
    const int *pw = reinterpret_cast<const int *>(p.ws) + 2 * r * p.S;
    Part a{kNoExp, 0.f};
    for (int t = threadIdx.x; t < p.S; t += 256) a = part_merge(a, Part{pw[2 * t], __int_as_float(pw[2 * t + 1])});
    a = block_merge<4>(a, lds, wave, lane);
    float norm, f;
    finish(a, norm, f);
    if (c == 0 && threadIdx.x == 0 && p.norm != nullptr) p.norm[r] = norm;
    if (p.y == nullptr) return;
    const int nvec = (int)(p.H / V::N);
    const int v0 = c * p.chunk_vecs;
    const int v1 = min(v0 + p.chunk_vecs, nvec);
    const char *xr = static_cast<const char *>(p.x) + r * p.x_stride * (XB ? 2 : 4);
    char *yr = static_cast<char *>(p.y) + r * p.y_stride * (YB ? 2 : 4);
    for (int vi = v0 + (int)threadIdx.x; vi < v1; vi += 256) {
        V v;
        v.load(xr + (int64_t)vi * 16);
        store_vec<XB, YB>(yr, vi, v.v, a.e, f);
    }
}

template <bool XB, bool YB>
hipError_t launch_onepass_t(const L2Params &p, hipStream_t s) {
    const int nvec = (int)(p.H / (XB ? 8 : 4));
    const int per_lane = (nvec + 63) / 64;
    const dim3 grid((unsigned)((p.rows + 3) / 4)), block(256);
    if (per_lane <= 1) hipLaunchKernelGGL((l2norm_onepass_kernel<XB, YB, 1>), grid, block, 0, s, p);
    else if (per_lane <= 2) hipLaunchKernelGGL((l2norm_onepass_kernel<XB, YB, 2>), grid, block, 0, s, p);
    else if (per_lane <= 4) hipLaunchKernelGGL((l2norm_onepass_kernel<XB, YB, 4>), grid, block, 0, s, p);
    else if (per_lane <= 8) hipLaunchKernelGGL((l2norm_onepass_kernel<XB, YB, 8>), grid, block, 0, s, p);
    else if (per_lane <= 16) hipLaunchKernelGGL((l2norm_onepass_kernel<XB, YB, 16>), grid, block, 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool XB, bool YB>
hipError_t launch_split_t(const L2Params &p, hipStream_t s) {
    const dim3 grid((unsigned)(p.rows * p.S)), block(256);
    hipLaunchKernelGGL((l2norm_partial_kernel<XB>), grid, block, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((l2norm_scale_kernel<XB, YB>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_l2norm(const L2Params &p, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    if (p.S <= 1) {
        if (p.x_bf16) return p.y_bf16 ? launch_onepass_t<true, true>(p, s) : launch_onepass_t<true, false>(p, s);
        return p.y_bf16 ? launch_onepass_t<false, true>(p, s) : launch_onepass_t<false, false>(p, s);
    }
    if (p.x_bf16) return p.y_bf16 ? launch_split_t<true, true>(p, s) : launch_split_t<true, false>(p, s);
    return p.y_bf16 ? launch_split_t<false, true>(p, s) : launch_split_t<false, false>(p, s);
}

}  // namespace attn
