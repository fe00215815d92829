// combine.hip -- global step of the split-K update on gfx950.
//
// "Neptune论文浅读" section 6: after the chunks have been reduced
// independently, each chunk's sum and output are repaired with the global max
// (the repair term of section 4, h(t, r, r') = t * exp(r - r')) and added up:
//     M = max_s m_s,  w_s = exp(m_s - M),  L = sum_s w_s l_s,
//     O = sum_s w_s o_s / L,  LSE = M + ln L.
// One wavefront per output row; lanes own d columns, and stride over the
// chunks for the max and the weighted sum of l.  Chunks with m_s = -inf carry
// no key and get weight 0.  The sums run in a fixed order, so the result is
// bitwise reproducible.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams c) {
    constexpr int DPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t rows = (int64_t)c.B * c.Hq * c.Lq;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;   // whole wavefront leaves together; no barrier below
    const int S = c.S;
    const float *mrow = c.m_part + row * S;
    const float *lrow = c.l_part + row * S;
    const float *orow = c.o_part + row * S * D;

    float M = -INFINITY;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, mrow[s]);
    M = wave_max64(M);

    float o[DPL];
#pragma unroll
    for (int q = 0; q < DPL; ++q) o[q] = 0.f;
    float L = 0.f;
    if (M != -INFINITY) {
        float lp = 0.f;
        for (int s = lane; s < S; s += 64) {
            const float ms = mrow[s];
            if (ms != -INFINITY) lp = fmaf(expf(ms - M), lrow[s], lp);
        }
        L = wave_sum64(lp);
        for (int s = 0; s < S; ++s) {
            const float ms = mrow[s];
            if (ms == -INFINITY) continue;
            const float w = expf(ms - M);
#pragma unroll
            for (int q = 0; q < DPL; ++q) o[q] = fmaf(w, orow[(int64_t)s * D + lane + 64 * q], o[q]);
        }
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    const int i = (int)(row % c.Lq);
    const int64_t bh = row / c.Lq;
    const int h = (int)(bh % c.Hq);
    const int b = (int)(bh / c.Hq);
    const int64_t obase = (int64_t)b * c.o_sb + (int64_t)h * c.o_sh + (int64_t)i * c.o_sl + lane;
#pragma unroll
    for (int q = 0; q < DPL; ++q) {
        const float val = o[q] * inv;
        if (c.o_bf16)
            static_cast<uint16_t *>(c.o)[obase + 64 * q] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xffffu);
        else
            static_cast<float *>(c.o)[obase + 64 * q] = val;
    }
    if (c.lse != nullptr && lane == 0) c.lse[row] = (L > 0.f) ? M + logf(L) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineParams &c, hipStream_t stream) {
    const int64_t rows = (int64_t)c.B * c.Hq * c.Lq;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (c.D == 128)
        hipLaunchKernelGGL(combine_kernel<128>, grid, block, 0, stream, c);
    else if (c.D == 64)
        hipLaunchKernelGGL(combine_kernel<64>, grid, block, 0, stream, c);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
