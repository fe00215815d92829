// combine.hip -- global step of the split-K update on gfx950.
//
// "Neptune论文浅读" section 6: after the chunks have been reduced
// independently, each chunk's sum and output are repaired with the global max
// (the repair term of section 4, h(t, r, r') = t * exp(r - r')) and added up:
//     M = max_s m_s,  w_s = exp(m_s - M),  L = sum_s w_s l_s,
//     O = sum_s w_s o_s / L,  LSE = M + ln L.
// One wavefront per output row; lanes own groups of 4 d columns and a phase
// of the chunks, so all of a row's partial loads are issued together.  Chunks with m_s = -inf carry
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
    // one wavefront per row: lane = (phase, 4-column group); the phases split
    // the chunks so that every partial load of the row is in flight at once
    constexpr int G4 = D / 4;        // float4 column groups
    constexpr int P = 64 / G4;       // chunk phases
    const int lane = threadIdx.x & 63;
    const int cg = lane % G4;
    const int ph = lane / G4;
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

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != -INFINITY) {
        float lp = 0.f;
        for (int s = lane; s < S; s += 64) {
            const float ms = mrow[s];
            if (ms != -INFINITY) lp = fmaf(expf(ms - M), lrow[s], lp);
        }
        L = wave_sum64(lp);
#pragma unroll 4
        for (int s = ph; s < S; s += P) {
            const float ms = mrow[s];
            const f32x4 ov = *reinterpret_cast<const f32x4 *>(orow + (int64_t)s * D + cg * 4);
            const float w = (ms == -INFINITY) ? 0.f : expf(ms - M);
            acc[0] = fmaf(w, ov[0], acc[0]);
            acc[1] = fmaf(w, ov[1], acc[1]);
            acc[2] = fmaf(w, ov[2], acc[2]);
            acc[3] = fmaf(w, ov[3], acc[3]);
        }
    }
    // add the phases (lanes with the same column group)
#pragma unroll
    for (int o = G4; o < 64; o <<= 1)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += __shfl_xor(acc[q], o, 64);

    if (ph == 0) {
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        const int i = (int)(row % c.Lq);
        const int64_t bh = row / c.Lq;
        const int h = (int)(bh % c.Hq);
        const int b = (int)(bh / c.Hq);
        const int64_t obase = (int64_t)b * c.o_sb + (int64_t)h * c.o_sh + (int64_t)i * c.o_sl + cg * 4;
        const float o0 = acc[0] * inv, o1 = acc[1] * inv, o2 = acc[2] * inv, o3 = acc[3] * inv;
        if (c.o_bf16) {
            uint16_t *dst = static_cast<uint16_t *>(c.o) + obase;
            const uint32_t w0 = pack_bf16x2(o0, o1), w1 = pack_bf16x2(o2, o3);
            dst[0] = (uint16_t)(w0 & 0xffffu); dst[1] = (uint16_t)(w0 >> 16);
            dst[2] = (uint16_t)(w1 & 0xffffu); dst[3] = (uint16_t)(w1 >> 16);
        } else {
            float *dst = static_cast<float *>(c.o) + obase;
            dst[0] = o0; dst[1] = o1; dst[2] = o2; dst[3] = o3;
        }
        if (c.lse != nullptr && cg == 0) c.lse[row] = (L > 0.f) ? M + logf(L) : -INFINITY;
    }
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
