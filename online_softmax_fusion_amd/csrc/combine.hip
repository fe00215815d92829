// combine.hip -- global step of the split-K update on gfx950.
//
// "Neptune论文浅读" section 6: after the chunks have been reduced
// independently, each chunk's sum and output are repaired with the global max
// (the repair term of section 4, h(t, r, r') = t * exp(r - r')) and added up:
//     M = max_s m_s,  w_s = exp(m_s - M),  L = sum_s w_s l_s,
//     O = sum_s w_s o_s / L,  LSE = M + ln L.
// One workgroup of W waves per output row.  A lane owns a group of 4 d columns
// and a phase of the chunks (chunks ph, ph + P, ...); it folds its chunks in
// with the same rolling update the chunks were made with (a running max, and
// a repair of its partial sums when the max grows), so the m, l and o loads of
// a batch of chunks are all issued at once and there is no separate pass for
// the max.  The phases are then merged pairwise (repair to the larger max,
// add), first across lanes, then across the waves through LDS.  Chunks with
// m_s = -inf carry no key and get weight 0.  Every sum runs in a fixed order,
// so the result is bitwise reproducible.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

// partial state of a phase: running max M, repaired sum L and output acc
struct Part {
    float M, L;
    f32x4 acc;
};

// fold the state b into a (both repaired to the larger max)
__device__ __forceinline__ void merge(Part &a, const Part &b) {
    const float M = fmaxf(a.M, b.M);
    const float wa = (a.M == -INFINITY) ? 0.f : expf(a.M - M);
    const float wb = (b.M == -INFINITY) ? 0.f : expf(b.M - M);
    a.L = a.L * wa + b.L * wb;
    a.acc = a.acc * wa + b.acc * wb;
    a.M = M;
}

template <int D, int W>
__global__ __launch_bounds__(64 * W) void combine_kernel(CombineParams c) {
    constexpr int G4 = D / 4;         // float4 column groups
    constexpr int P = 64 * W / G4;    // chunk phases
    constexpr int NB = 8;             // chunks per lane whose loads are issued together
    __shared__ float lds_M[W], lds_L[W];
    __shared__ f32x4 lds_acc[W][G4];

    const int t = threadIdx.x;
    const int cg = t % G4;
    const int ph = t / G4;
    const int64_t row = blockIdx.x;
    const int S = c.S;
    const float *mrow = c.m_part + row * S;
    const float *lrow = c.l_part + row * S;
    const float *orow = c.o_part + row * S * D + cg * 4;

    Part st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = ph; s0 < S; s0 += NB * P) {
        float ms[NB], ls[NB];
        f32x4 ov[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int s = s0 + u * P;
            const bool ok = s < S;
            ms[u] = ok ? mrow[s] : -INFINITY;
            ls[u] = ok ? lrow[s] : 0.f;
            ov[u] = ok ? *reinterpret_cast<const f32x4 *>(orow + (int64_t)s * D) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (ms[u] == -INFINITY) continue;
            if (ms[u] > st.M) {
                const float a = (st.M == -INFINITY) ? 0.f : expf(st.M - ms[u]);
                st.L *= a;
                st.acc *= a;
                st.M = ms[u];
            }
            const float w = expf(ms[u] - st.M);
            st.L = fmaf(w, ls[u], st.L);
            st.acc += ov[u] * w;
        }
    }
    // merge the phases of this wave (lanes G4 apart share a column group)
#pragma unroll
    for (int o = G4; o < 64; o <<= 1) {
        Part other;
        other.M = __shfl_xor(st.M, o, 64);
        other.L = __shfl_xor(st.L, o, 64);
#pragma unroll
        for (int q = 0; q < 4; ++q) other.acc[q] = __shfl_xor(st.acc[q], o, 64);
        merge(st, other);
    }
    if (W > 1) {
        const int wave = t >> 6;
        if ((t & 63) < G4) {
            lds_acc[wave][cg] = st.acc;
            if (cg == 0) {
                lds_M[wave] = st.M;
                lds_L[wave] = st.L;
            }
        }
        __syncthreads();
        if (t >= G4) return;   // no barrier below
#pragma unroll
        for (int w = 1; w < W; ++w) merge(st, Part{lds_M[w], lds_L[w], lds_acc[w][cg]});
    } else if (t >= G4) {
        return;
    }

    const float inv = (st.L > 0.f) ? 1.f / st.L : 0.f;
    const int i = (int)(row % c.Lq);
    const int64_t bh = row / c.Lq;
    const int h = (int)(bh % c.Hq);
    const int b = (int)(bh / c.Hq);
    const int64_t obase = (int64_t)b * c.o_sb + (int64_t)h * c.o_sh + (int64_t)i * c.o_sl + cg * 4;
    const float o0 = st.acc[0] * inv, o1 = st.acc[1] * inv, o2 = st.acc[2] * inv, o3 = st.acc[3] * inv;
    if (c.o_bf16) {
        uint16_t *dst = static_cast<uint16_t *>(c.o) + obase;
        const uint32_t w0 = pack_bf16x2(o0, o1), w1 = pack_bf16x2(o2, o3);
        dst[0] = (uint16_t)(w0 & 0xffffu); dst[1] = (uint16_t)(w0 >> 16);
        dst[2] = (uint16_t)(w1 & 0xffffu); dst[3] = (uint16_t)(w1 >> 16);
    } else {
        float *dst = static_cast<float *>(c.o) + obase;
        dst[0] = o0; dst[1] = o1; dst[2] = o2; dst[3] = o3;
    }
    if (c.lse != nullptr && cg == 0) c.lse[row] = (st.L > 0.f) ? st.M + logf(st.L) : -INFINITY;
}

template <int D>
hipError_t launch_combine_d(const CombineParams &c, int64_t rows, hipStream_t stream) {
    // few rows: four waves per row, so that a row's chunks are read by more
    // lanes at once; many rows: one wave per row
    if (rows <= 2048)
        hipLaunchKernelGGL((combine_kernel<D, 4>), dim3((unsigned)rows), dim3(256), 0, stream, c);
    else
        hipLaunchKernelGGL((combine_kernel<D, 1>), dim3((unsigned)rows), dim3(64), 0, stream, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineParams &c, hipStream_t stream) {
    const int64_t rows = (int64_t)c.B * c.Hq * c.Lq;
    if (rows == 0) return hipSuccess;
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    if (c.D == 128) return launch_combine_d<128>(c, rows, stream);
    if (c.D == 64) return launch_combine_d<64>(c, rows, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
