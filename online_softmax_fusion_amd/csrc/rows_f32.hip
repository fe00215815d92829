// rows_f32.hip -- attention forward for fp32 Q/K/V on gfx950 (vector ALU).
//
// fp32 inputs are kept in fp32 end to end (no bf16 rounding of Q, K, V or P),
// so this path uses the vector units rather than the bf16 matrix cores.  One
// wavefront owns one query row (grid x) and one key range (grid y: the whole
// key axis for prefill, one chunk for split-K decode).  It runs the online
// softmax of "Neptune论文浅读" section 3 over blocks of 64 keys:
//   lane j scores key j of the block (q in LDS, k row from global memory),
//   block max and sum by wave reductions, the running sum and the output
//   repaired by exp(m_old - m_new) (section 4), then every lane adds the
//   block's weighted values for its own d columns.
// Prefill writes O = o / l and LSE = m + ln l; decode writes the chunk's
// un-normalised o, its m and l (section 6).  Scores use expf (natural base).
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int D, int BIAS, bool PARTIAL>
__global__ __launch_bounds__(64) void rows_f32_kernel(FwdParams p) {
    constexpr int DPL = D / 64;   // d columns per lane
    __shared__ __attribute__((aligned(16))) float qs[D];
    __shared__ float ps[64];

    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;           // (b * Hq + h) * Lq + i
    const int s = blockIdx.y;
    const int i = (int)(row % p.Lq);
    const int64_t bh = row / p.Lq;
    const int h = (int)(bh % p.Hq);
    const int b = (int)(bh / p.Hq);
    const int hk = h / p.G;
    const int qpos = i + (p.Lk - p.Lq);

    int k_lo = 0, k_hi = p.Lk;
    if (PARTIAL) {
        k_lo = s * p.chunk;
        k_hi = min(k_lo + p.chunk, p.Lk);
    }
    int jmin, jmax;   // causal and window bounds
    key_range(p, qpos, jmin, jmax);
    k_lo = max(k_lo, jmin);
    k_hi = min(k_hi, jmax + 1);

    const float *qr = static_cast<const float *>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)i * p.q_sl;
    const float *kp = static_cast<const float *>(p.k) + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const float *vp = static_cast<const float *>(p.v) + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
    for (int d = lane; d < D; d += 64) qs[d] = qr[d];
    __syncthreads();

    float slope = 0.f;
    if (BIAS == kBiasAlibi) slope = p.slopes[h];

    float m = -INFINITY, l = 0.f;
    float o[DPL];
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[c] = 0.f;

    for (int kb = k_lo; kb < k_hi; kb += 64) {
        const int j = kb + lane;
        float x = -INFINITY;
        if (j < k_hi) {
            const float *kr = kp + (int64_t)j * p.k_sl;
            float dot = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; d += 4) {
                const f32x4 kv = *reinterpret_cast<const f32x4 *>(kr + d);
                const f32x4 qv = *reinterpret_cast<const f32x4 *>(&qs[d]);
                dot = fmaf(qv[0], kv[0], dot);
                dot = fmaf(qv[1], kv[1], dot);
                dot = fmaf(qv[2], kv[2], dot);
                dot = fmaf(qv[3], kv[3], dot);
            }
            x = dot * p.scale;
            if (p.softcap > 0.f) x = p.softcap * tanhf(x / p.softcap);
            if (BIAS == kBiasAlibi) {
                x -= slope * fabsf((float)(qpos - j));
            } else if (BIAS == kBiasDenseF32) {
                x += static_cast<const float *>(p.bias)[(int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh +
                                                         (int64_t)i * p.bias_si + (int64_t)j * p.bias_sj];
            } else if (BIAS == kBiasDenseBf16) {
                x += bf16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[(int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh +
                                                                            (int64_t)i * p.bias_si + (int64_t)j * p.bias_sj]);
            }
        }
        const float m_new = fmaxf(m, wave_max(x));
        const float alpha = (m_new == -INFINITY) ? 1.f : expf(m - m_new);
        const float pv = (x == -INFINITY) ? 0.f : expf(x - m_new);
        l = l * alpha + wave_sum(pv);
        ps[lane] = pv;
        __syncthreads();
        const int nk = min(64, k_hi - kb);
#pragma unroll
        for (int c = 0; c < DPL; ++c) o[c] *= alpha;
        for (int jj = 0; jj < nk; ++jj) {
            const float pj = ps[jj];
            const float *vr = vp + (int64_t)(kb + jj) * p.v_sl + lane;
#pragma unroll
            for (int c = 0; c < DPL; ++c) o[c] = fmaf(pj, vr[c * 64], o[c]);
        }
        m = m_new;
        __syncthreads();
    }

    if (PARTIAL) {
        const int64_t idx = row * p.num_splits + s;
        float *op = p.o_part + idx * D + lane;
#pragma unroll
        for (int c = 0; c < DPL; ++c) op[c * 64] = o[c];
        if (lane == 0) {
            p.m_part[idx] = m;
            p.l_part[idx] = l;
        }
    } else {
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
        const int64_t obase = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)i * p.o_sl + lane;
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
            const float val = o[c] * inv;
            if (p.o_bf16)
                static_cast<uint16_t *>(p.o)[obase + c * 64] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xffffu);
            else
                static_cast<float *>(p.o)[obase + c * 64] = val;
        }
        if (p.lse != nullptr && lane == 0) p.lse[row] = (l > 0.f) ? m + logf(l) : -INFINITY;
    }
}

template <int D, bool PARTIAL>
hipError_t launch_rows_t(const FwdParams &p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.B * p.Hq * p.Lq;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)rows, PARTIAL ? (unsigned)p.num_splits : 1u), block(64);
    // the soft cap is a run-time branch here (this path is not bound by the vector units)
    switch (bias_base(p.bias_kind)) {
        case kBiasNoneScaled:
        case kBiasNone: hipLaunchKernelGGL((rows_f32_kernel<D, kBiasNone, PARTIAL>), grid, block, 0, stream, p); break;
        case kBiasAlibi: hipLaunchKernelGGL((rows_f32_kernel<D, kBiasAlibi, PARTIAL>), grid, block, 0, stream, p); break;
        case kBiasDenseF32: hipLaunchKernelGGL((rows_f32_kernel<D, kBiasDenseF32, PARTIAL>), grid, block, 0, stream, p); break;
        case kBiasDenseBf16: hipLaunchKernelGGL((rows_f32_kernel<D, kBiasDenseBf16, PARTIAL>), grid, block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_f32(const FwdParams &p, int partial, hipStream_t stream) {
    if (p.D == 128) return partial ? launch_rows_t<128, true>(p, stream) : launch_rows_t<128, false>(p, stream);
    if (p.D == 64) return partial ? launch_rows_t<64, true>(p, stream) : launch_rows_t<64, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
