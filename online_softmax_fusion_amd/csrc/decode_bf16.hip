// decode_bf16.hip -- local step of the split-K update for bf16 K/V on gfx950.
//
// "Neptune论文浅读" section 6: the key dimension is cut into chunks, each chunk
// is reduced independently (its own max, sum and output), and a global step
// repairs and merges the chunks (combine.hip).  This kernel is the local step.
//
// Grid: (chunk s, b * Hkv + hk, 32-row block).  The G = Hq / Hkv query heads
// of one K/V group, times the Lq query rows, are stacked as the rows of one
// matrix-core tile, so every K/V element is fetched from HBM once per group
// instead of once per query head (the GQA grouping of the CMU 15-779 Lecture 11
// Mirage notes, section 7.1).  The chunk's keys are dealt to the NW waves of
// the workgroup in 32-key blocks; each wave runs the rolling update over its
// blocks:
//   * K of a block goes straight from global memory into matrix-core A
//     operands (no LDS): lane l loads key perm32(l % 32) so that the scores
//     land in the layout the P V product consumes.
//   * V of a block is transposed through a small wave-private LDS slice (the
//     matrix core wants 8 consecutive keys of one d per lane).
//   * loads of block n+1 are issued before the arithmetic of block n.
// At the end the NW waves' (m, l, O) are merged in LDS (repair by 2^(m_w - M))
// and the chunk's un-normalised o, its reference m (natural-log units) and l
// are written to the partial buffers.  Decode is HBM-bound: the matrix cores
// are mostly idle, the design goal is bytes in flight.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

template <int D, int NW, int BIAS>
__global__ __launch_bounds__(NW * 64, 2) void decode_bf16_kernel(FwdParams p) {
    constexpr int KS = D / 16;          // k-steps of K Q^T
    constexpr int DB = D / 32;          // 32-row blocks of O^T
    constexpr int VSTR = 32 + 8;        // LDS row stride of a wave's V^T slice
    constexpr int NDC = D / 64;         // V d-chunks (of 8) per lane per key group
    constexpr int OSTR = D + 4;         // LDS row stride of the merge buffer (floats)

    __shared__ __attribute__((aligned(16))) uint16_t lds_v[NW][D * VSTR];
    __shared__ __attribute__((aligned(16))) float lds_o[32 * OSTR];
    __shared__ float lds_m[NW][32];
    __shared__ float lds_l[32];

    const int s = blockIdx.x;
    const int bhk = blockIdx.y;
    const int rb = blockIdx.z;
    const int b = bhk / p.Hkv;
    const int hk = bhk - b * p.Hkv;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r = lane & 31;
    const int hh = lane >> 5;
    const int off = p.Lk - p.Lq;

    // this lane's stacked row: group member g, query row i
    const int nrows = p.G * p.Lq;
    const int rho = rb * 32 + r;
    const bool row_ok = rho < nrows;
    const int rho_c = row_ok ? rho : 0;
    const int g = rho_c / p.Lq;
    const int qi = rho_c - g * p.Lq;
    const int h = hk * p.G + g;
    const int qpos = qi + off;

    const int k_lo = s * p.chunk;
    const int k_hi = min(k_lo + p.chunk, p.Lk);
    const int nblk = (k_hi > k_lo) ? (k_hi - k_lo + 31) / 32 : 0;

    const uint16_t *kp = static_cast<const uint16_t *>(p.k) + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vp = static_cast<const uint16_t *>(p.v) + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;

    u32x4 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = u32x4{0, 0, 0, 0};
    if (row_ok) {
        const uint16_t *qr = static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb +
                             (int64_t)h * p.q_sh + (int64_t)qi * p.q_sl + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = load16(qr + ks * 16);
    }
    float slope_l2 = 0.f;
    if (BIAS == kBiasAlibi) slope_l2 = p.slopes[h] * kLog2e;

    // V unit of this lane inside a 32-key block: keys 4*v_kg .. +3, d-chunks v_dg + 8*c
    const int v_kg = lane & 7;
    const int v_dg = lane >> 3;
    uint16_t *vslice = lds_v[wave];

    u32x4 kc[KS], kn[KS];
    u32x4 vc[4 * NDC], vn[4 * NDC];

    auto load_block = [&](int kb0, u32x4 (&kd)[KS], u32x4 (&vd)[4 * NDC]) {
        const int jk = kb0 + perm32(r);
        const bool kok = jk < k_hi;
        const uint16_t *kr = kp + (int64_t)(kok ? jk : k_lo) * p.k_sl + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kd[ks] = kok ? load16(kr + ks * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int jv = kb0 + v_kg * 4 + u;
            const bool vok = jv < k_hi;
            const uint16_t *vr = vp + (int64_t)(vok ? jv : k_lo) * p.v_sl;
#pragma unroll
            for (int c = 0; c < NDC; ++c)
                vd[u * NDC + c] = vok ? load16(vr + (v_dg + 8 * c) * 8) : u32x4{0, 0, 0, 0};
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    int it = wave;
    if (it < nblk) load_block(k_lo + it * 32, kc, vc);
    for (; it < nblk; it += NW) {
        const int kb0 = k_lo + it * 32;
        const bool more = it + NW < nblk;
        if (more) load_block(kb0 + NW * 32, kn, vn);

        // V^T of the current block into this wave's LDS slice
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                const bool odd = e & 1;
                const uint32_t x0 = vc[0 * NDC + c][w], x1 = vc[1 * NDC + c][w];
                const uint32_t x2 = vc[2 * NDC + c][w], x3 = vc[3 * NDC + c][w];
                const uint32_t lo = odd ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
                const uint32_t hi = odd ? ((x2 >> 16) | (x3 & 0xffff0000u)) : ((x2 & 0xffffu) | (x3 << 16));
                const int d = (v_dg + 8 * c) * 8 + e;
                *reinterpret_cast<u32x2 *>(&vslice[d * VSTR + v_kg * 4]) = u32x2{lo, hi};
            }
        }

        // S^T = K Q^T for 32 keys
        f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma32(as_bf16x8(kc[ks]), as_bf16x8(qreg[ks]), sacc);

        const bool need_mask = (kb0 + 32 > k_hi) || p.causal;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = kb0 + (e >> 3) * 16 + hh * 8 + (e & 7);
            float x = sacc[e] * p.scale_log2;
            if (BIAS == kBiasAlibi) {
                x -= slope_l2 * fabsf((float)(qpos - j));
            } else if (BIAS == kBiasDenseF32 || BIAS == kBiasDenseBf16) {
                const int bj = min(j, p.Lk - 1);
                const int64_t idx = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh +
                                    (int64_t)qi * p.bias_si + (int64_t)bj * p.bias_sj;
                float bv;
                if (BIAS == kBiasDenseF32)
                    bv = static_cast<const float *>(p.bias)[idx];
                else
                    bv = bf16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[idx]);
                x = fmaf(bv, kLog2e, x);
            }
            if (need_mask && (j >= k_hi || (p.causal && j > qpos))) x = -INFINITY;
            sacc[e] = x;
            mx = fmaxf(mx, x);
        }
        mx = xor32_max(mx);
        const float m_new = fmaxf(m_run, mx);
        if (m_new > m_run) {
            const float alpha = exp2_fast(m_run - m_new);   // m_run = -inf gives 0
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        uint32_t pk[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const float p0 = exp2_fast(sacc[e] - m_use);
            const float p1 = exp2_fast(sacc[e + 1] - m_use);
            l_run += p0 + p1;
            pk[e >> 1] = pack_bf16x2(p0, p1);
        }
        // O^T += V^T P^T over two 16-key halves
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const bf16x8 bop = as_bf16x8(u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t *vr = &vslice[(db * 32 + r) * VSTR + half * 16 + hh * 8];
                oacc[db] = mfma32(as_bf16x8(load16(vr)), bop, oacc[db]);
            }
        }
        if (more) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kc[ks] = kn[ks];
#pragma unroll
            for (int u = 0; u < 4 * NDC; ++u) vc[u] = vn[u];
        }
    }

    // merge the waves of the workgroup: M = max_w m_w, repair each by 2^(m_w - M)
    const float l_wave = xor32_sum(l_run);
    if (hh == 0) lds_m[wave][r] = m_run;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_m[w][r]);
    const float alpha = (M == -INFINITY) ? 0.f : exp2_fast(m_run - M);
    for (int w = 0; w < NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float *dst = &lds_o[r * OSTR + db * 32 + i * 8 + hh * 4];
                    f32x4 v4 = f32x4{oacc[db][4 * i] * alpha, oacc[db][4 * i + 1] * alpha,
                                     oacc[db][4 * i + 2] * alpha, oacc[db][4 * i + 3] * alpha};
                    if (w > 0) v4 += *reinterpret_cast<f32x4 *>(dst);
                    *reinterpret_cast<f32x4 *>(dst) = v4;
                }
            }
            if (hh == 0) lds_l[r] = (w > 0 ? lds_l[r] : 0.f) + l_wave * alpha;
        }
        __syncthreads();
    }

    // write the chunk's partial for every valid stacked row
    constexpr int T = NW * 64;
    for (int c = tid; c < 32 * (D / 4); c += T) {
        const int rr = c / (D / 4);
        const int d4 = c - rr * (D / 4);
        const int rho2 = rb * 32 + rr;
        if (rho2 >= nrows) continue;
        const int g2 = rho2 / p.Lq;
        const int i2 = rho2 - g2 * p.Lq;
        const int h2 = hk * p.G + g2;
        const int64_t R = ((int64_t)b * p.Hq + h2) * p.Lq + i2;
        float *dst = p.o_part + (R * p.num_splits + s) * D + d4 * 4;
        *reinterpret_cast<f32x4 *>(dst) = *reinterpret_cast<const f32x4 *>(&lds_o[rr * OSTR + d4 * 4]);
        if (d4 == 0) {
            float Mr = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) Mr = fmaxf(Mr, lds_m[w][rr]);
            p.m_part[R * p.num_splits + s] = (Mr == -INFINITY) ? -INFINITY : Mr * kLn2;
            p.l_part[R * p.num_splits + s] = lds_l[rr];
        }
    }
}

template <int D, int BIAS>
hipError_t launch_decode_t(const FwdParams &p, hipStream_t stream) {
    constexpr int NW = 4;
    const int64_t rblocks = ((int64_t)p.G * p.Lq + 31) / 32;
    if (rblocks == 0 || p.B == 0) return hipSuccess;
    dim3 grid((unsigned)p.num_splits, (unsigned)(p.B * p.Hkv), (unsigned)rblocks), block(NW * 64);
    hipLaunchKernelGGL((decode_bf16_kernel<D, NW, BIAS>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const FwdParams &p, hipStream_t stream) {
    switch (p.bias_kind) {
        case kBiasNone: return launch_decode_t<D, kBiasNone>(p, stream);
        case kBiasAlibi: return launch_decode_t<D, kBiasAlibi>(p, stream);
        case kBiasDenseF32: return launch_decode_t<D, kBiasDenseF32>(p, stream);
        case kBiasDenseBf16: return launch_decode_t<D, kBiasDenseBf16>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_bf16(const FwdParams &p, hipStream_t stream) {
    if (p.D == 128) return launch_decode_d<128>(p, stream);
    if (p.D == 64) return launch_decode_d<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
