// prefill_bf16.hip -- fused attention forward for bf16 Q/K/V on gfx950.
//
// One workgroup owns a tile of BR = 32 * NW query rows of one (b, h) and
// rolls over the keys in tiles of BC = 64 (the rolling update of
// "Neptune论文浅读" section 5; the same three-level loop as the kernel in the
// CANN FlashAttention post: query tile outside, K/V tiles inside, on-chip
// compute innermost).  Per K/V tile and per wave (32 query rows):
//
//   1. S^T = K Q^T on the matrix cores (32x32x16 bf16, fp32 accumulate).  Q
//      stays in registers for the whole loop; K comes from LDS.  Keys are
//      placed in the matrix-core rows with the perm32 shuffle so that each lane
//      ends up holding 32 scores of ONE query row (its column), in exactly the
//      order the P V product wants them.
//   2. score modifier in the log2 domain: t = s * scale * log2(e) + bias *
//      log2(e); the causal mask and the key tail are applied only on tiles that
//      cross them.
//   3. rolling update (Neptune notes section 3 and section 4): the row max
//      over the tile needs one cross-half swap (v_permlane32_swap); when the
//      max grows, the running sum and the output are repaired by
//      2^(m_old - m_new).  The repair is taken lazily: it runs only when some
//      row's max has grown by more than TAU = 8 (a factor 256), which keeps
//      every exponent <= 2^8 and is exact in real arithmetic because the final
//      normalisation uses the same reference m.
//   4. P = 2^(t - m) in fp32; the row sum l accumulates the fp32 values (each
//      lane keeps a partial over its half of the keys; the halves are added
//      once at the end); P is packed to bf16 in registers.
//   5. O^T += V^T P^T on the matrix cores, V^T read from LDS (V is transposed
//      on its way into LDS), P^T straight from registers.  Each lane's output
//      accumulators all belong to its own query row, so the repair in step 3
//      is lane-local.
//
// K/V tiles are double-buffered: the global loads for tile t+1 are issued
// before the matrix work on tile t and written to the other LDS buffer after
// it (the DMA/compute overlap described in the CANN post), one barrier per
// tile.  Causal tiles above the diagonal are never loaded; a wave whose rows
// are all above a tile's keys skips its matrix work.  Epilogue: O = O / l,
// LSE = m ln 2 + ln l; a row with no visible key gets O = 0, LSE = -inf.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr float kTau = 8.0f;

template <int D, int NW, int BIAS, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64, 2) void prefill_bf16_kernel(FwdParams p) {
    constexpr int BR = 32 * NW;      // query rows per workgroup
    constexpr int BC = 64;           // keys per tile
    constexpr int T = NW * 64;       // threads
    constexpr int KSTR = D + 8;      // LDS row stride of the K tile (elements)
    constexpr int VSTR = BC + 8;     // LDS row stride of the V^T tile (elements)
    constexpr int KS = D / 16;       // k-steps of Q K^T
    constexpr int DB = D / 32;       // 32-row blocks of O^T
    constexpr int NK = BC * D / 8 / T;   // 16-byte K chunks per thread per tile
    constexpr int KU = NK;               // keys per V transpose unit
    static_assert(NK >= 1 && BC * D / 8 == NK * T, "tile does not split evenly");
    static_assert(KU == 1 || KU == 2 || KU == 4 || KU == 8, "unsupported V unit");

    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][BC * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][D * VSTR];

    const int BH = p.B * p.Hq;
    const int nqt = (p.Lq + BR - 1) / BR;
    int qt = blockIdx.x / BH;
    const int bh = blockIdx.x - qt * BH;
    if (p.causal) qt = nqt - 1 - qt;  // heaviest query tiles first
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    const int hk = h / p.G;
    const int q0 = qt * BR;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r = lane & 31;
    const int hh = lane >> 5;
    const int off = p.Lk - p.Lq;
    const int qrow = q0 + wave * 32 + r;
    const int wrow0 = q0 + wave * 32;
    const int wrow1 = min(wrow0 + 31, p.Lq - 1);

    int kv_end = p.Lk;
    if (p.causal) kv_end = min(p.Lk, min(q0 + BR, p.Lq) + off);
    if (kv_end < 0) kv_end = 0;
    const int ntiles = (kv_end + BC - 1) / BC;

    const uint16_t *qp = static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    const uint16_t *kp = static_cast<const uint16_t *>(p.k) + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vp = static_cast<const uint16_t *>(p.v) + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;

    // Q fragment: lane holds row qrow, d = 16*ks + 8*hh .. +7 for each k-step.
    u32x4 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = u32x4{0, 0, 0, 0};
    if (qrow < p.Lq) {
        const uint16_t *qr = qp + (int64_t)qrow * p.q_sl + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = load16(qr + ks * 16);
    }

    float slope_l2 = 0.f;
    if (BIAS == kBiasAlibi) slope_l2 = p.slopes[h] * kLog2e;

    // staging registers for the next tile
    u32x4 kst[NK];
    u32x4 vst[KU];
    const int v_kg = tid % (BC / KU);   // V unit: keys KU*v_kg .. +KU-1
    const int v_dc = tid / (BC / KU);   //         d = 8*v_dc .. +7

    auto load_tile = [&](int t) {
        const int kbase = t * BC;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = tid + i * T;
            const int key = c / (D / 8);
            const int dc = c - key * (D / 8);
            const int j = kbase + key;
            kst[i] = (j < p.Lk) ? load16(kp + (int64_t)j * p.k_sl + dc * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int j = kbase + v_kg * KU + u;
            vst[u] = (j < p.Lk) ? load16(vp + (int64_t)j * p.v_sl + v_dc * 8) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int c = tid + i * T;
            const int key = c / (D / 8);
            const int dc = c - key * (D / 8);
            const int row = (key & ~31) | perm32(key & 31);
            store16(&lds_k[buf][row * KSTR + dc * 8], kst[i]);
        }
        // transpose: V^T[d][keys] for d = 8*v_dc + e
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            const bool odd = e & 1;
            uint32_t packed[KU / 2 > 0 ? KU / 2 : 1];
            if (KU == 1) {
                const uint32_t x = vst[0][w];
                uint16_t *dst = &lds_v[buf][(v_dc * 8 + e) * VSTR + v_kg];
                *dst = odd ? (uint16_t)(x >> 16) : (uint16_t)(x & 0xffffu);
                continue;
            }
#pragma unroll
            for (int u = 0; u < KU / 2; ++u) {
                const uint32_t x0 = vst[2 * u][w];
                const uint32_t x1 = vst[2 * u + 1][w];
                packed[u] = odd ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
            }
            uint16_t *dst = &lds_v[buf][(v_dc * 8 + e) * VSTR + v_kg * KU];
            if (KU == 2) {
                *reinterpret_cast<uint32_t *>(dst) = packed[0];
            } else if (KU == 4) {
                *reinterpret_cast<u32x2 *>(dst) = u32x2{packed[0], packed[1]};
            } else {
                *reinterpret_cast<u32x4 *>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
            }
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY;   // running max, log2 units
    float l_run = 0.f;         // running sum over this lane's half of the keys

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
    }

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) load_tile(t + 1);
        const int kt0 = t * BC;
        const bool active = (wrow0 < p.Lq) && (!p.causal || kt0 <= wrow1 + off);
        if (active) {
            const bool need_mask = (kt0 + BC > p.Lk) || (p.causal && kt0 + BC - 1 > wrow0 + off);
            // 1. S^T = K Q^T
            f32x16 s[BC / 32];
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
                const uint16_t *kr = &lds_k[buf][(kb * 32 + r) * KSTR + hh * 8];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    s[kb] = mfma32(as_bf16x8(load16(kr + ks * 16)), as_bf16x8(qreg[ks]), s[kb]);
            }
            // 2. score modifier, log2 units; tile max
            float mx = -INFINITY;
            const int qpos = qrow + off;
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = kt0 + kb * 32 + (e >> 3) * 16 + hh * 8 + (e & 7);
                    float x = s[kb][e] * p.scale_log2;
                    if (BIAS == kBiasAlibi) {
                        x -= slope_l2 * fabsf((float)(qpos - j));
                    } else if (BIAS == kBiasDenseF32 || BIAS == kBiasDenseBf16) {
                        const int bi = min(qrow, p.Lq - 1);
                        const int bj = min(j, p.Lk - 1);
                        const int64_t idx = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh +
                                            (int64_t)bi * p.bias_si + (int64_t)bj * p.bias_sj;
                        float bv;
                        if (BIAS == kBiasDenseF32)
                            bv = static_cast<const float *>(p.bias)[idx];
                        else
                            bv = bf16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[idx]);
                        x = fmaf(bv, kLog2e, x);
                    }
                    if (need_mask && (j >= p.Lk || (p.causal && j > qpos))) x = -INFINITY;
                    s[kb][e] = x;
                    mx = fmaxf(mx, x);
                }
            }
            mx = xor32_max(mx);
            // 3. lazy repair of l and O when the max has grown by more than TAU
            if (__any(mx > m_run + kTau)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
                m_run = m_new;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            // 4. P = 2^(t - m) in fp32, summed in fp32, packed to bf16
            uint32_t pk[BC / 32][8];
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const float p0 = exp2_fast(s[kb][e] - m_use);
                    const float p1 = exp2_fast(s[kb][e + 1] - m_use);
                    l_run += p0 + p1;
                    pk[kb][e >> 1] = pack_bf16x2(p0, p1);
                }
            }
            // 5. O^T += V^T P^T
#pragma unroll
            for (int kk = 0; kk < BC / 16; ++kk) {
                const int kb = kk >> 1;
                const int half = kk & 1;
                const bf16x8 bop = as_bf16x8(u32x4{pk[kb][4 * half], pk[kb][4 * half + 1],
                                                   pk[kb][4 * half + 2], pk[kb][4 * half + 3]});
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint16_t *vr = &lds_v[buf][(db * 32 + r) * VSTR + kk * 16 + hh * 8];
                    oacc[db] = mfma32(as_bf16x8(load16(vr)), bop, oacc[db]);
                }
            }
        }
        if (t + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    // epilogue
    const float l_tot = xor32_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow < p.Lq) {
        const int64_t obase = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)qrow * p.o_sl;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = db * 32 + i * 8 + hh * 4;
                const float o0 = oacc[db][4 * i + 0] * inv, o1 = oacc[db][4 * i + 1] * inv;
                const float o2 = oacc[db][4 * i + 2] * inv, o3 = oacc[db][4 * i + 3] * inv;
                if (OUT_BF16) {
                    uint16_t *dst = static_cast<uint16_t *>(p.o) + obase + d0;
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
                } else {
                    float *dst = static_cast<float *>(p.o) + obase + d0;
                    *reinterpret_cast<f32x4 *>(dst) = f32x4{o0, o1, o2, o3};
                }
            }
        }
        if (p.lse != nullptr && hh == 0) {
            const float lse = (l_tot > 0.f) ? m_run * kLn2 + logf(l_tot) : -INFINITY;
            p.lse[((int64_t)b * p.Hq + h) * p.Lq + qrow] = lse;
        }
    }
}

template <int D, int NW, int BIAS>
hipError_t launch_prefill_t(const FwdParams &p, hipStream_t stream) {
    const int BR = 32 * NW;
    const int64_t nqt = (p.Lq + BR - 1) / BR;
    const int64_t blocks = nqt * (int64_t)p.B * p.Hq;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks), block(NW * 64);
    if (p.o_bf16)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, BIAS, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, BIAS, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const FwdParams &p, hipStream_t stream) {
    constexpr int NW = 4;
    switch (p.bias_kind) {
        case kBiasNone: return launch_prefill_t<D, NW, kBiasNone>(p, stream);
        case kBiasAlibi: return launch_prefill_t<D, NW, kBiasAlibi>(p, stream);
        case kBiasDenseF32: return launch_prefill_t<D, NW, kBiasDenseF32>(p, stream);
        case kBiasDenseBf16: return launch_prefill_t<D, NW, kBiasDenseBf16>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const FwdParams &p, hipStream_t stream) {
    if (p.D == 128) return launch_prefill_d<128>(p, stream);
    if (p.D == 64) return launch_prefill_d<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
