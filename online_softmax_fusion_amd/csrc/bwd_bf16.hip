// bwd_bf16.hip -- gradients of the fused attention forward for bf16 Q/K/V on
// gfx950.
//
// The backward pass recomputes the attention weights from the saved
// log-sum-exp instead of storing them (the single-pass backward that the
// review "Optimal Software Pipelining and Warp Specialization for Tensor Core
// GPUs" describes in section 7.2, with its five matrix products and one
// exponential per tile).  With P = 2^(s * scale * log2(e) - LSE * log2(e)):
//
//   Delta_i = <dO_i, O_i>,  dP = dO V^T,  dS = P (dP - Delta)  [* cap slope]
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// That review's kernel gathers dQ with atomic additions in global memory.
// Here two kernels share the work instead, so that nothing is accumulated
// through memory and the result is deterministic:
//
//   bwd_dq_kernel    one workgroup per tile of 32 * NW query rows (like the
//                    forward): Q and dO stay in registers, K/V tiles of 64 keys
//                    stream through LDS.  Per tile and wave: S^T = K Q^T and
//                    dP^T = V dO^T (keys in the matrix-core rows, perm32 order,
//                    so each lane holds 32 scores of one query row in the order
//                    the next product reads them), P and dS in registers, then
//                    dQ^T += K^T dS^T with K read through the transposing LDS
//                    read.  It also forms Delta from O and dO, and writes Delta
//                    and LSE * log2(e) per row for the second kernel.
//   bwd_dkdv_kernel  one workgroup per 32 * NW keys of one K/V head: K and V
//                    stay in registers, Q/dO tiles of 64 rows of every query
//                    head of the group stream through LDS.  Per 32 query rows
//                    and wave: S = Q K^T and dP = dO V^T (queries in perm32
//                    order), P and dS in registers, dV^T += dO^T P and
//                    dK^T += Q^T dS with dO and Q read transposed.
//
// Both kernels read each streamed tile twice: as rows (16-byte reads along d)
// and transposed (ds_read_b64_tr_b16 along the rows).  One XOR swizzle of the
// 16-byte chunks serves both patterns without bank conflicts (see BwdCfg), so
// each tile is stored once.  Tiles are double-buffered with direct
// global->LDS loads, one barrier per tile; tiles that cross the causal
// diagonal, the window edges or the end of the rows take a masked code path.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kXcds = 8;

template <int D>
struct BwdCfg {
    static constexpr int BT = 64;          // rows per streamed tile
    static constexpr int RB = 2 * D;       // bytes per row in LDS (no padding)
    static constexpr int KS = D / 16;      // k-steps over d
    static constexpr int DB = D / 32;      // 32-row blocks over d
    static constexpr int TILE = BT * RB;   // bytes of one tile
    // XOR swizzle of the 16-byte chunk index of a row.  Row reads: 16 lanes
    // read one chunk of 16 rows (a permutation of 16 consecutive rows).
    // Transposing reads: 32 lanes read 4 chunks of 4 consecutive rows.  With
    // 64 banks of 4 bytes, D = 128 (one row per 256 bytes) takes the two
    // 2-bit halves of row % 16 swapped, D = 64 (two rows per 256 bytes) takes
    // bit 1 of the row to chunk bit 2 and bits 2-3 to chunk bits 0-1.  In both
    // cases rows r and r + 16 share a swizzle, and for the rows the
    // transposing reads start at (8h + 0..3), row + 4 has swizzle ^ 1.
    static __device__ __forceinline__ int swz(int row) {
        return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
    }
    static __device__ __forceinline__ int off(int row, int chunk) { return row * RB + ((chunk ^ swz(row)) << 4); }
    // row-read operand: matrix-core row r = lane % 32 reads tile row perm32(r),
    // chunk 2 * ks + lane / 32 at row_base(lane) ^ (ks << 5)
    static __device__ __forceinline__ int row_base(int lane) { return off(perm32(lane & 31), lane >> 5); }
    // transposing read of rows 8 * (lane / 32) + 0..3, d = lane % 32 of a
    // 32-wide d block: d block db at tr_base ^ (db << 6); rows + 4 at
    // (tr_base ^ 16) ^ (db << 6) + 4 * RB; rows + 16 * k at + 16 * k * RB
    static __device__ __forceinline__ int tr_base(int lane) {
        const int g = lane >> 4, sl = lane & 15;
        const int row = (g >> 1) * 8 + (sl >> 2);
        const int e = (g & 1) * 16 + 4 * (sl & 3);
        return off(row, e >> 3) + (e & 7) * 2;
    }
};

// A operand of a transposed product: 8 consecutive tile rows (rows0 + 8h +
// 0..7, h = lane / 32) of d = 32 * db + lane % 32.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char *tile, int tbase, int db, int rows0) {
    using C = BwdCfg<D>;
    const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(tile + (tbase ^ (db << 6)) + rows0 * C::RB));
    const u32x2 hi =
        lds_read_tr16(reinterpret_cast<const uint16_t *>(tile + ((tbase ^ 16) ^ (db << 6)) + (rows0 + 4) * C::RB));
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Weight and gradient of one score.  s: <q, k>; dp: <dO, v>; lse: LSE in log2
// units of the row (+inf for a row without weight); delta: <dO, O> of the row;
// dist: |position - key| (ALiBi); bias_v: the dense bias value.  Returns P in
// *pr and dU = P (dP - Delta) times the soft cap's slope.
template <int BIAS>
__device__ __forceinline__ float grad_of_score(const FwdParams &p, float s, float dp, float lse, float delta,
                                               float slope_l2, float dist, float bias_v, float *pr) {
    constexpr int BK = bias_base(BIAS);
    constexpr bool CAP = bias_cap(BIAS);
    constexpr bool FOLD = (BIAS == kBiasNone || BIAS == kBiasNoneScaled);
    float P, slope = 1.f;
    if (FOLD) {
        P = exp2_fast(fmaf(s, p.scale_log2, -lse));
    } else {
        float x = s * p.scale_log2;
        if (CAP) {
            x = soft_cap(x, p.cap_l2, p.cap_k, p.cap_inv);
            const float t = x * p.cap_inv;   // tanh of the scaled score over the cap
            slope = fmaf(-t, t, 1.f);
        }
        if (BK == kBiasAlibi) x = fmaf(-slope_l2, dist, x);
        if (BK == kBiasDenseF32 || BK == kBiasDenseBf16) x = fmaf(bias_v, kLog2e, x);
        P = exp2_fast(x - lse);
    }
    *pr = P;
    float du = P * (dp - delta);
    if (CAP) du *= slope;
    return du;
}

template <int BIAS>
__device__ __forceinline__ float dense_bias(const FwdParams &p, int b, int h, int i, int j) {
    constexpr int BK = bias_base(BIAS);
    if (BK != kBiasDenseF32 && BK != kBiasDenseBf16) return 0.f;
    const int bi = min(max(i, 0), p.Lq - 1);
    const int bj = min(max(j, 0), p.Lk - 1);
    const int64_t idx = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh + (int64_t)bi * p.bias_si +
                        (int64_t)bj * p.bias_sj;
    if (BK == kBiasDenseF32) return static_cast<const float *>(p.bias)[idx];
    return bf16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[idx]);
}

// Four consecutive values of a 32-row block of an accumulator, scaled, to row
// `row` of a [.., D] output at element d0.
__device__ __forceinline__ void store4(void *base, int64_t idx, bool bf16, float a, float b, float c, float d) {
    if (bf16) {
        uint16_t *dst = static_cast<uint16_t *>(base) + idx;
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
    } else {
        float *dst = static_cast<float *>(base) + idx;
        *reinterpret_cast<f32x4 *>(dst) = f32x4{a, b, c, d};
    }
}

// Direct global->LDS load of a 64-row tile (rows [r0, r0 + 64) of rows
// `base_`, `lbytes_` bytes apart, `nvalid_` of them present) into the LDS
// tile `LDS_`: lane fills LDS bytes [i*T*16 + wave*1024 + 16*lane, +16) from
// byte offset goff_ (+ round i's rows).  Missing rows read as zero.
#define BWD_LOAD_TILE(LDS_, SRC_, LBYTES_, NVALID_, GOFF_)                                                      \
    do {                                                                                                        \
        const __amdgpu_buffer_rsrc_t rs_ = make_rsrc((SRC_), (uint32_t)((NVALID_) - 1) * (LBYTES_) + D * 2);    \
        _Pragma("unroll") for (int i_ = 0; i_ < NC; ++i_) {                                                     \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                           \
                rs_, (__attribute__((address_space(3))) void *)((LDS_) + i_ * T * 16 + wave * 1024), 16,        \
                (int)(GOFF_), (int)(i_ * RROWS * (LBYTES_)), 0, 0);                                             \
        }                                                                                                       \
    } while (0)

// ---------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------
template <int D, int BIAS, bool MASK>
__device__ __forceinline__ void dq_tile(const FwdParams &p, const char *lk, const char *lv, int rbase, int tbase,
                                        const u32x4 (&qreg)[D / 16], const u32x4 (&doreg)[D / 16],
                                        f32x16 (&dqacc)[D / 32], float lse, float delta, int kt0, int wrow0,
                                        int wjmin, int wjmax, int qpos, int jmin, int jmax, int qrow,
                                        float slope_l2, int b, int h, int lane) {
    using C = BwdCfg<D>;
    if (MASK && !((wrow0 < p.Lq) && kt0 <= wjmax && kt0 + C::BT - 1 >= wjmin)) return;
    const int hh = lane >> 5;
    // S^T = K Q^T and dP^T = V dO^T, two 32-key blocks each
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][e] = dp[kb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = mfma32(as_bf16x8(load16(lk + ((rbase ^ (ks << 5)) + kb * 32 * C::RB))), as_bf16x8(qreg[ks]), s[kb]);
            dp[kb] = mfma32(as_bf16x8(load16(lv + ((rbase ^ (ks << 5)) + kb * 32 * C::RB))), as_bf16x8(doreg[ks]), dp[kb]);
        }
    // dU = P (dP - Delta) [* slope], packed to bf16 in the B-operand layout
    const float dbase = (float)(qpos - kt0 - hh * 8);
    uint32_t dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            float du[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int eo = kb * 32 + ((e + u) >> 3) * 16 + ((e + u) & 7);
                const int j = kt0 + eo + hh * 8;
                float pr;
                du[u] = grad_of_score<BIAS>(p, s[kb][e + u], dp[kb][e + u], lse, delta, slope_l2,
                                            fabsf(dbase - (float)eo), dense_bias<BIAS>(p, b, h, qrow, j), &pr);
                if (MASK && (j < jmin || j > jmax)) du[u] = 0.f;
            }
            dsk[kb][e >> 1] = pack_bf16x2(du[0], du[1]);
        }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kk = 0; kk < C::BT / 16; ++kk) {
        const int kb = kk >> 1, half = kk & 1;
        const bf16x8 bop = as_bf16x8(u32x4{dsk[kb][4 * half], dsk[kb][4 * half + 1], dsk[kb][4 * half + 2],
                                           dsk[kb][4 * half + 3]});
#pragma unroll
        for (int db = 0; db < C::DB; ++db) dqacc[db] = mfma32(tr_operand<D>(lk, tbase, db, kk * 16), bop, dqacc[db]);
    }
}

template <int D, int NW, int BIAS>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdParams bp) {
    using C = BwdCfg<D>;
    const FwdParams &p = bp.f;
    constexpr int BR = 32 * NW;
    constexpr int BC = C::BT;
    constexpr int T = NW * 64;
    constexpr int NC = C::TILE / (T * 16);
    constexpr int RROWS = T * 16 / C::RB;
    static_assert(NC >= 1 && C::TILE == NC * T * 16, "tile does not split evenly");
    static_assert(RROWS % 16 == 0, "rounds must keep the swizzle");

    __shared__ __attribute__((aligned(1024))) char lds_k0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_k1[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v1[C::TILE];

    // work item: XCD-contiguous ranges of a head-major list, heavy tiles first
    const int nqt = (p.Lq + BR - 1) / BR;
    const int nblocks = (int)gridDim.x;
    int item = blockIdx.x;
    if (nblocks % kXcds == 0) item = (blockIdx.x % kXcds) * (nblocks / kXcds) + blockIdx.x / kXcds;
    const int bh = item / nqt;
    int qt = item - bh * nqt;
    if (p.causal) qt = nqt - 1 - qt;
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    const int hk = h / p.G;
    const int q0 = qt * BR;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 31;
    const int hh = lane >> 5;
    const int off = p.Lk - p.Lq;
    const int qrow = q0 + wave * 32 + r;
    const int qpos = qrow + off;
    const int wrow0 = q0 + wave * 32;
    const int wrow1 = min(wrow0 + 31, p.Lq - 1);
    int jmin, jmax, wjmin, wjmax, unused;
    key_range(p, qpos, jmin, jmax);
    key_range(p, wrow0 + off, wjmin, unused);
    key_range(p, wrow1 + off, unused, wjmax);
    const int rlast = min(q0 + BR, p.Lq) - 1;
    int gjmin0, gjmax0, gjmin1, gjmax1;
    key_range(p, q0 + off, gjmin0, gjmax0);
    key_range(p, rlast + off, gjmin1, gjmax1);
    int t_first = 0, t_end = 0;
    if (rlast >= q0 && gjmax1 >= gjmin0) {
        t_first = gjmin0 / BC;
        t_end = gjmax1 / BC + 1;
    }
    const int u_first = max(t_first, (gjmin1 + BC - 1) / BC);
    const int u_end = min(t_end, gjmax0 >= 0 ? (gjmax0 + 1) / BC : 0);

    const uint16_t *kp = static_cast<const uint16_t *>(p.k) + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vp = static_cast<const uint16_t *>(p.v) + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;

    // Q, dO fragments (row qrow, d = 16*ks + 8*hh .. +7), Delta = <dO, O>
    u32x4 qreg[C::KS], doreg[C::KS];
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = doreg[ks] = u32x4{0, 0, 0, 0};
    const int64_t row_id = ((int64_t)b * p.Hq + h) * p.Lq + qrow;
    if (qrow < p.Lq) {
        const uint16_t *qr = static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh +
                             (int64_t)qrow * p.q_sl + hh * 8;
        const uint16_t *dr = static_cast<const uint16_t *>(bp.dout) + (int64_t)b * bp.do_sb + (int64_t)h * bp.do_sh +
                             (int64_t)qrow * bp.do_sl + hh * 8;
        const int64_t orow = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)qrow * p.o_sl + hh * 8;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            qreg[ks] = load16(qr + ks * 16);
            doreg[ks] = load16(dr + ks * 16);
            float ov[8];
            if (p.o_bf16) {
                const u32x4 o = load16(static_cast<const uint16_t *>(p.o) + orow + ks * 16);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    ov[2 * t] = bf16_bits_to_f32(o[t] & 0xffffu);
                    ov[2 * t + 1] = bf16_bits_to_f32(o[t] >> 16);
                }
            } else {
                const float *of = static_cast<const float *>(p.o) + orow + ks * 16;
                const f32x4 a = *reinterpret_cast<const f32x4 *>(of);
                const f32x4 c = *reinterpret_cast<const f32x4 *>(of + 4);
                ov[0] = a[0]; ov[1] = a[1]; ov[2] = a[2]; ov[3] = a[3];
                ov[4] = c[0]; ov[5] = c[1]; ov[6] = c[2]; ov[7] = c[3];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                dsum = fmaf(bf16_bits_to_f32(doreg[ks][t] & 0xffffu), ov[2 * t], dsum);
                dsum = fmaf(bf16_bits_to_f32(doreg[ks][t] >> 16), ov[2 * t + 1], dsum);
            }
        }
    }
    const float delta = xor32_sum(dsum);
    float lse = INFINITY;   // a row without weight (LSE = -inf, or past the end) gets P = 0
    if (qrow < p.Lq) {
        const float l = p.lse[row_id];
        if (l != -INFINITY) lse = l * kLog2e;
        if (hh == 0) {
            bp.delta[row_id] = delta;
            bp.lse_l2[row_id] = lse;
        }
    }

    float slope_l2 = 0.f;
    if (bias_base(BIAS) == kBiasAlibi) slope_l2 = p.slopes[h] * kLog2e;

    const int rbase = C::row_base(lane);
    const int tbase = C::tr_base(lane);
    const uint32_t kl_bytes = (uint32_t)p.k_sl * 2u;
    const uint32_t vl_bytes = (uint32_t)p.v_sl * 2u;
    uint32_t kgoff, vgoff;
    {
        const int pos = wave * 1024 + lane * 16;
        const int row = pos / C::RB;
        const int pc = (pos % C::RB) / 16;
        kgoff = (uint32_t)row * kl_bytes + (uint32_t)((pc ^ C::swz(row)) * 16);
        vgoff = (uint32_t)row * vl_bytes + (uint32_t)((pc ^ C::swz(row)) * 16);
    }

    f32x16 dqacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dqacc[db][e] = 0.f;

#define BWD_DQ_LOADS(TT_, KL_, VL_)                                                                             \
    do {                                                                                                        \
        const int j0_ = (TT_) * BC;                                                                             \
        const int nv_ = min(BC, p.Lk - j0_);                                                                    \
        BWD_LOAD_TILE(KL_, kp + (int64_t)j0_ * p.k_sl, kl_bytes, nv_, kgoff);                                   \
        BWD_LOAD_TILE(VL_, vp + (int64_t)j0_ * p.v_sl, vl_bytes, nv_, vgoff);                                   \
    } while (0)
#define BWD_DQ_STEP(MASK_, BUF_, TT_)                                                                           \
    dq_tile<D, BIAS, MASK_>(p, (BUF_) ? lds_k1 : lds_k0, (BUF_) ? lds_v1 : lds_v0, rbase, tbase, qreg, doreg,    \
                            dqacc, lse, delta, (TT_) * BC, wrow0, wjmin, wjmax, qpos, jmin, jmax, qrow, slope_l2, \
                            b, h, lane)

    if (t_end > t_first) {
        BWD_DQ_LOADS(t_first, lds_k0, lds_v0);
        wait_vmem();
        __syncthreads();
    }
    for (int t = t_first; t < t_end; ++t) {
        const bool masked = t < u_first || t >= u_end;
        if (((t - t_first) & 1) == 0) {
            if (t + 1 < t_end) BWD_DQ_LOADS(t + 1, lds_k1, lds_v1);
            if (masked)
                BWD_DQ_STEP(true, 0, t);
            else
                BWD_DQ_STEP(false, 0, t);
        } else {
            if (t + 1 < t_end) BWD_DQ_LOADS(t + 1, lds_k0, lds_v0);
            if (masked)
                BWD_DQ_STEP(true, 1, t);
            else
                BWD_DQ_STEP(false, 1, t);
        }
        wait_vmem();
        __syncthreads();
    }
#undef BWD_DQ_STEP
#undef BWD_DQ_LOADS

    if (qrow < p.Lq) {
        const int64_t base = (int64_t)b * bp.dq_sb + (int64_t)h * bp.dq_sh + (int64_t)qrow * bp.dq_sl;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store4(bp.dq, base + db * 32 + i * 8 + hh * 4, bp.grad_bf16, dqacc[db][4 * i] * sc,
                       dqacc[db][4 * i + 1] * sc, dqacc[db][4 * i + 2] * sc, dqacc[db][4 * i + 3] * sc);
    }
}

// ---------------------------------------------------------------------------
// dK/dV kernel
// ---------------------------------------------------------------------------
// 32 query rows (tile rows qs0 .. qs0 + 31, global row i0 + tile row) against
// this wave's 32 keys.
template <int D, int BIAS, bool MASK>
__device__ __forceinline__ void dkdv_rows(const FwdParams &p, const char *lq, const char *ldo, const float *llse,
                                          const float *ldel, int rbase, int tbase, const u32x4 (&kreg)[D / 16],
                                          const u32x4 (&vreg)[D / 16], f32x16 (&dkacc)[D / 32],
                                          f32x16 (&dvacc)[D / 32], int qs0, int i0, int key, int imin, int imax,
                                          float slope_l2, int b, int h, int lane) {
    using C = BwdCfg<D>;
    const int hh = lane >> 5;
    // S = Q K^T, dP = dO V^T (query perm32(r) in matrix-core row r)
    f32x16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        s = mfma32(as_bf16x8(load16(lq + ((rbase ^ (ks << 5)) + qs0 * C::RB))), as_bf16x8(kreg[ks]), s);
        dp = mfma32(as_bf16x8(load16(ldo + ((rbase ^ (ks << 5)) + qs0 * C::RB))), as_bf16x8(vreg[ks]), dp);
    }
    // element e of this lane: tile row qs0 + (e / 8) * 16 + 8 * hh + e % 8
    f32x4 L[4], Dl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int rr = qs0 + (g >> 1) * 16 + hh * 8 + (g & 1) * 4;
        L[g] = *reinterpret_cast<const f32x4 *>(llse + rr);
        Dl[g] = *reinterpret_cast<const f32x4 *>(ldel + rr);
    }
    const int ibase = i0 + qs0 + hh * 8;
    const float dbase = (float)(ibase + (p.Lk - p.Lq) - key);
    uint32_t pk[8], dk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        float pr[2], du[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int eo = ((e + u) >> 3) * 16 + ((e + u) & 7);
            const int i = ibase + eo;
            du[u] = grad_of_score<BIAS>(p, s[e + u], dp[e + u], L[(e + u) >> 2][(e + u) & 3],
                                        Dl[(e + u) >> 2][(e + u) & 3], slope_l2, fabsf(dbase + (float)eo),
                                        dense_bias<BIAS>(p, b, h, i, key), &pr[u]);
            if (MASK && (i < imin || i > imax)) pr[u] = du[u] = 0.f;
        }
        pk[e >> 1] = pack_bf16x2(pr[0], pr[1]);
        dk[e >> 1] = pack_bf16x2(du[0], du[1]);
    }
    // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 bp_ = as_bf16x8(u32x4{pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]});
        const bf16x8 bd_ = as_bf16x8(u32x4{dk[4 * kk], dk[4 * kk + 1], dk[4 * kk + 2], dk[4 * kk + 3]});
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            dvacc[db] = mfma32(tr_operand<D>(ldo, tbase, db, qs0 + kk * 16), bp_, dvacc[db]);
            dkacc[db] = mfma32(tr_operand<D>(lq, tbase, db, qs0 + kk * 16), bd_, dkacc[db]);
        }
    }
}

template <int D, int NW, int BIAS>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(BwdParams bp) {
    using C = BwdCfg<D>;
    const FwdParams &p = bp.f;
    constexpr int BK = 32 * NW;          // keys per workgroup
    constexpr int BQ = C::BT;            // query rows per streamed tile
    constexpr int T = NW * 64;
    constexpr int NC = C::TILE / (T * 16);
    constexpr int RROWS = T * 16 / C::RB;
    static_assert(NC >= 1 && C::TILE == NC * T * 16, "tile does not split evenly");
    static_assert(RROWS % 16 == 0, "rounds must keep the swizzle");
    static_assert(NW >= 2, "waves 0 and 1 load the per-row values");

    __shared__ __attribute__((aligned(1024))) char lds_q0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_q1[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_o0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_o1[C::TILE];
    __shared__ __attribute__((aligned(256))) float lds_l0[BQ];
    __shared__ __attribute__((aligned(256))) float lds_l1[BQ];
    __shared__ __attribute__((aligned(256))) float lds_d0[BQ];
    __shared__ __attribute__((aligned(256))) float lds_d1[BQ];

    // work item: XCD-contiguous ranges of a head-major list; key tiles in
    // ascending order (under the causal mask the first ones see the most rows)
    const int nkt = (p.Lk + BK - 1) / BK;
    const int nblocks = (int)gridDim.x;
    int item = blockIdx.x;
    if (nblocks % kXcds == 0) item = (blockIdx.x % kXcds) * (nblocks / kXcds) + blockIdx.x / kXcds;
    const int bhk = item / nkt;
    const int kt = item - bhk * nkt;
    const int b = bhk / p.Hkv;
    const int hk = bhk - b * p.Hkv;
    const int k0 = kt * BK;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 31;
    const int hh = lane >> 5;
    const int key = k0 + wave * 32 + r;
    int imin, imax;
    query_range(p, key, imin, imax);
    // rows seen by some key of this wave, and of the workgroup
    const int kw0 = k0 + wave * 32;
    const int kwl = min(kw0 + 31, p.Lk - 1);
    int wimin = 0, wimax = -1, unused;
    if (kw0 < p.Lk) {
        query_range(p, kw0, wimin, unused);
        query_range(p, kwl, unused, wimax);
    }
    const int klast = min(k0 + BK, p.Lk) - 1;
    int gimin0, gimax0, gimin1, gimax1;
    query_range(p, k0, gimin0, gimax0);
    query_range(p, klast, gimin1, gimax1);
    // query tiles [t_first, t_end) hold every row some key sees; tiles
    // [u_first, u_end) are seen in full by every key (no mask)
    int t_first = 0, t_end = 0;
    if (gimax1 >= gimin0 && gimax1 >= 0) {
        t_first = gimin0 / BQ;
        t_end = gimax1 / BQ + 1;
    }
    int u_first = max(t_first, (gimin1 + BQ - 1) / BQ);
    int u_end = min(t_end, gimax0 >= 0 ? (gimax0 + 1) / BQ : 0);
    if (k0 + BK > p.Lk || gimax1 < gimin1 || gimax0 < gimin0) u_end = u_first;   // a partial key tile: all masked
    const int nt = t_end - t_first;
    const int iters = nt * p.G;

    const uint16_t *kp = static_cast<const uint16_t *>(p.k) + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vp = static_cast<const uint16_t *>(p.v) + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
    u32x4 kreg[C::KS], vreg[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kreg[ks] = vreg[ks] = u32x4{0, 0, 0, 0};
    if (key < p.Lk) {
        const uint16_t *kr = kp + (int64_t)key * p.k_sl + hh * 8;
        const uint16_t *vr = vp + (int64_t)key * p.v_sl + hh * 8;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            kreg[ks] = load16(kr + ks * 16);
            vreg[ks] = load16(vr + ks * 16);
        }
    }

    const int rbase = C::row_base(lane);
    const int tbase = C::tr_base(lane);
    const uint32_t ql_bytes = (uint32_t)p.q_sl * 2u;
    const uint32_t dl_bytes = (uint32_t)bp.do_sl * 2u;
    uint32_t qgoff, dgoff;
    {
        const int pos = wave * 1024 + lane * 16;
        const int row = pos / C::RB;
        const int pc = (pos % C::RB) / 16;
        qgoff = (uint32_t)row * ql_bytes + (uint32_t)((pc ^ C::swz(row)) * 16);
        dgoff = (uint32_t)row * dl_bytes + (uint32_t)((pc ^ C::swz(row)) * 16);
    }

    f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dkacc[db][e] = dvacc[db][e] = 0.f;

    // iteration it: query head hk*G + it / nt, query tile t_first + it % nt
#define BWD_KV_LOADS(IT_, QL_, OL_, LL_, DL_)                                                                   \
    do {                                                                                                        \
        const int hi_ = (IT_) / nt;                                                                             \
        const int h_ = hk * p.G + hi_;                                                                          \
        const int q0_ = (t_first + (IT_) - hi_ * nt) * BQ;                                                      \
        const int nv_ = min(BQ, p.Lq - q0_);                                                                    \
        BWD_LOAD_TILE(QL_, static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb + (int64_t)h_ * p.q_sh +     \
                               (int64_t)q0_ * p.q_sl, ql_bytes, nv_, qgoff);                                    \
        BWD_LOAD_TILE(OL_, static_cast<const uint16_t *>(bp.dout) + (int64_t)b * bp.do_sb +                    \
                               (int64_t)h_ * bp.do_sh + (int64_t)q0_ * bp.do_sl, dl_bytes, nv_, dgoff);         \
        const int64_t rw_ = ((int64_t)b * p.Hq + h_) * p.Lq + q0_;                                              \
        if (wave == 0)                                                                                          \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(bp.lse_l2 + rw_, (uint32_t)nv_ * 4u),           \
                                                     (__attribute__((address_space(3))) void *)(LL_), 4,        \
                                                     lane * 4, 0, 0, 0);                                        \
        if (wave == 1)                                                                                          \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(bp.delta + rw_, (uint32_t)nv_ * 4u),            \
                                                     (__attribute__((address_space(3))) void *)(DL_), 4,        \
                                                     lane * 4, 0, 0, 0);                                        \
    } while (0)
#define BWD_KV_STEP(MASK_, BUF_, IT_)                                                                           \
    do {                                                                                                        \
        const int hi_ = (IT_) / nt;                                                                             \
        const int h_ = hk * p.G + hi_;                                                                          \
        const int q0_ = (t_first + (IT_) - hi_ * nt) * BQ;                                                      \
        const float sl_ = bias_base(BIAS) == kBiasAlibi ? p.slopes[h_] * kLog2e : 0.f;                          \
        if (!(MASK_) || (wimax >= wimin && q0_ <= wimax && q0_ + BQ - 1 >= wimin)) {                            \
            _Pragma("unroll 1") for (int sub_ = 0; sub_ < BQ / 32; ++sub_)                                      \
                dkdv_rows<D, BIAS, MASK_>(p, (BUF_) ? lds_q1 : lds_q0, (BUF_) ? lds_o1 : lds_o0,                \
                                          (BUF_) ? lds_l1 : lds_l0, (BUF_) ? lds_d1 : lds_d0, rbase, tbase,     \
                                          kreg, vreg, dkacc, dvacc, sub_ * 32, q0_, key, imin, imax, sl_, b,    \
                                          h_, lane);                                                            \
        }                                                                                                       \
    } while (0)

    if (iters > 0) {
        BWD_KV_LOADS(0, lds_q0, lds_o0, lds_l0, lds_d0);
        wait_vmem();
        __syncthreads();
    }
    for (int it = 0; it < iters; ++it) {
        const int tq = t_first + it % nt;
        const bool masked = tq < u_first || tq >= u_end;
        if ((it & 1) == 0) {
            if (it + 1 < iters) BWD_KV_LOADS(it + 1, lds_q1, lds_o1, lds_l1, lds_d1);
            if (masked)
                BWD_KV_STEP(true, 0, it);
            else
                BWD_KV_STEP(false, 0, it);
        } else {
            if (it + 1 < iters) BWD_KV_LOADS(it + 1, lds_q0, lds_o0, lds_l0, lds_d0);
            if (masked)
                BWD_KV_STEP(true, 1, it);
            else
                BWD_KV_STEP(false, 1, it);
        }
        wait_vmem();
        __syncthreads();
    }
#undef BWD_KV_STEP
#undef BWD_KV_LOADS

    if (key < p.Lk) {
        const int64_t kb = (int64_t)b * bp.dk_sb + (int64_t)hk * bp.dk_sh + (int64_t)key * bp.dk_sl;
        const int64_t vb = (int64_t)b * bp.dv_sb + (int64_t)hk * bp.dv_sh + (int64_t)key * bp.dv_sl;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = db * 32 + i * 8 + hh * 4;
                store4(bp.dk, kb + d0, bp.grad_bf16, dkacc[db][4 * i] * sc, dkacc[db][4 * i + 1] * sc,
                       dkacc[db][4 * i + 2] * sc, dkacc[db][4 * i + 3] * sc);
                store4(bp.dv, vb + d0, bp.grad_bf16, dvacc[db][4 * i], dvacc[db][4 * i + 1], dvacc[db][4 * i + 2],
                       dvacc[db][4 * i + 3]);
            }
    }
}

template <int D, int BIAS>
hipError_t launch_bwd_t(const BwdParams &p, hipStream_t stream) {
    constexpr int NW = 4;
    const int64_t nqt = (p.f.Lq + 32 * NW - 1) / (32 * NW);
    const int64_t dq_blocks = nqt * (int64_t)p.f.B * p.f.Hq;
    const int64_t nkt = (p.f.Lk + 32 * NW - 1) / (32 * NW);
    const int64_t kv_blocks = nkt * (int64_t)p.f.B * p.f.Hkv;
    if (dq_blocks > 0x7fffffff || kv_blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (dq_blocks > 0) {
        hipLaunchKernelGGL((bwd_dq_kernel<D, NW, BIAS>), dim3((unsigned)dq_blocks), dim3(NW * 64), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (kv_blocks > 0) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, BIAS>), dim3((unsigned)kv_blocks), dim3(NW * 64), 0, stream, p);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int D>
hipError_t launch_bwd_d(const BwdParams &p, hipStream_t stream) {
    // the folded exponent needs no sign condition on the scale here (no max)
    const int kind = p.f.bias_kind == kBiasNoneScaled ? (int)kBiasNone : p.f.bias_kind;
    switch (kind) {
        case kBiasNone: return launch_bwd_t<D, kBiasNone>(p, stream);
        case kBiasAlibi: return launch_bwd_t<D, kBiasAlibi>(p, stream);
        case kBiasDenseF32: return launch_bwd_t<D, kBiasDenseF32>(p, stream);
        case kBiasDenseBf16: return launch_bwd_t<D, kBiasDenseBf16>(p, stream);
        case kBiasNoneCap: return launch_bwd_t<D, kBiasNoneCap>(p, stream);
        case kBiasAlibiCap: return launch_bwd_t<D, kBiasAlibiCap>(p, stream);
        case kBiasDenseF32Cap: return launch_bwd_t<D, kBiasDenseF32Cap>(p, stream);
        case kBiasDenseBf16Cap: return launch_bwd_t<D, kBiasDenseBf16Cap>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams &p, hipStream_t stream) {
    if (p.f.D == 128) return launch_bwd_d<128>(p, stream);
    if (p.f.D == 64) return launch_bwd_d<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
