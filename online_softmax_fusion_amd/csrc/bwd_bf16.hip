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
//                    dK^T += Q^T dS with dO and Q read transposed.  At d = 128
//                    bwd_dkdv_pair_kernel does this work instead, with the K/V
//                    rows in LDS and pairs of waves splitting the query rows,
//                    so that two waves fit on each SIMD.
//
// Both kernels read each streamed tile twice: as rows (16-byte reads along d)
// and transposed (ds_read_b64_tr_b16 along the rows).  One XOR swizzle of the
// 16-byte chunks serves both patterns without bank conflicts (see BwdCfg), so
// each tile is stored once.  Tiles are double-buffered in two LDS stages,
// filled by buffer-to-LDS loads issued one tile ahead, one barrier per tile;
// tiles that cross the causal diagonal, the window edges or the end of the
// rows take a masked code path.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {


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

// A 64-row tile (rows `src` .. + 63, `lbytes` apart, `nvalid` of them present)
// into the LDS tile at byte address `lds`: lane fills LDS bytes
// [i*T*16 + wave*1024 + 16*lane, +16) of round i from byte offset goff of the
// source (+ round i's rows, RROWS rows per round).  Missing rows read as 0:
// the whole offset goes in the vector offset, which the hardware checks
// against the descriptor's range (the scalar offset is not checked).
template <int D, int T>
__device__ __forceinline__ void dma_tile(const void *src, uint32_t lbytes, int nvalid, uint32_t lds, int wave,
                                         uint32_t goff) {
    using C = BwdCfg<D>;
    constexpr int NC = C::TILE / (T * 16);
    constexpr int RROWS = T * 16 / C::RB;
    static_assert(NC >= 1 && C::TILE == NC * T * 16, "tile does not split evenly");
    static_assert(RROWS % 16 == 0, "rounds must keep the swizzle");
    const i32x4 rs = rsrc_words(src, (uint32_t)(nvalid - 1) * lbytes + D * 2);
#pragma unroll
    for (int i = 0; i < NC; ++i) dma16(rs, lds + i * T * 16 + wave * 1024, goff + (uint32_t)(i * RROWS) * lbytes);
}

// this lane's source offset inside a tile: LDS position wave*1024 + 16*lane
// holds chunk pc of row `row`, i.e. logical chunk pc ^ swz(row) of that row
template <int D>
__device__ __forceinline__ uint32_t tile_goff(int wave, int lane, uint32_t lbytes) {
    using C = BwdCfg<D>;
    const int pos = wave * 1024 + lane * 16;
    const int row = pos / C::RB;
    const int pc = (pos % C::RB) / 16;
    return (uint32_t)row * lbytes + (uint32_t)((pc ^ C::swz(row)) * 16);
}

// ---------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------
// One K/V tile for this wave.  `masked` tiles (the causal diagonal, window
// edges, key tail) zero the scores of keys a row cannot see; only that
// elementwise step branches on it, so the matrix chains and the dQ
// accumulators are the same code and registers on both kinds of tile.
template <int D, int BIAS>
__device__ __forceinline__ void dq_tile(const FwdParams &p, const char *lk, const char *lv, int rbase, int tbase,
                                        const u32x4 (&qreg)[D / 16], const u32x4 (&doreg)[D / 16],
                                        f32x16 (&dqacc)[D / 32], float lse, float delta, int kt0, int wrow0,
                                        int wjmin, int wjmax, int qpos, int jmin, int jmax, int qrow,
                                        float slope_l2, int b, int h, int lane, bool masked) {
    using C = BwdCfg<D>;
    if (masked && !((wrow0 < p.Lq) && kt0 <= wjmax && kt0 + C::BT - 1 >= wjmin)) return;
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
    // schedule (D = 128): two operand reads in flight ahead of the matrix core
    // (3.6-4% faster backward than the compiler's own order, measured; at
    // D = 64 the hints measured 0-1.6% slower and are left out)
    if constexpr (D == 128) {
        constexpr int RA = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
#pragma unroll
        for (int i = 0; i < 4 * C::KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < 4 * C::KS - RA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
    // dU = P (dP - Delta) [* slope] (in place of the scores), then on masked
    // tiles zeroed outside [jmin, jmax], packed to bf16 in the B-operand layout
    const float dbase = (float)(qpos - kt0 - hh * 8);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int eo = kb * 32 + (e >> 3) * 16 + (e & 7);
            const int j = kt0 + eo + hh * 8;
            float pr;
            s[kb][e] = grad_of_score<BIAS>(p, s[kb][e], dp[kb][e], lse, delta, slope_l2, fabsf(dbase - (float)eo),
                                           dense_bias<BIAS>(p, b, h, qrow, j), &pr);
        }
    if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = kt0 + kb * 32 + (e >> 3) * 16 + (e & 7) + hh * 8;
                if (j < jmin || j > jmax) s[kb][e] = 0.f;
            }
    }
    uint32_t dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) dsk[kb][e >> 1] = pack_bf16x2(s[kb][e], s[kb][e + 1]);
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kk = 0; kk < C::BT / 16; ++kk) {
        const int kb = kk >> 1, half = kk & 1;
        const bf16x8 bop = as_bf16x8(u32x4{dsk[kb][4 * half], dsk[kb][4 * half + 1], dsk[kb][4 * half + 2],
                                           dsk[kb][4 * half + 3]});
#pragma unroll
        for (int db = 0; db < C::DB; ++db) dqacc[db] = mfma32(tr_operand<D>(lk, tbase, db, kk * 16), bop, dqacc[db]);
    }
    // schedule (D = 128): the two transposing reads of four products ahead
    if constexpr (D == 128) {
        constexpr int RV = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * RV, 1);
#pragma unroll
        for (int i = 0; i < C::BT / 16 * C::DB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            if (i < C::BT / 16 * C::DB - RV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
    }
}

template <int D, int NW, int BIAS>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdParams bp) {
    using C = BwdCfg<D>;
    const FwdParams &p = bp.f;
    constexpr int BR = 32 * NW;
    constexpr int BC = C::BT;
    constexpr int T = NW * 64;
    constexpr int STAGE = 2 * C::TILE;   // K tile, then V tile

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    // work item: XCD-contiguous ranges of heads; under a causal mask the last
    // query tile sees the most keys and goes first
    const int nqt = (p.Lq + BR - 1) / BR;
    const WorkItem wi = xcd_work_item(nqt, p.causal && !p.window, p.num_xcds);
    const int bh = wi.head;
    const int qt = p.causal ? nqt - 1 - wi.rank : wi.rank;
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
    const uint32_t kgoff = tile_goff<D>(wave, lane, kl_bytes);
    const uint32_t vgoff = tile_goff<D>(wave, lane, vl_bytes);
    const uint32_t lds0 = lds_addr(smem);

    f32x16 dqacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dqacc[db][e] = 0.f;

    // K/V tile t into stage `st`
    auto issue = [&](int t, int st) {
        const int j0 = t * BC;
        const int nv = min(BC, p.Lk - j0);
        const uint32_t dst = lds0 + st * STAGE;
        dma_tile<D, T>(kp + (int64_t)j0 * p.k_sl, kl_bytes, nv, dst, wave, kgoff);
        dma_tile<D, T>(vp + (int64_t)j0 * p.v_sl, vl_bytes, nv, dst + C::TILE, wave, vgoff);
    };
    if (t_end > t_first) {
        issue(t_first, 0);
        wait_all_loads();
        __syncthreads();
    }
    for (int t = t_first; t < t_end; ++t) {
        const int st = (t - t_first) & 1;
        if (t + 1 < t_end) issue(t + 1, st ^ 1);
        const char *lk = smem + st * STAGE;
        dq_tile<D, BIAS>(p, lk, lk + C::TILE, rbase, tbase, qreg, doreg, dqacc, lse, delta, t * BC, wrow0, wjmin,
                         wjmax, qpos, jmin, jmax, qrow, slope_l2, b, h, lane, t < u_first || t >= u_end);
        wait_all_loads();
        __syncthreads();
    }

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
// P and dU of this lane's 16 scores (element e: tile row qs0 + (e / 8) * 16 +
// 8h + e % 8, h = lane / 32), packed to bf16 pairs.  With MASK, rows outside
// [imin, imax] (the rows that see this lane's key) get 0.
template <int BIAS, bool MASK>
__device__ __forceinline__ void dkdv_scores(const FwdParams &p, const f32x16 &s, const f32x16 &dp,
                                            const f32x4 (&L)[4], const f32x4 (&Dl)[4], int ibase, int key,
                                            int imin, int imax, float slope_l2, int b, int h, uint32_t (&pk)[8],
                                            uint32_t (&dk)[8]) {
    const float dbase = (float)(ibase + (p.Lk - p.Lq) - key);
    // element offset eo is visible iff (unsigned)(eo - lo) <= span; a key no
    // row sees (imax < imin) gets lo = -1, span = 0, which admits no eo >= 0
    const bool seen = imax >= imin;
    const int lo = seen ? imin - ibase : -1;
    const uint32_t span = seen ? (uint32_t)(imax - imin) : 0u;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        float pr[2], du[2];
        // with ALiBi the distances are formed pair by pair where they are used
        // (not all sixteen ahead of the products, which costs registers)
        float db = dbase;
        if constexpr (bias_base(BIAS) == kBiasAlibi) asm volatile("" : "+v"(db));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int eo = ((e + u) >> 3) * 16 + ((e + u) & 7);
            du[u] = grad_of_score<BIAS>(p, s[e + u], dp[e + u], L[(e + u) >> 2][(e + u) & 3],
                                        Dl[(e + u) >> 2][(e + u) & 3], slope_l2, fabsf(db + (float)eo),
                                        dense_bias<BIAS>(p, b, h, ibase + eo, key), &pr[u]);
            if (MASK && (uint32_t)(eo - lo) > span) pr[u] = du[u] = 0.f;
        }
        pk[e >> 1] = pack_bf16x2(pr[0], pr[1]);
        dk[e >> 1] = pack_bf16x2(du[0], du[1]);
    }
}

// 32 query rows (tile rows qs0 .. qs0 + 31, global row i0 + tile row) against
// this wave's 32 keys.
template <int D, int BIAS>
__device__ __forceinline__ void dkdv_rows(const FwdParams &p, const char *lq, const char *ldo, const float *llse,
                                          const float *ldel, int rbase, int tbase, const u32x4 (&kreg)[D / 16],
                                          const u32x4 (&vreg)[D / 16], f32x16 (&dkacc)[D / 32],
                                          f32x16 (&dvacc)[D / 32], int qs0, int i0, int key, int imin, int imax,
                                          bool masked, float slope_l2, int b, int h, int lane) {
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
    // schedule (D = 128): four operand reads ahead of the matrix core (one
    // wave per SIMD: only this wave's own order hides the LDS latency)
    if constexpr (D == 128) {
        constexpr int KA = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, KA, 2);
#pragma unroll
        for (int i = 0; i < 2 * C::KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            if (i < 2 * C::KS - KA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
        }
    }
    f32x4 L[4], Dl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int rr = qs0 + (g >> 1) * 16 + hh * 8 + (g & 1) * 4;
        L[g] = *reinterpret_cast<const f32x4 *>(llse + rr);
        Dl[g] = *reinterpret_cast<const f32x4 *>(ldel + rr);
    }
    const int ibase = i0 + qs0 + hh * 8;
    uint32_t pk[8], dk[8];
    // the branch covers only the elementwise part, so both paths leave the
    // accumulators alone (and in the same registers)
    if (masked)
        dkdv_scores<BIAS, true>(p, s, dp, L, Dl, ibase, key, imin, imax, slope_l2, b, h, pk, dk);
    else
        dkdv_scores<BIAS, false>(p, s, dp, L, Dl, ibase, key, imin, imax, slope_l2, b, h, pk, dk);
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
    // schedule (D = 128): the two transposing reads of two products ahead
    if constexpr (D == 128) {
        constexpr int KV = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KV, 3);
#pragma unroll
        for (int i = 0; i < 4 * C::DB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
            if (i < 4 * C::DB - KV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
        }
    }
}

// The same for a wave whose keys' K and V rows sit in LDS (rows read like the
// Q rows: key row kr of lane r at kvb ^ (ks << 5)) instead of registers.
template <int D, int BIAS>
__device__ __forceinline__ void dkdv_rows_kv(const FwdParams &p, const char *lq, const char *ldo, const float *llse,
                                             const float *ldel, int rbase, int tbase, const char *lk, const char *lv,
                                             int kvb, f32x16 (&dkacc)[D / 32], f32x16 (&dvacc)[D / 32], int qs0,
                                             int i0, int key, int imin, int imax, bool masked, float slope_l2, int b,
                                             int h, int lane) {
    using C = BwdCfg<D>;
    const int hh = lane >> 5;
    // S = Q K^T, dP = dO V^T (query perm32(r) in matrix-core row r)
    f32x16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        s = mfma32(as_bf16x8(load16(lq + ((rbase ^ (ks << 5)) + qs0 * C::RB))), as_bf16x8(load16(lk + (kvb ^ (ks << 5)))),
                   s);
        dp = mfma32(as_bf16x8(load16(ldo + ((rbase ^ (ks << 5)) + qs0 * C::RB))),
                    as_bf16x8(load16(lv + (kvb ^ (ks << 5)))), dp);
    }
    // schedule: the two operand reads of each product four products ahead of
    // it (1 and 2 measured 6% and 0.5% slower)
    {
        constexpr int KA = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KA, 2);
#pragma unroll
        for (int i = 0; i < 2 * C::KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            if (i < 2 * C::KS - KA) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
        }
    }
    f32x4 L[4], Dl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int rr = qs0 + (g >> 1) * 16 + hh * 8 + (g & 1) * 4;
        L[g] = *reinterpret_cast<const f32x4 *>(llse + rr);
        Dl[g] = *reinterpret_cast<const f32x4 *>(ldel + rr);
    }
    const int ibase = i0 + qs0 + hh * 8;
    uint32_t pk[8], dk[8];
    if (masked)
        dkdv_scores<BIAS, true>(p, s, dp, L, Dl, ibase, key, imin, imax, slope_l2, b, h, pk, dk);
    else
        dkdv_scores<BIAS, false>(p, s, dp, L, Dl, ibase, key, imin, imax, slope_l2, b, h, pk, dk);
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
    {
        constexpr int KV = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KV, 3);
#pragma unroll
        for (int i = 0; i < 4 * C::DB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
            if (i < 4 * C::DB - KV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
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
    static_assert(NW >= 2, "waves 0 and 1 load the per-row values");
    // one stage: Q tile, dO tile, LSE (log2 units) and Delta of its BQ rows
    constexpr int STAGE = 2 * C::TILE + 2 * BQ * 4;

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    // work item: XCD-contiguous ranges of K/V heads; key tiles in ascending
    // order (under the causal mask the first ones see the most rows)
    const int nkt = (p.Lk + BK - 1) / BK;
    const WorkItem wi = xcd_work_item(nkt, p.causal && !p.window, p.num_xcds);
    const int bhk = wi.head;
    const int kt = wi.rank;
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
    const uint32_t qgoff = tile_goff<D>(wave, lane, ql_bytes);
    const uint32_t dgoff = tile_goff<D>(wave, lane, dl_bytes);
    const uint32_t lds0 = lds_addr(smem);

    f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dkacc[db][e] = dvacc[db][e] = 0.f;

    // iteration it: query head hk*G + it / nt, query tile t_first + it % nt,
    // its tiles in stage it & 1
    auto issue = [&](int it, int st) {
        const int hi = it / nt;
        const int hq = hk * p.G + hi;
        const int q0 = (t_first + it - hi * nt) * BQ;
        const int nv = min(BQ, p.Lq - q0);
        const uint32_t dst = lds0 + st * STAGE;
        dma_tile<D, T>(static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh +
                           (int64_t)q0 * p.q_sl, ql_bytes, nv, dst, wave, qgoff);
        dma_tile<D, T>(static_cast<const uint16_t *>(bp.dout) + (int64_t)b * bp.do_sb + (int64_t)hq * bp.do_sh +
                           (int64_t)q0 * bp.do_sl, dl_bytes, nv, dst + C::TILE, wave, dgoff);
        const int64_t rw = ((int64_t)b * p.Hq + hq) * p.Lq + q0;
        // the lane's byte offset, formed here from the lane id rather than held across the loop
        const uint32_t l4 = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) * 4u;
        if (wave == 0) dma4(rsrc_words(bp.lse_l2 + rw, (uint32_t)nv * 4u), dst + 2 * C::TILE, l4);
        if (wave == 1) dma4(rsrc_words(bp.delta + rw, (uint32_t)nv * 4u), dst + 2 * C::TILE + BQ * 4, l4);
    };
    auto step = [&](bool masked, int it, int st) {
        const int hi = it / nt;
        const int hq = hk * p.G + hi;
        const int q0 = (t_first + it - hi * nt) * BQ;
        if (masked && !(wimax >= wimin && q0 <= wimax && q0 + BQ - 1 >= wimin)) return;
        const float sl = bias_base(BIAS) == kBiasAlibi ? p.slopes[hq] * kLog2e : 0.f;
        const char *sb = smem + st * STAGE;
        const float *ll = reinterpret_cast<const float *>(sb + 2 * C::TILE);
#pragma unroll 1
        for (int sub = 0; sub < BQ / 32; ++sub) {
            dkdv_rows<D, BIAS>(p, sb, sb + C::TILE, ll, ll + BQ, rbase, tbase, kreg, vreg, dkacc, dvacc, sub * 32,
                               q0, key, imin, imax, masked, sl, b, hq, lane);
        }
    };

    if (iters > 0) {
        issue(0, 0);
        wait_all_loads();
        __syncthreads();
    }
    for (int it = 0; it < iters; ++it) {
        const int st = it & 1;
        if (it + 1 < iters) issue(it + 1, st ^ 1);
        const int tq = t_first + it % nt;
        step(tq < u_first || tq >= u_end, it, st);
        wait_all_loads();
        __syncthreads();
    }

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

// dK/dV with two waves per SIMD (d = 128): eight waves per workgroup in four
// pairs, each pair owning 32 of the workgroup's 128 keys.  The keys' K and V
// rows sit in LDS (64 KiB, loaded once) instead of registers, which brings a
// wave under the 256 registers that two waves per SIMD allow; the two waves of
// a pair take alternate 32-row halves of every streamed Q/dO tile and add
// their partial dK, dV through LDS at the end, so the sums keep one order
// (bitwise deterministic).
template <int D, int BIAS>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(BwdParams bp) {
    using C = BwdCfg<D>;
    const FwdParams &p = bp.f;
    constexpr int NW = 8;
    constexpr int BK = 128;              // keys per workgroup
    constexpr int BQ = C::BT;            // query rows per streamed tile
    constexpr int T = NW * 64;
    constexpr int STAGE = 2 * C::TILE + 2 * BQ * 4;
    static_assert(BK == 2 * C::BT, "the key block is two tiles");
    static_assert(D * 64 * 4 <= 2 * C::TILE, "a pair's partial sums fit in half of the K/V area");

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
    __shared__ __attribute__((aligned(1024))) char kvs[4 * C::TILE];   // K rows 0..127, then V rows 0..127

    const int nkt = (p.Lk + BK - 1) / BK;
    const WorkItem wi = xcd_work_item(nkt, p.causal && !p.window, p.num_xcds);
    const int bhk = wi.head;
    const int kt = wi.rank;
    const int b = bhk / p.Hkv;
    const int hk = bhk - b * p.Hkv;
    const int k0 = kt * BK;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1;
    const int half = wave & 1;
    const int lane = tid & 63;
    const int r = lane & 31;
    const int hh = lane >> 5;
    const int key = k0 + pair * 32 + r;
    int imin, imax;
    query_range(p, key, imin, imax);
    const int kw0 = k0 + pair * 32;
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
    const int rbase = C::row_base(lane);
    const int tbase = C::tr_base(lane);
    const int kvb = C::off(pair * 32 + r, hh);
    const uint32_t ql_bytes = (uint32_t)p.q_sl * 2u;
    const uint32_t dl_bytes = (uint32_t)bp.do_sl * 2u;
    const uint32_t qgoff = tile_goff<D>(wave, lane, ql_bytes);
    const uint32_t dgoff = tile_goff<D>(wave, lane, dl_bytes);
    const uint32_t lds0 = lds_addr(smem);

    // the workgroup's K and V rows (rows past Lk read as zero; no row sees those keys)
    {
        const uint32_t kl_bytes = (uint32_t)p.k_sl * 2u;
        const uint32_t vl_bytes = (uint32_t)p.v_sl * 2u;
        const uint32_t kvs0 = lds_addr(kvs);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kr0 = k0 + t * C::BT;
            const int nv = min(C::BT, p.Lk - kr0);
            if (nv > 0) {
                dma_tile<D, T>(kp + (int64_t)kr0 * p.k_sl, kl_bytes, nv, kvs0 + t * C::TILE, wave,
                               tile_goff<D>(wave, lane, kl_bytes));
                dma_tile<D, T>(vp + (int64_t)kr0 * p.v_sl, vl_bytes, nv, kvs0 + (2 + t) * C::TILE, wave,
                               tile_goff<D>(wave, lane, vl_bytes));
            }
        }
    }

    f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dkacc[db][e] = dvacc[db][e] = 0.f;

    auto issue = [&](int it, int st) {
        const int hi = it / nt;
        const int hq = hk * p.G + hi;
        const int q0 = (t_first + it - hi * nt) * BQ;
        const int nv = min(BQ, p.Lq - q0);
        const uint32_t dst = lds0 + st * STAGE;
        dma_tile<D, T>(static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh +
                           (int64_t)q0 * p.q_sl, ql_bytes, nv, dst, wave, qgoff);
        dma_tile<D, T>(static_cast<const uint16_t *>(bp.dout) + (int64_t)b * bp.do_sb + (int64_t)hq * bp.do_sh +
                           (int64_t)q0 * bp.do_sl, dl_bytes, nv, dst + C::TILE, wave, dgoff);
        const int64_t rw = ((int64_t)b * p.Hq + hq) * p.Lq + q0;
        // the lane's byte offset, formed here from the lane id rather than held across the loop
        const uint32_t l4 = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) * 4u;
        if (wave == 0) dma4(rsrc_words(bp.lse_l2 + rw, (uint32_t)nv * 4u), dst + 2 * C::TILE, l4);
        if (wave == 1) dma4(rsrc_words(bp.delta + rw, (uint32_t)nv * 4u), dst + 2 * C::TILE + BQ * 4, l4);
    };
    auto step = [&](bool masked, int it, int st) {
        const int hi = it / nt;
        const int hq = hk * p.G + hi;
        const int q0 = (t_first + it - hi * nt) * BQ;
        if (masked && !(wimax >= wimin && q0 <= wimax && q0 + BQ - 1 >= wimin)) return;
        const float sl = bias_base(BIAS) == kBiasAlibi ? p.slopes[hq] * kLog2e : 0.f;
        const char *sb = smem + st * STAGE;
        const float *ll = reinterpret_cast<const float *>(sb + 2 * C::TILE);
        dkdv_rows_kv<D, BIAS>(p, sb, sb + C::TILE, ll, ll + BQ, rbase, tbase, kvs, kvs + 2 * C::TILE, kvb, dkacc,
                              dvacc, half * 32, q0, key, imin, imax, masked, sl, b, hq, lane);
    };

    if (iters > 0) issue(0, 0);
    wait_all_loads();
    __syncthreads();
    for (int it = 0; it < iters; ++it) {
        const int st = it & 1;
        if (it + 1 < iters) issue(it + 1, st ^ 1);
        const int tq = t_first + it % nt;
        step(tq < u_first || tq >= u_end, it, st);
        wait_all_loads();
        __syncthreads();
    }

    // the pair's two partial sums: the second wave leaves its accumulators in
    // LDS (lane-interleaved), the first adds them in
    float *red = pair < 2 ? reinterpret_cast<float *>(kvs) + pair * (D * 64)
                          : reinterpret_cast<float *>(smem) + (pair - 2) * (D * 64);
    if (half == 1) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                red[((db * 16 + e) * 2) * 64 + lane] = dkacc[db][e];
                red[((db * 16 + e) * 2 + 1) * 64 + lane] = dvacc[db][e];
            }
    }
    __syncthreads();
    if (half == 1 || key >= p.Lk) return;
    const int64_t kb = (int64_t)b * bp.dk_sb + (int64_t)hk * bp.dk_sh + (int64_t)key * bp.dk_sl;
    const int64_t vb = (int64_t)b * bp.dv_sb + (int64_t)hk * bp.dv_sh + (int64_t)key * bp.dv_sl;
    const float sc = p.scale;
    // one d block at a time (a compiler barrier between blocks keeps the
    // partner's values from being read all at once beside the accumulators)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            dkacc[db][e] += red[((db * 16 + e) * 2) * 64 + lane];
            dvacc[db][e] += red[((db * 16 + e) * 2 + 1) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = db * 32 + i * 8 + hh * 4;
            store4(bp.dk, kb + d0, bp.grad_bf16, dkacc[db][4 * i] * sc, dkacc[db][4 * i + 1] * sc,
                   dkacc[db][4 * i + 2] * sc, dkacc[db][4 * i + 3] * sc);
            store4(bp.dv, vb + d0, bp.grad_bf16, dvacc[db][4 * i], dvacc[db][4 * i + 1], dvacc[db][4 * i + 2],
                   dvacc[db][4 * i + 3]);
        }
        asm volatile("" ::: "memory");
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
        // d = 128: the paired-wave form (128 keys per workgroup as well), for
        // every score modifier
        if constexpr (D == 128)
            hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, BIAS>), dim3((unsigned)kv_blocks), dim3(512), 0, stream, p);
        else
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
