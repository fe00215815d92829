// prefill_bf16.hip -- fused attention forward for bf16 Q/K/V on gfx950.
//
// One workgroup owns a tile of BR = 32 * NW query rows of one (b, h) (NW = 4
// or 8 waves, chosen per problem, see prefill_waves) and rolls over the keys
// in tiles of BC = 64 (the rolling update of
// "Neptune论文浅读" section 5; the same three-level loop as the kernel in the
// CANN FlashAttention post: query tile outside, K/V tiles inside, on-chip
// compute innermost).  Per K/V tile and per wave (32 query rows):
//
//   1. S^T = K Q^T on the matrix cores (32x32x16 bf16, fp32 accumulate).  Q
//      stays in registers for the whole loop; K comes from LDS.  Keys are
//      placed in the matrix-core rows with the perm32 shuffle so that each lane
//      ends up holding 32 scores of ONE query row (its column), in exactly the
//      order the P V product wants them.
//   2. score modifier: without a bias the scale is folded into the exponent
//      (one FMA per score: t = s * scale * log2(e) - m); with a bias the score
//      is formed first, t = s * scale * log2(e) + bias * log2(e); the soft cap
//      c tanh(t / c) is a polynomial in s where every score of the tile is
//      within |t| <= c / 2, else formed through 2^(2t / c).  The causal
//      mask and the key tail are applied only on tiles that cross them (a
//      separate code path, so full tiles carry no compare at all).
//   3. rolling update (Neptune notes section 3 and section 4): the row max
//      over the tile needs one cross-half swap (v_permlane32_swap); when the
//      max grows, the running sum and the output are repaired by
//      2^(m_old - m_new).  The repair is taken lazily: it runs only when some
//      row's max has grown by more than TAU = 8 (a factor 256), which keeps
//      every exponent <= 2^8 and is exact in real arithmetic because the final
//      normalisation uses the same reference m.  Without a score modifier the
//      tile max is formed only when needed: the weights of step 4 are taken
//      against the running m first and kept if none exceeds 2^8.
//   4. P = 2^(t - m) in fp32; the row sum l accumulates the fp32 values (each
//      lane keeps a partial over its half of the keys; the halves are added
//      once at the end); P is packed to bf16 in registers.
//   5. O^T += V^T P^T on the matrix cores.  V stays in its natural [key][d]
//      layout in LDS and the A operand (8 consecutive keys of one d per lane)
//      is gathered with the transposing LDS read ds_read_b64_tr_b16; P^T comes
//      straight from registers.  Each lane's output accumulators all belong to
//      its own query row, so the repair in step 3 is lane-local.
//
// K/V tiles are double-buffered: the buffer loads for tile t+1 are issued
// before the matrix work on tile t and written to the other LDS buffer after
// it (the DMA/compute overlap described in the CANN post), one barrier per
// tile.  Buffer loads carry the key range in their descriptor, so rows past
// the end of K/V read as zero without any branch.  Causal tiles above the
// diagonal are never loaded; a wave whose rows are all above a tile's keys
// skips its matrix work.  Key tiles ascend, except for the causal biases that
// peak at the diagonal (folded ALiBi, tiled dense bias), which descend from
// it.  Workgroups are ordered so that each XCD (which has its own L2) works
// through whole heads, heaviest query tiles first.
// Epilogue: O = O / l, LSE = m ln 2 + ln l; a row with no visible key gets
// O = 0 and LSE = -inf.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr float kTau = 8.0f;
constexpr float kTauPow = 256.0f;   // 2^kTau

template <int D>
struct TileCfg {
    static constexpr int BC = 64;          // keys per tile
    static constexpr int RB = 2 * D;       // bytes per K/V row in LDS (no padding)
    static constexpr int CH = D / 8;       // 16-byte chunks per row
    static constexpr int RP = 256 / RB;    // rows per 256-byte span of the 64 LDS banks
    static constexpr int TILE = BC * RB;   // bytes of one K or V tile
    static constexpr int KS = D / 16;      // k-steps of Q K^T
    static constexpr int DB = D / 32;      // 32-row blocks of O^T
    // XOR swizzles of the 16-byte chunks of a row (rows stay unpadded so that
    // the direct global->LDS loads can fill them):
    //  K: 16 lanes reading one logical chunk of 16 consecutive rows hit 16
    //     different bank groups;
    //  V: the transposing reads of 4 rows x 4 chunks hit 16 different groups.
    static __device__ __forceinline__ int swz_k(int row) { return (row / RP) % CH; }
    static __device__ __forceinline__ int swz_v(int row) { return 4 * ((row / RP) % (4 / RP)); }
};

// Score modifier, rolling update, P and O^T += V^T P^T for one 64-key tile.
// lk / lv: LDS tiles; this lane's K operand chunk for k-step ks is at byte
// kbase ^ (ks << 5) (+32 rows per key block), its transposing-read word for
// d-block db at vbase ^ (db << 6) (+ key rows).
// Byte offset in an LDS bias tile of 16-byte chunk c (keys 8c .. 8c+7 of the
// tile) of row R: chunks are XOR-swizzled by the row so that the 16 rows read
// by 16 lanes at once hit 16 different bank groups.
__device__ __forceinline__ int bias_lds_off(int R, int c) { return (R * 8 + (c ^ ((R >> 1) & 7))) * 16; }

template <int D, int BIAS, bool MASK>
__device__ __forceinline__ void process_tile(const FwdParams &p, const char *lk, const char *lv, const char *lb,
                                             int kbase, int vbase,
                                             const u32x4 (&qreg)[D / 16], f32x16 (&oacc)[D / 32],
                                             float &m_run, float &l_run, int kt0, int qrow, int qpos,
                                             int jmin, int jmax, float slope_l2, int b, int h, int lane) {
    using C = TileCfg<D>;
    constexpr bool AC = (BIAS == kBiasAlibiCausal);
    // CE: the soft cap for caps up to 64 with a positive scale: the capped
    // score is increasing in the raw one, so a tile max is taken on raw scores
    // and capped once, and P is formed from the raw score directly, as
    // 2^(s P(s^2) - m) (the polynomial form, on unmasked tiles whose raw scores
    // all lie within cap_s0) or 2^(c - m - 2c / (2^(s * scale * k2) + 1))
    constexpr bool CE = (BIAS == kBiasNoneCapExp);
    constexpr bool FOLD = (BIAS == kBiasNone) || AC || CE;
    constexpr int BK = bias_base(BIAS);
    constexpr bool CAP = bias_cap(BIAS);
    const int hh = lane >> 5;

    // Causal ALiBi: every key j a row sees lies at or before the row's
    // position, so the bias -slope |pos - j| is slope (j - P0) - slope (pos -
    // P0) for any P0.  The second term is constant along the row and leaves
    // the softmax unchanged (the epilogue takes it out of the LSE); the first
    // depends on the key only, and one more matrix-core product adds it to
    // every row's raw score: the A operand holds v_j = (slope / scale) (j -
    // P0) split into three bf16 parts (hi + mid + lo = v_j to fp32 precision)
    // in k = 0..2 of key row j, the B operand ones in k = 0..2.  P0 is the
    // position of the wave's first row, which keeps v_j small for the keys
    // near the rows' positions (the ones that carry the weight): the fp32
    // score then carries an error of about 2^-23 slope log2(e) |j - P0|, at
    // most ~1e-4 (log2 units) over the keys with weight for slopes up to 64.
    // slope_l2 carries slope / scale for this kind.
    u32x4 ext_a[2], ext_b;
    if constexpr (AC) {
        // qpos - wrow is the workgroup's first position; the wave's is 32 wv past it
        const int wrow = ((int)threadIdx.x >> 6) * 32 + (lane & 31);   // the row's index in the workgroup
        const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
        const int jrel = kt0 + perm32(lane & 31) - (qpos - wrow) - 32 * wv;   // key of A row r minus P0
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const float v = slope_l2 * (float)(jrel + kb * 32);
            const uint32_t hi = pack_bf16x2(v, 0.f) & 0xffffu;
            const float r1 = v - __uint_as_float(hi << 16);
            const uint32_t mid = pack_bf16x2(r1, 0.f) & 0xffffu;
            const float r2 = r1 - __uint_as_float(mid << 16);
            const uint32_t lo = pack_bf16x2(r2, 0.f) & 0xffffu;
            ext_a[kb] = hh == 0 ? u32x4{hi | (mid << 16), lo, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
        }
        ext_b = hh == 0 ? u32x4{0x3f803f80u, 0x3f80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
    }

    // 1. S^T = K Q^T, the two 32-key blocks interleaved (two accumulation
    //    chains); the K operand reads run ahead of the matrix core (below).
    //    A lambda: the rare path of step 3 recomputes the scores from the K
    //    tile, which is still in LDS, rather than keeping them live.
    f32x16 s[2];
    auto qk = [&]() {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                s[kb] = mfma32(as_bf16x8(load16(lk + ((kbase ^ (ks << 5)) + kb * 32 * C::RB))), as_bf16x8(qreg[ks]), s[kb]);
        // schedule: operand reads ahead of the matrix core. For D = 128 two reads in flight ahead of
        // each product measured fastest (1 to 2% over 4, 6, 8 or 12; 1 spills); for D = 64 the
        // choice made no measurable difference and all eight are issued up front.
        constexpr int RA = C::KS == 8 ? 2 : 2 * C::KS;
        __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
#pragma unroll
        for (int i = 0; i < 2 * C::KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < 2 * C::KS - RA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (AC) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(as_bf16x8(ext_a[kb]), as_bf16x8(ext_b), s[kb]);
        }
    };

    // 2. score modifier
    const float sc = p.scale_log2;
    // tiled dense bias: this lane's values come 8 consecutive keys (one
    // 16-byte chunk of its row) at a time; element e of block kb is key
    // 32 kb + 16 (e / 8) + 8 hh + e % 8 of the tile, in chunk 4 kb + 2 (e / 8) + hh
    // chunk c of the lane's row R sits at bias_lds_off(R, c) = bbase ^ (c << 4),
    // bbase = bias_lds_off(R, 0); bbase is made opaque here so that the four
    // chunk addresses are formed per tile instead of being held in registers
    // across the loop
    int bbase = 0;
    if constexpr (BK == kBiasDenseBf16Tiled) {
        bbase = bias_lds_off(((int)threadIdx.x >> 6) * 32 + (lane & 31), 0);
        asm volatile("" : "+v"(bbase));
    }
    u32x4 bch{};
    // ALiBi distance qpos - j = dbase - (a compile-time offset of the element)
    const float dbase = (float)(qpos - kt0 - hh * 8);
    // the score modifier in place (log2 units; raw scores where the scale is
    // folded into the exponent, natural units with the tiled dense bias),
    // masked keys set to -inf; returns this lane's maximum
    auto modify = [&]() {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = kt0 + kb * 32 + (e >> 3) * 16 + hh * 8 + (e & 7);
                if (BK == kBiasDenseBf16Tiled && (e & 7) == 0)
                    bch = load16(lb + (bbase ^ ((4 * kb + 2 * (e >> 3) + hh) << 4)));
                float x = s[kb][e];
                if (BK == kBiasDenseBf16Tiled) {
                    // natural units, scale and bias in one FMA; the exponent
                    // takes log2(e)
                    const uint32_t wv = bch[(e & 7) >> 1];
                    const float bv = __uint_as_float((e & 1) ? (wv & 0xffff0000u) : (wv << 16));
                    x = fmaf(x, p.scale, bv);
                } else if (!FOLD) {
                    x *= sc;
                    if (CAP) {   // in log2 units
                        if constexpr (BIAS == kBiasNoneCapExp)
                            x = soft_cap_exp(x, p.cap_l2, p.cap_k);
                        else
                            x = soft_cap(x, p.cap_l2, p.cap_k, p.cap_inv);
                    }
                    if (BK == kBiasAlibi) {
                        x = fmaf(-slope_l2, fabsf(dbase - (float)(kb * 32 + (e >> 3) * 16 + (e & 7))), x);
                    } else if (BK == kBiasDenseF32 || BK == kBiasDenseBf16) {
                        const int bi = min(qrow, p.Lq - 1);
                        const int bj = min(j, p.Lk - 1);
                        const int64_t idx = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh +
                                            (int64_t)bi * p.bias_si + (int64_t)bj * p.bias_sj;
                        float bv;
                        if (BK == kBiasDenseF32)
                            bv = static_cast<const float *>(p.bias)[idx];
                        else
                            bv = bf16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[idx]);
                        x = fmaf(bv, kLog2e, x);
                    }
                }
                if (MASK && (j < jmin || j > jmax)) x = -INFINITY;
                s[kb][e] = x;
                mx = fmaxf(mx, x);
            }
        }
        return mx;
    };

    // weights P = 2^(t - m_use) in fp32, packed to bf16, t the score in log2
    // units (formed here from the units modify leaves); returns this lane's sum
    uint32_t pk[2][8];
    auto weights = [&](float m_use) {
        float lt = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                float p0, p1;
                if constexpr (CE) {
                    // capped - m = (c - m) - 2c / (2^(s * sc * k2) + 1); a masked score
                    // (-inf) would give 2^(-c - m), so it is zeroed explicitly
                    const float cm = p.cap_l2 - m_use, c2 = -2.f * p.cap_l2, u = sc * p.cap_k;
                    p0 = exp2_fast(fmaf(c2, __builtin_amdgcn_rcpf(exp2_fast(s[kb][e] * u) + 1.f), cm));
                    p1 = exp2_fast(fmaf(c2, __builtin_amdgcn_rcpf(exp2_fast(s[kb][e + 1] * u) + 1.f), cm));
                    if (MASK) {
                        if (s[kb][e] == -INFINITY) p0 = 0.f;
                        if (s[kb][e + 1] == -INFINITY) p1 = 0.f;
                    }
                } else if (FOLD) {
                    p0 = exp2_fast(fmaf(s[kb][e], sc, -m_use));
                    p1 = exp2_fast(fmaf(s[kb][e + 1], sc, -m_use));
                } else if (BK == kBiasDenseBf16Tiled) {
                    p0 = exp2_fast(fmaf(s[kb][e], kLog2e, -m_use));
                    p1 = exp2_fast(fmaf(s[kb][e + 1], kLog2e, -m_use));
                } else {
                    p0 = exp2_fast(s[kb][e] - m_use);
                    p1 = exp2_fast(s[kb][e + 1] - m_use);
                }
                lt += p0 + p1;
                pk[kb][e >> 1] = pack_bf16x2(p0, p1);
            }
        }
        return lt;
    };

    // the same weights with the cap as a polynomial in the raw score (CE
    // only, every raw score of the wave within |s| <= cap_s0): one
    // transcendental per score instead of three
    auto weights_poly = [&](float m_use) {
        float lt = 0.f;
        const float q0 = p.cap_q[0], q1 = p.cap_q[1], q2 = p.cap_q[2], q3 = p.cap_q[3];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float s0 = s[kb][e], s1 = s[kb][e + 1];
                const float w0 = s0 * s0, w1 = s1 * s1;
                const float c0 = fmaf(fmaf(fmaf(q3, w0, q2), w0, q1), w0, q0);
                const float c1 = fmaf(fmaf(fmaf(q3, w1, q2), w1, q1), w1, q0);
                const float p0 = exp2_fast(fmaf(s0, c0, -m_use));
                const float p1 = exp2_fast(fmaf(s1, c1, -m_use));
                lt += p0 + p1;
                pk[kb][e >> 1] = pack_bf16x2(p0, p1);
            }
        }
        return lt;
    };

    // lazy repair of l and O to the reference m_new (per lane; m_new >= m_run)
    auto repair = [&](float m_new) {
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        l_run *= alpha;
        // in place, so the accumulators keep their registers across this rarely
        // taken branch (no copies on the common path)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(oacc[db][e]) : "v"(alpha));
        m_run = m_new;
    };

    qk();
    if constexpr (BIAS == kBiasNone || CE) {
        // 3./4. Without a score modifier, or with the exp-form soft cap, the
        // weights are formed against the running reference m_run without the
        // tile's maximum.  If every weight of the wave is at
        // most 2^TAU (checked through this lane's sum, whose terms are >= 0)
        // they are kept: the reference may trail the true maximum by up to
        // TAU, as with the lazy repair.  Otherwise (the first tile, where
        // m_run = -inf gives inf or NaN weights, or a maximum that grew by
        // more than TAU) the tile's maximum is taken, l and O are repaired to
        // it when it grew, and the weights are formed again.  (With the folded
        // ALiBi bias the maximum grows by slope * 64 keys per tile, so the
        // other kinds take the maximum first.)
        if constexpr (MASK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = kt0 + kb * 32 + (e >> 3) * 16 + hh * 8 + (e & 7);
                    if (j < jmin || j > jmax) s[kb][e] = -INFINITY;
                }
        }
        float lt;
        if constexpr (CE && !MASK) {
            float amax = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(s[kb][e]));
            lt = __any(amax > p.cap_s0) ? weights(m_run) : weights_poly(m_run);
        } else {
            lt = weights(m_run);
        }
        if (__any(!(lt <= kTauPow))) {
            qk();
            float mx = xor32_max(modify()) * sc;   // sc > 0: max commutes with the scaling
            if constexpr (CE) {   // and with the cap, which is increasing
                if (mx != -INFINITY) mx = soft_cap_exp(mx, p.cap_l2, p.cap_k);
            }
            if (__any(mx > m_run)) repair(fmaxf(m_run, mx));
            lt = weights((m_run == -INFINITY) ? 0.f : m_run);
        }
        l_run += lt;
    } else {
        float mx = xor32_max(modify());
        if (FOLD) mx *= sc;   // sc > 0: max commutes with the scaling
        if (BK == kBiasDenseBf16Tiled) mx *= kLog2e;
        // 3. lazy repair of l and O when the max has grown by more than TAU
        if (__any(mx > m_run + kTau)) repair(fmaxf(m_run, mx));
        // 4. P = 2^(t - m) in fp32, summed in fp32, packed to bf16
        l_run += weights((m_run == -INFINITY) ? 0.f : m_run);
    }

    // 5. O^T += V^T P^T: A operand = 8 keys of one d per lane, by two
    //    transposing reads of 4 keys each (rows +0..3 and +4..7)
#pragma unroll
    for (int kk = 0; kk < C::BC / 16; ++kk) {
        const int kb = kk >> 1;
        const int half = kk & 1;
        const bf16x8 bop = as_bf16x8(u32x4{pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2],
                                           pk[kb][4 * half + 3]});
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(lv + (vbase ^ (db << 6)) + kk * 16 * C::RB));
            const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t *>(lv + (vbase ^ (db << 6)) + (kk * 16 + 4) * C::RB));
            oacc[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), bop, oacc[db]);
        }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * 4, 1);
#pragma unroll
    for (int i = 0; i < C::BC / 16 * C::DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (i < C::BC / 16 * C::DB - 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
}

// One tile of the rolling update for this wave.  Unmasked tiles lie below the
// diagonal of every row of the workgroup and inside the keys.  On masked
// tiles a wave whose rows are all above the tile's keys skips the work.
template <int D, int BIAS, bool MASK>
__device__ __forceinline__ void tile_step(const FwdParams &p, const char *lk, const char *lv, const char *lb,
                                          int kbase, int vbase,
                                          const u32x4 (&qreg)[D / 16], f32x16 (&oacc)[D / 32], float &m_run,
                                          float &l_run, int kt0, int wrow0, int wjmin, int wjmax, int qrow, int qpos,
                                          int jmin, int jmax, float slope_l2, int b, int h, int lane) {
    if (MASK && !((wrow0 < p.Lq) && kt0 <= wjmax && kt0 + TileCfg<D>::BC - 1 >= wjmin)) return;
    process_tile<D, BIAS, MASK>(p, lk, lv, lb, kbase, vbase, qreg, oacc, m_run, l_run, kt0, qrow, qpos, jmin, jmax,
                                slope_l2, b, h, lane);
}

// Direct global->LDS loads of K/V tile T_ into the LDS tile arrays KOFF_ /
// VOFF_ (and, with a tiled bias, of the workgroup's rows of bias columns
// [64 T_, 64 T_ + 64) into BOFF_): lane
// fills LDS bytes [i*T*16 + wave*1024 + 16*lane, +16) of each tile from the
// byte offsets kgoff / vgoff (+ round i's rows) inside the tile.  The whole
// offset goes in the vector offset, which the hardware checks against the
// descriptor's range (the scalar offset is not checked), so rows past the end
// of K/V read as zero (with overlapping rows they read valid data, which the
// mask discards).  A macro, because the
// buffer-to-LDS builtins have to appear in the kernel body itself.
#define ATTN_ISSUE_TILE_LOADS(T_, KOFF_, VOFF_, BOFF_)                                                          \
    do {                                                                                                        \
        const int j0_ = (T_) * BC;                                                                              \
        if constexpr (TB) {                                                                                     \
            _Pragma("unroll") for (int i_ = 0; i_ < NB; ++i_) {                                                 \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                       \
                    rb, (__attribute__((address_space(3))) void *)((BOFF_) + i_ * T * 16 + wave * 1024), 16,     \
                    (int)(bgoff + (uint32_t)i_ * bround + (uint32_t)j0_ * 2u), 0, 0, 0);                       \
            }                                                                                                   \
        }                                                                                                       \
        const int nvalid_ = min(BC, p.Lk - j0_);                                                                \
        const __amdgpu_buffer_rsrc_t rk_ =                                                                      \
            make_rsrc(kp + (int64_t)j0_ * p.k_sl, (uint32_t)(nvalid_ - 1) * kl_bytes + D * 2);                  \
        const __amdgpu_buffer_rsrc_t rv_ =                                                                      \
            make_rsrc(vp + (int64_t)j0_ * p.v_sl, (uint32_t)(nvalid_ - 1) * vl_bytes + D * 2);                  \
        _Pragma("unroll") for (int i_ = 0; i_ < NC; ++i_) {                                                     \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                           \
                rk_, (__attribute__((address_space(3))) void *)((KOFF_) + i_ * T * 16 + wave * 1024), 16,        \
                (int)(kgoff + (uint32_t)(i_ * RROWS) * kl_bytes), 0, 0, 0);                                     \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                           \
                rv_, (__attribute__((address_space(3))) void *)((VOFF_) + i_ * T * 16 + wave * 1024), 16,        \
                (int)(vgoff + (uint32_t)(i_ * RROWS) * vl_bytes), 0, 0, 0);                                     \
        }                                                                                                       \
    } while (0)

// The body of both prefill kernels.  PART: key chunk blockIdx.y of p.chunk
// keys (a multiple of the key tile), written as split-K partials (O not
// normalised, m in natural units, l) for the combine instead of O and LSE.
template <int D, int NW, int BIAS, bool OUT_BF16, bool PART>
__device__ __forceinline__ void prefill_body(const FwdParams &p) {
    using C = TileCfg<D>;
    constexpr int BR = 32 * NW;          // query rows per workgroup
    constexpr int BC = C::BC;
    constexpr int T = NW * 64;           // threads
    constexpr int NC = C::TILE / (T * 16);   // 16-byte direct loads per thread per tensor per tile
    static_assert(NC >= 1 && C::TILE == NC * T * 16, "tile does not split evenly");

    // two K and two V tiles, as separate objects so that the compiler can tell
    // the tile being filled by the direct loads from the tiles being read
    // (with one array it waits for the loads before every LDS read)
    __shared__ __attribute__((aligned(1024))) char lds_k0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_k1[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v1[C::TILE];
    // tiled dense bias: the workgroup's BR rows x 64 keys of bf16 per tile
    constexpr bool TB = (bias_base(BIAS) == kBiasDenseBf16Tiled);
    constexpr int BTILE = TB ? BR * BC * 2 : 16;
    constexpr int NB = BTILE / (T * 16);     // 16-byte direct loads per thread per bias tile
    static_assert(!TB || NB * T * 16 == BTILE, "bias tile does not split evenly");
    __shared__ __attribute__((aligned(TB ? 1024 : 16))) char lds_b0[BTILE];
    __shared__ __attribute__((aligned(TB ? 1024 : 16))) char lds_b1[BTILE];

    // work item: XCD-contiguous ranges of heads; under a causal mask the last
    // query tile sees the most keys and goes first
    const int nqt = (p.Lq + BR - 1) / BR;
    const WorkItem wi = xcd_work_item(nqt, p.causal && !p.window, p.num_xcds);
    const int bh = wi.head;
    const int qt = p.causal ? nqt - 1 - wi.rank : wi.rank;
    // a tiled bias shared by the batch: the batch elements of one head are
    // neighbours in the work order, so they run on one XCD at the same time and
    // the second reads each bias tile from that XCD's L2
    const bool bfirst = TB && p.bias_sb == 0 && p.B > 1;
    const int b = bfirst ? bh % p.B : bh / p.Hq;
    const int h = bfirst ? bh / p.B : bh - b * p.Hq;
    const int hk = h / p.G;
    const int q0 = qt * BR;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches on it stay scalar
    const int lane = tid & 63;
    const int r = lane & 31;
    const int hh = lane >> 5;
    const int off = p.Lk - p.Lq;
    const int qrow = q0 + wave * 32 + r;
    const int qpos = qrow + off;
    const int wrow0 = q0 + wave * 32;
    const int wrow1 = min(wrow0 + 31, p.Lq - 1);
    // visible keys: this lane's row, this wave's rows, the workgroup's rows
    int jmin, jmax, wjmin, wjmax, unused;
    key_range(p, qpos, jmin, jmax);
    key_range(p, wrow0 + off, wjmin, unused);
    key_range(p, wrow1 + off, unused, wjmax);
    const int rlast = min(q0 + BR, p.Lq) - 1;
    int gjmin0, gjmax0, gjmin1, gjmax1;
    key_range(p, q0 + off, gjmin0, gjmax0);
    key_range(p, rlast + off, gjmin1, gjmax1);
    // tiles [t_first, t_end) hold every key some row sees; tiles
    // [u_first, u_end) are visible in full to every row (no mask)
    int t_first = 0, t_end = 0;
    if (rlast >= q0 && gjmax1 >= gjmin0) {
        t_first = gjmin0 / BC;
        t_end = gjmax1 / BC + 1;
    }
    if constexpr (PART) {
        const int c0 = (int)blockIdx.y * (p.chunk / BC);
        t_first = max(t_first, c0);
        t_end = min(t_end, c0 + p.chunk / BC);
    }
    const int u_first = max(t_first, (gjmin1 + BC - 1) / BC);
    const int u_end = min(t_end, gjmax0 >= 0 ? (gjmax0 + 1) / BC : 0);

    const uint16_t *qp = static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    const uint16_t *kp = static_cast<const uint16_t *>(p.k) + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vp = static_cast<const uint16_t *>(p.v) + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;

    // Q fragment: lane holds row qrow, d = 16*ks + 8*hh .. +7 for each k-step.
    u32x4 qreg[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = u32x4{0, 0, 0, 0};
    if (qrow < p.Lq) {
        const uint16_t *qr = qp + (int64_t)qrow * p.q_sl + hh * 8;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = load16(qr + ks * 16);
    }

    float slope_l2 = 0.f;
    if (bias_base(BIAS) == kBiasAlibi) slope_l2 = p.slopes[h] * kLog2e;
    if (BIAS == kBiasAlibiCausal) slope_l2 = p.slopes[h] / p.scale;   // v_j per key of distance

    // per-lane LDS byte offsets: K operand of k-step ks at kbase ^ (ks << 5)
    // (+32 rows per key block); V transposing read of d-block db at
    // vbase ^ (db << 6) (+ key rows).  The XOR only touches the swizzled chunk
    // bits of the row.
    const int kbase = r * C::RB + ((hh ^ C::swz_k(r)) << 4);
    int vbase;
    {
        const int g = lane >> 4, sl = lane & 15;
        const int vrow = (g >> 1) * 8 + (sl >> 2);
        const int e = (g & 1) * 16 + 4 * (sl & 3);
        vbase = vrow * C::RB + (((e >> 3) ^ C::swz_v(vrow)) * 16) + (e & 7) * 2;
    }
    // direct loads: round i fills LDS bytes [i*T*16 + wave*1024 + 16*lane, +16)
    // of a tile; rounds differ by T*16/RB whole rows, so the per-lane source
    // offset is the same and the round's row offset goes in the scalar offset
    constexpr int RROWS = T * 16 / C::RB;
    const uint32_t kl_bytes = (uint32_t)p.k_sl * 2u;
    const uint32_t vl_bytes = (uint32_t)p.v_sl * 2u;
    uint32_t kgoff, vgoff;
    {
        const int pos = wave * 1024 + lane * 16;
        const int row = pos / C::RB;
        const int pc = (pos % C::RB) / 16;
        const int key = (row & ~31) | perm32(row & 31);
        kgoff = (uint32_t)key * kl_bytes + (uint32_t)((pc ^ C::swz_k(row)) * 16);
        vgoff = (uint32_t)row * vl_bytes + (uint32_t)((pc ^ C::swz_v(row)) * 16);
    }
    // tiled bias: round i fills slot s = i*T + tid of the tile (row s / 8,
    // position s % 8), which holds chunk (s % 8) ^ swizzle(row) of that row.
    // Rounds are T / 8 rows apart (a multiple of 16, so the swizzle is the
    // same in every round).  Rows past the last query and keys past the
    // plane's end lie outside the descriptor's range and read as zero (those
    // rows' results are not stored; keys past Lk are masked).
    static_assert(!TB || (T / 8) % 16 == 0, "bias rounds must keep the swizzle");
    const __amdgpu_buffer_rsrc_t rb =
        TB ? make_rsrc(static_cast<const uint16_t *>(p.bias) + (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh,
                       p.bias_plane_bytes)
           : make_rsrc(p.k, 0u);
    const uint32_t bround = TB ? (uint32_t)(T / 8) * (uint32_t)p.bias_si * 2u : 0u;   // bytes between rounds
    uint32_t bgoff = 0;
    if constexpr (TB) {
        const int R = q0 + (tid >> 3);
        bgoff = (uint32_t)R * (uint32_t)p.bias_si * 2u + (uint32_t)(((tid & 7) ^ ((tid >> 4) & 7)) * 16);
    }

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY;   // running max, log2 units
    float l_run = 0.f;         // running sum over this lane's half of the keys


    // Visiting order.  Keys ascend (a head's query tiles then start on the
    // same K/V tiles, which stay in L2), except with the folded causal ALiBi
    // bias and the tiled dense bias.  The folded bias makes the scores grow
    // with the key (it is largest at the row's own position), so ascending
    // keys would raise the running maximum by about slope * 64 keys on every
    // tile and repair l and O each time; descending from the diagonal, the
    // first tile holds the largest biases and later tiles rarely move the
    // maximum.  Under a causal mask dense position biases mostly share that
    // shape (largest near the diagonal), so the tiled dense bias descends
    // too there (kBiasDenseBf16TiledDesc); a bias without it pays the L2
    // effect instead (1-2%).  Step n handles tile t_end - 1 - n there.
    // Step n's tile sits in LDS buffer n & 1.  Masked tiles (the window's
    // left edge, the causal diagonal band, the key tail) take the generic
    // step; the unmasked middle runs two tiles per trip so that each LDS
    // buffer's address is a constant.
    constexpr bool REV = (BIAS == kBiasAlibiCausal) || (BIAS == kBiasDenseBf16TiledDesc);
    if (t_end > t_first) {
        ATTN_ISSUE_TILE_LOADS(REV ? t_end - 1 : t_first, lds_k0, lds_v0, lds_b0);
        wait_vmem();
        __syncthreads();
    }
#define ATTN_STEP(MASK_, BUF_, T_)                                                                               \
    tile_step<D, BIAS, MASK_>(p, (BUF_) ? lds_k1 : lds_k0, (BUF_) ? lds_v1 : lds_v0, (BUF_) ? lds_b1 : lds_b0,   \
                              kbase, vbase, qreg, oacc,                                                         \
                              m_run, l_run, (T_) * BC, wrow0, wjmin, wjmax, qrow, qpos, jmin, jmax, slope_l2, b, h, \
                              lane)
    // step N_ on tile T_, prefetching tile NEXT_ (if HAS_NEXT_) into the other buffer
#define ATTN_GENERIC_STEP(N_, T_, HAS_NEXT_, NEXT_)                                                            \
    do {                                                                                                        \
        const int tg_ = (T_);                                                                                   \
        const bool masked_ = tg_ < u_first || tg_ >= u_end;                                                     \
        if (((N_) & 1) == 0) {                                                                                  \
            if (HAS_NEXT_) ATTN_ISSUE_TILE_LOADS(NEXT_, lds_k1, lds_v1, lds_b1);                                \
            if (masked_)                                                                                        \
                ATTN_STEP(true, 0, tg_);                                                                        \
            else                                                                                                \
                ATTN_STEP(false, 0, tg_);                                                                       \
        } else {                                                                                                \
            if (HAS_NEXT_) ATTN_ISSUE_TILE_LOADS(NEXT_, lds_k0, lds_v0, lds_b0);                                \
            if (masked_)                                                                                        \
                ATTN_STEP(true, 1, tg_);                                                                        \
            else                                                                                                \
                ATTN_STEP(false, 1, tg_);                                                                       \
        }                                                                                                       \
        wait_vmem();                                                                                            \
        __syncthreads();                                                                                        \
    } while (0)
    if constexpr (REV) {
        // descending: tile t is step t_end - 1 - t
        int t = t_end - 1;
        for (; t >= t_first && !(t < u_end && ((t_end - 1 - t) & 1) == 0); --t)
            ATTN_GENERIC_STEP(t_end - 1 - t, t, t > t_first, t - 1);
        for (; t - 1 >= u_first; t -= 2) {
            ATTN_ISSUE_TILE_LOADS(t - 1, lds_k1, lds_v1, lds_b1);
            ATTN_STEP(false, 0, t);
            wait_vmem();
            __syncthreads();
            if (t - 2 >= t_first) ATTN_ISSUE_TILE_LOADS(t - 2, lds_k0, lds_v0, lds_b0);
            ATTN_STEP(false, 1, t - 1);
            wait_vmem();
            __syncthreads();
        }
        for (; t >= t_first; --t) ATTN_GENERIC_STEP(t_end - 1 - t, t, t > t_first, t - 1);
    } else {
        // ascending: step t - t_first on tile t
        int t = t_first;
        for (; t < t_end && !(t >= u_first && ((t - t_first) & 1) == 0); ++t)
            ATTN_GENERIC_STEP(t - t_first, t, t + 1 < t_end, t + 1);
        for (; t + 1 < u_end; t += 2) {
            ATTN_ISSUE_TILE_LOADS(t + 1, lds_k1, lds_v1, lds_b1);
            ATTN_STEP(false, 0, t);
            wait_vmem();
            __syncthreads();
            if (t + 2 < t_end) ATTN_ISSUE_TILE_LOADS(t + 2, lds_k0, lds_v0, lds_b0);
            ATTN_STEP(false, 1, t + 1);
            wait_vmem();
            __syncthreads();
        }
        for (; t < t_end; ++t) ATTN_GENERIC_STEP(t - t_first, t, t + 1 < t_end, t + 1);
    }
#undef ATTN_GENERIC_STEP
#undef ATTN_STEP

    // epilogue
    const float l_tot = xor32_sum(l_run);
    if constexpr (PART) {
        if (qrow < p.Lq) {
            const int64_t prow = (((int64_t)b * p.Hq + h) * p.Lq + qrow) * p.num_splits + blockIdx.y;
            float *op = p.o_part + prow * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<f32x4 *>(op + db * 32 + i * 8 + hh * 4) =
                        f32x4{oacc[db][4 * i], oacc[db][4 * i + 1], oacc[db][4 * i + 2], oacc[db][4 * i + 3]};
            if (hh == 0) {
                float mp = (m_run == -INFINITY) ? -INFINITY : m_run * kLn2;
                // the folded ALiBi's row constant, as in the LSE of the plain prefill
                if constexpr (BIAS == kBiasAlibiCausal) mp -= p.slopes[h] * (float)r;
                p.m_part[prow] = mp;
                p.l_part[prow] = l_tot;
            }
        }
        return;
    }
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow < p.Lq) {
        const int64_t obase = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)qrow * p.o_sl;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
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
            float lse = (l_tot > 0.f) ? m_run * kLn2 + logf(l_tot) : -INFINITY;
            // the row constant of the folded ALiBi bias: slope (pos - P0), P0 the position
            // of the wave's first row
            if constexpr (BIAS == kBiasAlibiCausal) lse -= p.slopes[h] * (float)r;
            p.lse[((int64_t)b * p.Hq + h) * p.Lq + qrow] = lse;
        }
    }
}

template <int D, int NW, int BIAS, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64, 8 / NW) void prefill_bf16_kernel(FwdParams p) {
    prefill_body<D, NW, BIAS, OUT_BF16, false>(p);
}

// split-K form: grid (query tiles, key chunks), four waves
template <int D, int BIAS>
__global__ __launch_bounds__(256, 2) void prefill_part_kernel(FwdParams p) {
    prefill_body<D, 4, BIAS, false, true>(p);
}

template <int D, int BIAS>
hipError_t launch_prefill_part_t(const FwdParams &p, hipStream_t stream) {
    const int64_t nqt = (p.Lq + 127) / 128;
    const int64_t blocks = nqt * (int64_t)p.B * p.Hq;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff || p.num_splits < 1 || p.num_splits > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_part_kernel<D, BIAS>), dim3((unsigned)blocks, (unsigned)p.num_splits), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_part_d(const FwdParams &p, hipStream_t stream) {
    const int kind = (p.bias_kind == kBiasNone && !(p.scale_log2 > 0.f)) ? kBiasNoneScaled : p.bias_kind;
    switch (kind) {
        case kBiasNone: return launch_prefill_part_t<D, kBiasNone>(p, stream);
        case kBiasNoneScaled: return launch_prefill_part_t<D, kBiasNoneScaled>(p, stream);
        case kBiasAlibi:
            if (p.causal && p.scale > 0.f) {   // the folded form, as in the plain prefill
                FwdParams pa = p;
                pa.bias_kind = kBiasAlibiCausal;
                return launch_prefill_part_t<D, kBiasAlibiCausal>(pa, stream);
            }
            return launch_prefill_part_t<D, kBiasAlibi>(p, stream);
        case kBiasDenseF32: return launch_prefill_part_t<D, kBiasDenseF32>(p, stream);
        case kBiasDenseBf16: return launch_prefill_part_t<D, kBiasDenseBf16>(p, stream);
        case kBiasNoneCap:
            if (p.softcap <= 64.f && p.scale > 0.f) return launch_prefill_part_t<D, kBiasNoneCapExp>(p, stream);
            return launch_prefill_part_t<D, kBiasNoneCap>(p, stream);
        case kBiasAlibiCap: return launch_prefill_part_t<D, kBiasAlibiCap>(p, stream);
        case kBiasDenseF32Cap: return launch_prefill_part_t<D, kBiasDenseF32Cap>(p, stream);
        case kBiasDenseBf16Cap: return launch_prefill_part_t<D, kBiasDenseBf16Cap>(p, stream);
        default: return hipErrorInvalidValue;
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

// Waves per workgroup.  Eight waves (256 query rows; the two waves of a SIMD
// then come from one workgroup) halve the K/V loads per row and the number of
// workgroups, which pays when each row sees many keys; four waves (128 rows;
// the two waves of a SIMD come from two independent workgroups) overlap the
// vector-heavy phases of the two waves better and leave twice as many
// workgroups for short or unbalanced (causal) rows.  Measured on MI355X
// (d = 128): eight waves are faster for causal rows that see 4096 or more
// keys on average (1-6%: causal 8192, 16384, 32768; ALiBi causal 8192) and
// for non-causal rows of 2048 keys or more (1.5-3% at 2048, 4% at 4096, 5%
// at 8192); they are even at about 2048 keys for causal rows and at 1536
// non-causal, and 3-6% slower below that (non-causal 1024; causal 2048,
// whose rows see 1024 keys on average), with the soft cap (2%), and for a
// 4096-key sliding window (1%); with only 16 query rows against 32768 keys
// they are 38% slower (seven of the eight waves idle).
// A grid of fewer 256-row workgroups than CUs leaves CUs idle that the
// 128-row grid would use (B1 H8 Lq 2048 Lk 32768: 0.654 vs 0.483 ms), and
// with one 256-row workgroup per CU the uneven causal tiles finish unevenly
// (causal B1 H8 L8192: 0.192 vs 0.169 ms) unless rows see 8192 keys or more
// (causal B1 H16 Lq 4096 Lk 16384: 0.466 vs 0.477 ms).
int prefill_waves(const FwdParams &p) {
    const int64_t cus = p.num_cus > 0 ? p.num_cus : 256;
    if (p.D != 128 || bias_cap(p.bias_kind) || p.window) return 4;   // the rule was measured at d = 128
    if (p.Lq < 1024) return 4;   // few rows: most waves of a 256-row tile would idle (Lq = 16: 678 vs 490 us)
    const int64_t avg_keys = p.causal ? (int64_t)p.Lk - ((int64_t)p.Lq - 1) / 2 : (int64_t)p.Lk;
    if (avg_keys < (p.causal ? 4096 : 2048)) return 4;
    const int64_t blocks8 = (int64_t)p.B * p.Hq * (((int64_t)p.Lq + 255) / 256);
    if (blocks8 < cus) return 4;
    if (p.causal && blocks8 < 2 * cus && avg_keys < 8192) return 4;
    return 8;
}

// A bf16 dense bias can be loaded a tile at a time with the K/V tiles when its
// keys are contiguous and every row starts 16-byte aligned, and one (b, h)
// plane of it spans less than 4 GiB (the 32-bit range of a buffer load).
bool bias_tiles_fit(const FwdParams &p) {
    if (p.bias_sj != 1 || p.Lq < 1 || p.Lk < 1) return false;
    if ((reinterpret_cast<uintptr_t>(p.bias) & 15u) || (p.bias_si * 2) % 16 || (p.bias_sb * 2) % 16 ||
        (p.bias_sh * 2) % 16)
        return false;
    // the offsets of the last workgroup's rows (up to 255 past the last query)
    // and keys stay below 2^32 as well
    const int64_t plane = (((int64_t)p.Lq - 1) * p.bias_si + p.Lk) * 2;
    const int64_t reach = ((int64_t)p.Lq + 256) * p.bias_si * 2 + ((int64_t)p.Lk + 64) * 2;
    return p.bias_si >= p.Lk && plane > 0 && reach < ((int64_t)1 << 32);
}

template <int D, int NW>
hipError_t launch_prefill_k(const FwdParams &p, int kind, hipStream_t stream) {
    switch (kind) {
        case kBiasDenseBf16Tiled:
            if constexpr (D == 128 && NW == 8) return launch_prefill_t<D, NW, kBiasDenseBf16Tiled>(p, stream);
            return hipErrorInvalidValue;
        case kBiasDenseBf16TiledDesc:
            if constexpr (D == 128 && NW == 8) return launch_prefill_t<D, NW, kBiasDenseBf16TiledDesc>(p, stream);
            return hipErrorInvalidValue;
        case kBiasAlibiCausal: return launch_prefill_t<D, NW, kBiasAlibiCausal>(p, stream);
        case kBiasNone: return launch_prefill_t<D, NW, kBiasNone>(p, stream);
        case kBiasNoneScaled: return launch_prefill_t<D, NW, kBiasNoneScaled>(p, stream);
        case kBiasAlibi: return launch_prefill_t<D, NW, kBiasAlibi>(p, stream);
        case kBiasDenseF32: return launch_prefill_t<D, NW, kBiasDenseF32>(p, stream);
        case kBiasDenseBf16: return launch_prefill_t<D, NW, kBiasDenseBf16>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_prefill_d(const FwdParams &p, hipStream_t stream) {
    // the folded-scale path needs a positive scale; otherwise form the score explicitly
    const int kind = (p.bias_kind == kBiasNone && !(p.scale_log2 > 0.f)) ? kBiasNoneScaled : p.bias_kind;
    switch (kind) {   // the soft-capped kinds run with four waves only
        case kBiasNoneCap:
            if (p.softcap <= 64.f && p.scale > 0.f) return launch_prefill_t<D, 4, kBiasNoneCapExp>(p, stream);
            return launch_prefill_t<D, 4, kBiasNoneCap>(p, stream);
        case kBiasAlibiCap: return launch_prefill_t<D, 4, kBiasAlibiCap>(p, stream);
        case kBiasDenseF32Cap: return launch_prefill_t<D, 4, kBiasDenseF32Cap>(p, stream);
        case kBiasDenseBf16Cap: return launch_prefill_t<D, 4, kBiasDenseBf16Cap>(p, stream);
        default: break;
    }
    if (kind == kBiasAlibi && p.causal && p.scale > 0.f) {
        // every visible key lies at or before its row: the bias folds into the scores
        FwdParams pa = p;
        pa.bias_kind = kBiasAlibiCausal;
        if (D == 128 && prefill_waves(p) == 8) return launch_prefill_k<D, 8>(pa, kBiasAlibiCausal, stream);
        return launch_prefill_k<D, 4>(pa, kBiasAlibiCausal, stream);
    }
    if (D == 128 && kind == kBiasDenseBf16 && bias_tiles_fit(p)) {
        // the bias tile takes LDS beside K and V: one 8-wave workgroup per CU
        FwdParams pt = p;
        pt.bias_kind = p.causal ? kBiasDenseBf16TiledDesc : kBiasDenseBf16Tiled;
        pt.bias_plane_bytes = (uint32_t)(((int64_t)p.Lq - 1) * p.bias_si + p.Lk) * 2u;
        return launch_prefill_k<D, 8>(pt, pt.bias_kind, stream);
    }
    if (D == 128 && prefill_waves(p) == 8) return launch_prefill_k<D, 8>(p, kind, stream);
    return launch_prefill_k<D, 4>(p, kind, stream);
}

}  // namespace

hipError_t launch_prefill_bf16(const FwdParams &p, hipStream_t stream) {
    if (p.D == 128) return launch_prefill_d<128>(p, stream);
    if (p.D == 64) return launch_prefill_d<64>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_part_bf16(const FwdParams &p, hipStream_t stream) {
    if (p.chunk < 64 || p.chunk % 64 != 0) return hipErrorInvalidValue;   // whole key tiles per chunk
    if (p.D == 128) return launch_prefill_part_d<128>(p, stream);
    if (p.D == 64) return launch_prefill_part_d<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace attn
