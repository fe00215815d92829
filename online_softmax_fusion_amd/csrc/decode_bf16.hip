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
// the workgroup in 32-key blocks, round robin.  Decode reads every K/V byte
// once and does little arithmetic per byte, so the kernel is built to keep as
// many bytes in flight as HBM needs:
//   * each wave streams its own blocks from HBM straight into NST private LDS
//     stages with buffer-to-LDS loads (1 KiB per instruction, whole rows, no
//     staging registers); the loads of block n + NST are issued as soon as
//     block n has been consumed, and a wave waits only for its own oldest
//     stage (a counted vmcnt), never for the other waves;
//   * K rows are stored with the perm32 shuffle and an XOR swizzle of their
//     16-byte chunks; the matrix-core A operand of S^T = K Q^T is one 16-byte
//     LDS read per k-step, free of bank conflicts;
//   * V stays in its natural [key][d] layout and the A operand of
//     O^T += V^T P^T (8 consecutive keys of one d per lane) is gathered with
//     the transposing read ds_read_b64_tr_b16;
//   * the rolling update runs per 32-key block with the lazy repair of the
//     prefill kernel (the reference max may trail the true max by up to
//     TAU = 8 in log2 units; exact in real arithmetic since l and O share it).
// At the end the waves' (m, l, O) are merged through LDS (repair by
// 2^(m_w - M)) and the chunk's un-normalised o, its reference m (natural-log
// units) and l are written to the partial buffers, for the valid rows only.
//
// The buffer-to-LDS loads are issued from inline assembly, which sets M0 (the
// LDS base of the load) itself; nothing else in this file uses M0.  The file
// is compiled with the matrix-core results kept in ordinary VGPRs
// (-amdgpu-mfma-vgpr-form), because with one workgroup per CU the compiler
// would otherwise park the accumulators in AGPRs and copy them every trip.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr float kTau = 8.0f;

// wait until at most N vector memory loads are outstanding (a compiler
// barrier for memory accesses as well)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D>
struct BlockCfg {
    static constexpr int BK = 32;             // keys per block
    static constexpr int RB = 2 * D;          // bytes per K/V row in LDS
    static constexpr int CH = D / 8;          // 16-byte chunks per row
    static constexpr int RP = 256 / RB;       // rows per 256-byte span of the 64 LDS banks
    static constexpr int TB = BK * RB;        // bytes of one K or V block
    static constexpr int NL = TB / 1024;      // 1 KiB wave loads per tensor per block
    static constexpr int STAGE = 2 * TB;      // K block then V block
    static constexpr int KS = D / 16;         // k-steps of K Q^T
    static constexpr int DB = D / 32;         // 32-row blocks of O^T
    static __device__ __forceinline__ int swz_k(int row) { return (row / RP) % CH; }
    static __device__ __forceinline__ int swz_v(int row) { return 4 * ((row / RP) % (4 / RP)); }
};

// wait until at most `later` blocks' loads (issued after the awaited block)
// are outstanding
template <int NLB, int NST>
__device__ __forceinline__ void wait_blocks(int later) {
    if (NST >= 4 && later >= 3) { wait_vmcnt<(NST >= 4 ? 3 * NLB : 0)>(); return; }
    if (NST >= 3 && later >= 2) { wait_vmcnt<(NST >= 3 ? 2 * NLB : 0)>(); return; }
    if (NST >= 2 && later >= 1) { wait_vmcnt<NLB>(); return; }
    wait_vmcnt<0>();
}

// One 32-key block of the rolling update for this wave: S^T = K Q^T from the
// K block at lk, score modifier and mask, lazy repair, P = 2^(t - m), and
// O^T += V^T P^T from the V block at lv.
template <int D, int BIAS>
__device__ __forceinline__ void decode_block(const FwdParams &p, const char *lk, const char *lv, int kbase,
                                             int vbase, const u32x4 (&qreg)[D / 16], f32x16 (&oacc)[D / 32],
                                             float &m_run, float &l_run, int kb0, int k_hi, int qi, int qpos,
                                             int jmin, int jmax, float slope_l2, int b, int h, int lane) {
    using C = BlockCfg<D>;
    constexpr int BK = bias_base(BIAS);
    constexpr bool CAP = bias_cap(BIAS);
    const int hh = lane >> 5;

    // S^T = K Q^T: two accumulation chains over the k-steps
    f32x16 s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < C::KS; ks += 2) {
        s0 = mfma32(as_bf16x8(load16(lk + (kbase ^ (ks << 5)))), as_bf16x8(qreg[ks]), s0);
        s1 = mfma32(as_bf16x8(load16(lk + (kbase ^ ((ks + 1) << 5)))), as_bf16x8(qreg[ks + 1]), s1);
    }
    const bool need_mask = (kb0 + C::BK > k_hi) || p.causal || p.window;
    float mx = -INFINITY;
    f32x16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int j = kb0 + (e >> 3) * 16 + hh * 8 + (e & 7);
        float x = (s0[e] + s1[e]) * p.scale_log2;
        if (CAP) x = soft_cap(x, p.cap_l2, p.cap_k, p.cap_inv);   // in log2 units
        if (BK == kBiasAlibi) {
            x -= slope_l2 * fabsf((float)(qpos - j));
        } else if (BK == kBiasDenseF32 || BK == kBiasDenseBf16) {
            const int bj = min(j, p.Lk - 1);
            const int64_t idx = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh + (int64_t)qi * p.bias_si +
                                (int64_t)bj * p.bias_sj;
            float bv;
            if (BK == kBiasDenseF32)
                bv = static_cast<const float *>(p.bias)[idx];
            else
                bv = bf16_bits_to_f32(static_cast<const uint16_t *>(p.bias)[idx]);
            x = fmaf(bv, kLog2e, x);
        }
        if (need_mask && (j >= k_hi || j < jmin || j > jmax)) x = -INFINITY;
        sc[e] = x;
        mx = fmaxf(mx, x);
    }
    mx = xor32_max(mx);

    // lazy repair: only when some row's max has grown by more than TAU
    if (__any(mx > m_run + kTau)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(oacc[db][e]) : "v"(alpha));
        m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
        const float p0 = exp2_fast(sc[e] - m_use);
        const float p1 = exp2_fast(sc[e + 1] - m_use);
        l_run += p0 + p1;
        pk[e >> 1] = pack_bf16x2(p0, p1);
    }
    // O^T += V^T P^T over the two 16-key halves of the block
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const bf16x8 bop = as_bf16x8(u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const char *vt = lv + (vbase ^ (db << 6));
            const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(vt + half * 16 * C::RB));
            const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t *>(vt + (half * 16 + 4) * C::RB));
            oacc[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), bop, oacc[db]);
        }
    }
}

// Direct loads of the 32-key block at key kb0 into a wave's stage at LDS
// address dst (K block, then V block).  Rows at or past Lk fall outside the
// descriptor's range and read as zero.  The stage's earlier LDS reads are
// complete before it is overwritten.
template <int D>
__device__ __forceinline__ void issue_block(const FwdParams &p, const uint16_t *kp, const uint16_t *vp,
                                            uint32_t kl_bytes, uint32_t vl_bytes, int kb0, uint32_t dst,
                                            const uint32_t (&koff)[BlockCfg<D>::NL],
                                            const uint32_t (&voff)[BlockCfg<D>::NL]) {
    using C = BlockCfg<D>;
    const int nvalid = min(C::BK, p.Lk - kb0);
    const i32x4 rk = rsrc_words(kp + (int64_t)kb0 * p.k_sl, (uint32_t)(nvalid - 1) * kl_bytes + D * 2);
    const i32x4 rv = rsrc_words(vp + (int64_t)kb0 * p.v_sl, (uint32_t)(nvalid - 1) * vl_bytes + D * 2);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < C::NL; ++i) dma16(rk, dst + i * 1024, koff[i]);
#pragma unroll
    for (int i = 0; i < C::NL; ++i) dma16(rv, dst + C::TB + i * 1024, voff[i]);
}

template <int D, int NW, int NST, int BIAS>
__global__ __launch_bounds__(NW * 64) void decode_bf16_kernel(FwdParams p) {
    using C = BlockCfg<D>;
    static_assert(NST >= 1 && NST <= 4 && (NST - 1) * 2 * C::NL < 64, "stage count");
    constexpr int NLB = 2 * C::NL;   // load instructions per block
    // one LDS object per stage, so the compiler can tell the stage being
    // filled from the stage being read
    __shared__ __attribute__((aligned(1024))) char lds_s0[NW][C::STAGE];
    __shared__ __attribute__((aligned(1024))) char lds_s1[NW][NST > 1 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char lds_s2[NW][NST > 2 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char lds_s3[NW][NST > 3 ? C::STAGE : 16];
    __shared__ float lds_m[NW][32];
    __shared__ float lds_l[NW][32];

    const int s = blockIdx.x;
    const int bhk = blockIdx.y;
    const int rb = blockIdx.z;
    const int b = bhk / p.Hkv;
    const int hk = bhk - b * p.Hkv;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: descriptors stay scalar
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
    int jmin, jmax;
    key_range(p, qpos, jmin, jmax);

    // the chunk's keys, narrowed to those some query row of the group can see
    // (rows of all Lq positions share a workgroup, so take the first and last)
    int gjmin, gjmax, unused;
    key_range(p, off, gjmin, unused);
    key_range(p, p.Lq - 1 + off, unused, gjmax);
    const int k_lo = max(s * p.chunk, gjmin);
    const int k_hi = min(min(s * p.chunk + p.chunk, p.Lk), gjmax + 1);
    const int nblk = (k_hi > k_lo) ? (k_hi - k_lo + C::BK - 1) / C::BK : 0;
    const int nmine = (wave < nblk) ? (nblk - wave + NW - 1) / NW : 0;

    const uint16_t *kp = static_cast<const uint16_t *>(p.k) + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vp = static_cast<const uint16_t *>(p.v) + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
    const uint32_t kl_bytes = (uint32_t)p.k_sl * 2u;
    const uint32_t vl_bytes = (uint32_t)p.v_sl * 2u;

    // direct-load source offsets: load i of a block fills LDS bytes
    // [i*1024 + 16*lane, +16) of the K (V) block, i.e. row pos / RB, chunk
    // slot (pos % RB) / 16; K row `row` holds key perm32(row) with its chunks
    // XOR-swizzled, V rows hold keys in order
    uint32_t koff[C::NL], voff[C::NL];
#pragma unroll
    for (int i = 0; i < C::NL; ++i) {
        const int pos = i * 1024 + lane * 16;
        const int row = pos / C::RB;
        const int pc = (pos % C::RB) / 16;
        koff[i] = (uint32_t)perm32(row) * kl_bytes + (uint32_t)((pc ^ C::swz_k(row)) * 16);
        voff[i] = (uint32_t)row * vl_bytes + (uint32_t)((pc ^ C::swz_v(row)) * 16);
    }
    // LDS read offsets: K operand of k-step ks at kbase ^ (ks << 5); V
    // transposing read of d-block db at vbase ^ (db << 6) (+ key rows)
    const int kbase = r * C::RB + ((hh ^ C::swz_k(r)) << 4);
    int vbase;
    {
        const int gq = lane >> 4, sl = lane & 15;
        const int vrow = (gq >> 1) * 8 + (sl >> 2);
        const int e = (gq & 1) * 16 + 4 * (sl & 3);
        vbase = vrow * C::RB + (((e >> 3) ^ C::swz_v(vrow)) * 16) + (e & 7) * 2;
    }

    // prologue: the first NST blocks of this wave
#define DEC_ISSUE(STG_, KB0_) \
    issue_block<D>(p, kp, vp, kl_bytes, vl_bytes, (KB0_), lds_addr((STG_)[wave]), koff, voff)
    if (nmine > 0) DEC_ISSUE(lds_s0, k_lo + wave * C::BK);
    if (NST > 1 && nmine > 1) DEC_ISSUE(lds_s1, k_lo + (wave + NW) * C::BK);
    if (NST > 2 && nmine > 2) DEC_ISSUE(lds_s2, k_lo + (wave + 2 * NW) * C::BK);
    if (NST > 3 && nmine > 3) DEC_ISSUE(lds_s3, k_lo + (wave + 3 * NW) * C::BK);

    // Q fragment and slope, loaded after the first blocks' loads and taken
    // here, so that the wait for them sits outside the loop
    u32x4 qreg[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = u32x4{0, 0, 0, 0};
    if (row_ok) {
        const uint16_t *qr = static_cast<const uint16_t *>(p.q) + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh +
                             (int64_t)qi * p.q_sl + hh * 8;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = load16(qr + ks * 16);
    }
    float slope_l2 = 0.f;
    if (bias_base(BIAS) == kBiasAlibi) slope_l2 = p.slopes[h] * kLog2e;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) asm volatile("" : "+v"(qreg[ks]));
    asm volatile("" : "+v"(slope_l2));

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
    float m_run = -INFINITY;   // reference max, log2 units
    float l_run = 0.f;         // running sum over this lane's half of the keys

    // block n of this wave sits in stage n % NST; after it is consumed the
    // stage is refilled with block n + NST
#define DEC_STEP(STG_, N_)                                                                                       \
    do {                                                                                                         \
        const int n_ = (N_);                                                                                     \
        wait_blocks<NLB, NST>(min(NST - 1, nmine - 1 - n_));                                                     \
        const int kb0 = k_lo + (wave + n_ * NW) * C::BK;                                                         \
        decode_block<D, BIAS>(p, (STG_)[wave], (STG_)[wave] + C::TB, kbase, vbase, qreg, oacc, m_run, l_run,     \
                              kb0, k_hi, qi, qpos, jmin, jmax, slope_l2, b, h, lane);                                        \
        if (n_ + NST < nmine) DEC_ISSUE(STG_, kb0 + NST * NW * C::BK);                                           \
    } while (0)
    for (int n = 0; n < nmine; n += NST) {
        DEC_STEP(lds_s0, n);
        if (NST > 1) {
            if (n + 1 >= nmine) break;
            DEC_STEP(lds_s1, n + 1);
        }
        if (NST > 2) {
            if (n + 2 >= nmine) break;
            DEC_STEP(lds_s2, n + 2);
        }
        if (NST > 3) {
            if (n + 3 >= nmine) break;
            DEC_STEP(lds_s3, n + 3);
        }
    }
#undef DEC_STEP
#undef DEC_ISSUE

    // merge the waves: wave w leaves its (m, l, O) of the valid rows in LDS
    // (O over its own first stage, which it no longer reads), then the
    // workgroup forms M = max_w m_w and the repaired sums
    const int nvalid_rows = min(32, nrows - rb * 32);
    const float l_wave = xor32_sum(l_run);
    float *lo_w = reinterpret_cast<float *>(lds_s0[wave]);
    if (r < nvalid_rows) {
        if (hh == 0) {
            lds_m[wave][r] = m_run;
            lds_l[wave][r] = l_wave;
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4 *>(&lo_w[r * D + db * 32 + i * 8 + hh * 4]) =
                    f32x4{oacc[db][4 * i], oacc[db][4 * i + 1], oacc[db][4 * i + 2], oacc[db][4 * i + 3]};
    }
    __syncthreads();

    constexpr int T = NW * 64;
    for (int c = tid; c < nvalid_rows * (D / 4); c += T) {
        const int rr = c / (D / 4);
        const int d4 = c - rr * (D / 4);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_m[w][rr]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = lds_m[w][rr];
            const float a = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
            const f32x4 ow = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(lds_s0[w]) + rr * D + d4 * 4);
            acc += ow * a;
            L += lds_l[w][rr] * a;
        }
        const int rho2 = rb * 32 + rr;
        const int g2 = rho2 / p.Lq;
        const int i2 = rho2 - g2 * p.Lq;
        const int h2 = hk * p.G + g2;
        const int64_t R = ((int64_t)b * p.Hq + h2) * p.Lq + i2;
        *reinterpret_cast<f32x4 *>(p.o_part + (R * p.num_splits + s) * D + d4 * 4) = acc;
        if (d4 == 0) {
            p.m_part[R * p.num_splits + s] = (M == -INFINITY) ? -INFINITY : M * kLn2;
            p.l_part[R * p.num_splits + s] = L;
        }
    }
}

template <int D, int BIAS>
hipError_t launch_decode_t(const FwdParams &p, hipStream_t stream) {
    constexpr int NW = 4;    // waves per workgroup
    constexpr int NST = 2;   // LDS stages per wave (D = 128: 4 * 2 * 16 KiB, one workgroup per CU)
    const int64_t rblocks = ((int64_t)p.G * p.Lq + 31) / 32;
    if (rblocks == 0 || p.B == 0) return hipSuccess;
    dim3 grid((unsigned)p.num_splits, (unsigned)(p.B * p.Hkv), (unsigned)rblocks), block(NW * 64);
    hipLaunchKernelGGL((decode_bf16_kernel<D, NW, NST, BIAS>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const FwdParams &p, hipStream_t stream) {
    switch (p.bias_kind) {
        case kBiasNone: return launch_decode_t<D, kBiasNone>(p, stream);
        case kBiasAlibi: return launch_decode_t<D, kBiasAlibi>(p, stream);
        case kBiasDenseF32: return launch_decode_t<D, kBiasDenseF32>(p, stream);
        case kBiasDenseBf16: return launch_decode_t<D, kBiasDenseBf16>(p, stream);
        case kBiasNoneCap: return launch_decode_t<D, kBiasNoneCap>(p, stream);
        case kBiasAlibiCap: return launch_decode_t<D, kBiasAlibiCap>(p, stream);
        case kBiasDenseF32Cap: return launch_decode_t<D, kBiasDenseF32Cap>(p, stream);
        case kBiasDenseBf16Cap: return launch_decode_t<D, kBiasDenseBf16Cap>(p, stream);
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
