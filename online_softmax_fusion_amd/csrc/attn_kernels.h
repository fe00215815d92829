// attn_kernels.h -- parameter block and launch functions of the gfx950 kernels
// (internal to libattn_mi355x.so; the public interface is include/attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// kBiasNoneScaled: no bias, score formed explicitly (used when the scale is not
// positive).  The *Cap kinds add the soft cap of the scaled score.
// Four kinds are chosen by the prefill launcher and never set by the host
// interface: kBiasDenseBf16Tiled, a bf16 dense bias whose rows are contiguous
// and 16-byte aligned, loaded a tile at a time into LDS beside K and V, and
// kBiasDenseBf16TiledDesc, the same under a causal mask with the key tiles
// visited from the diagonal down; kBiasAlibiCausal, ALiBi under a causal mask
// with a positive scale, whose bias is added to the scores by one more
// matrix-core product; and kBiasNoneCapExp, the soft cap without a bias for
// caps up to 64, formed by the exp form alone (soft_cap_exp).
enum BiasKind {
    kBiasNone = 0, kBiasAlibi = 1, kBiasDenseF32 = 2, kBiasDenseBf16 = 3, kBiasNoneScaled = 4,
    kBiasNoneCap = 5, kBiasAlibiCap = 6, kBiasDenseF32Cap = 7, kBiasDenseBf16Cap = 8,
    kBiasDenseBf16Tiled = 9, kBiasAlibiCausal = 10, kBiasNoneCapExp = 11, kBiasDenseBf16TiledDesc = 12
};
// whether a kind carries the soft cap, and its bias part
constexpr bool bias_cap(int kind) {
    return (kind >= kBiasNoneCap && kind <= kBiasDenseBf16Cap) || kind == kBiasNoneCapExp;
}
constexpr int bias_base(int kind) {
    return (kind == kBiasNoneCap || kind == kBiasNoneCapExp) ? kBiasNoneScaled
           : kind == kBiasDenseBf16TiledDesc                  ? kBiasDenseBf16Tiled
           : bias_cap(kind)                                   ? kind - 5
                                                              : kind;
}

// tanh(y) = y * (c0 + c1 y^2 + c2 y^4 + c3 y^6) for |y| <= 1/2, to an
// absolute error of 1.3e-7: a minimax fit (Lawson's iteration on
// Chebyshev nodes) of tanh(y) / y as a cubic in y^2 against the absolute
// error of the product, coefficients rounded to float.  The soft cap c
// tanh(t / c) then carries at most c * 1.3e-7 of error, against the exact
// exp form's two more transcendental instructions per score.
constexpr float kTanhPoly[4] = {0.9999976754188538f, -0.33320656418800354f, 0.13145145773887634f,
                                -0.04337248206138611f};

// One attention problem after validation.  Strides are in elements.
struct FwdParams {
    const void *q, *k, *v;
    int64_t q_sb, q_sh, q_sl;
    int64_t k_sb, k_sh, k_sl;
    int64_t v_sb, v_sh, v_sl;
    void *o;
    int64_t o_sb, o_sh, o_sl;
    float *lse;
    const void *bias;
    int64_t bias_sb, bias_sh, bias_si, bias_sj;
    const float *slopes;
    float *o_part, *m_part, *l_part;   // split-K partials (decode)
    int B, Hq, Hkv, G, Lq, Lk, D;
    int causal;
    int bias_kind;                      // BiasKind
    int o_bf16;                         // 1: o is bf16, 0: fp32
    int num_splits, chunk;              // decode: number of key chunks, keys per chunk
    float scale;                        // softmax scale (natural units)
    float scale_log2;                   // scale * log2(e)
    float softcap;                      // soft cap of the scaled score (natural units); 0 = off
    float cap_l2;                       // soft cap in log2 units (softcap * log2(e)); 0 = off
    float cap_k;                        // 2 / softcap: 2^(x * cap_k) = e^(2 x / cap_l2)
    float cap_inv;                      // 1 / cap_l2
    float cap_q[4];                     // capped score (log2 units) = s * (q0 + q1 w + q2 w^2 + q3 w^3),
                                        // w = s^2, for raw scores |s| <= cap_s0 (tanh_poly, scaled)
    float cap_s0;                       // raw-score range of cap_q: 0.5 * softcap / scale
    int window;                         // 1: apply win_left / win_right
    int win_left, win_right;            // keys left / right of the query position; < 0 = unbounded
    int num_cus, num_xcds;              // compute units and XCDs of the launch device
    uint32_t bias_plane_bytes;          // kBiasDenseBf16Tiled: bytes of one (b, h) plane of the bias
};

// Visible key range [jmin, jmax] of the query at end-aligned position
// pos = i + Lk - Lq (so pos <= Lk - 1): causal bound, window bounds, keys that
// exist.  jmax < jmin means no visible key (only for pos < 0).  Both ends are
// non-decreasing in pos, so the rows of a tile see the keys between the
// first row's jmin and the last row's jmax.
__host__ __device__ inline void key_range(const FwdParams &p, int pos, int &jmin, int &jmax) {
    int64_t lo = 0, hi = (int64_t)p.Lk - 1;
    if (p.causal && pos < hi) hi = pos;
    if (p.window) {
        if (p.win_left >= 0 && (int64_t)pos - p.win_left > lo) lo = (int64_t)pos - p.win_left;
        if (p.win_right >= 0 && (int64_t)pos + p.win_right < hi) hi = (int64_t)pos + p.win_right;
    }
    jmin = (int)lo;
    jmax = (int)hi;
}

// Query rows [imin, imax] that see key j (0 <= j < Lk), the inverse of
// key_range: row i sees j iff jmin(i + Lk - Lq) <= j <= jmax(i + Lk - Lq).
// Both ends are non-decreasing in j.  imax < imin means no row sees j.
__host__ __device__ inline void query_range(const FwdParams &p, int j, int &imin, int &imax) {
    const int64_t off = (int64_t)p.Lk - p.Lq;
    int64_t plo = -((int64_t)1 << 40), phi = (int64_t)1 << 40;   // positions i + off that see j
    if (p.causal && (int64_t)j > plo) plo = j;
    if (p.window) {
        if (p.win_right >= 0 && (int64_t)j - p.win_right > plo) plo = (int64_t)j - p.win_right;
        if (p.win_left >= 0 && (int64_t)j + p.win_left < phi) phi = (int64_t)j + p.win_left;
    }
    int64_t lo = plo - off, hi = phi - off;
    if (lo < 0) lo = 0;
    if (hi > (int64_t)p.Lq - 1) hi = (int64_t)p.Lq - 1;
    if (j < 0 || j >= p.Lk || hi < lo) {
        lo = 0;
        hi = -1;
    }
    imin = (int)lo;
    imax = (int)hi;
}

// Gradients of one attention problem (the forward problem plus dO and the
// outputs).  Strides are in elements.
struct BwdParams {
    FwdParams f;                        // f.o: the forward's output (read); f.lse: its LSE (read)
    const void *dout;
    int64_t do_sb, do_sh, do_sl;
    void *dq, *dk, *dv;
    int64_t dq_sb, dq_sh, dq_sl;
    int64_t dk_sb, dk_sh, dk_sl;
    int64_t dv_sb, dv_sh, dv_sl;
    float *delta;                       // [B*Hq*Lq] <dO_i, O_i>, written by the dQ kernel
    float *lse_l2;                      // [B*Hq*Lq] LSE in log2 units (+inf for an empty row), same
    int grad_bf16;                      // 1: dq, dk, dv are bf16, 0: fp32
};

struct CombineParams {
    const float *o_part, *m_part, *l_part;
    void *o;
    int64_t o_sb, o_sh, o_sl;
    float *lse;
    int B, Hq, Lq, D, S;
    int o_bf16;
};

// Row-wise L2 norm (one pass when S <= 1, else split over the row).  Strides
// in elements; ws holds rows * S (int exponent, float scaled sum) pairs.
struct L2Params {
    const void *x;
    int64_t x_stride;
    void *y;
    int64_t y_stride;
    float *norm;
    int64_t rows, H;
    int x_bf16, y_bf16;
    int S, chunk_vecs;                  // split count, 16-byte vectors per chunk
    void *ws;
};

// bf16 prefill with the rolling update (matrix cores, D in {64, 128}).
hipError_t launch_prefill_bf16(const FwdParams &p, hipStream_t stream);
// split-K prefill: key chunks of p.chunk keys (a multiple of 64), p.num_splits of them,
// partials to p.o_part / p.m_part / p.l_part in the decode kernel's layout
hipError_t launch_prefill_part_bf16(const FwdParams &p, hipStream_t stream);
// bf16 split-K decode partials (matrix cores, D in {64, 128}).
hipError_t launch_decode_bf16(const FwdParams &p, hipStream_t stream);
// fp32 path: one wavefront per query row; partial != 0 writes split-K partials.
hipError_t launch_rows_f32(const FwdParams &p, int partial, hipStream_t stream);
// log-sum-exp combine of split-K partials.
hipError_t launch_combine(const CombineParams &c, hipStream_t stream);
// row-wise L2 norm
hipError_t launch_l2norm(const L2Params &p, hipStream_t stream);
// bf16 backward: dQ (and Delta, LSE in log2 units), then dK and dV.
hipError_t launch_bwd_bf16(const BwdParams &p, hipStream_t stream);

}  // namespace attn
