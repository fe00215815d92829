// attn_kernels.h -- parameter block and launch functions of the gfx950 kernels
// (internal to libattn_mi355x.so; the public interface is include/attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// kBiasNoneScaled: no bias, score formed explicitly (used when the scale is not positive)
enum BiasKind { kBiasNone = 0, kBiasAlibi = 1, kBiasDenseF32 = 2, kBiasDenseBf16 = 3, kBiasNoneScaled = 4 };

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
};

struct CombineParams {
    const float *o_part, *m_part, *l_part;
    void *o;
    int64_t o_sb, o_sh, o_sl;
    float *lse;
    int B, Hq, Lq, D, S;
    int o_bf16;
};

// bf16 prefill with the rolling update (matrix cores, D in {64, 128}).
hipError_t launch_prefill_bf16(const FwdParams &p, hipStream_t stream);
// bf16 split-K decode partials (matrix cores, D in {64, 128}).
hipError_t launch_decode_bf16(const FwdParams &p, hipStream_t stream);
// fp32 path: one wavefront per query row; partial != 0 writes split-K partials.
hipError_t launch_rows_f32(const FwdParams &p, int partial, hipStream_t stream);
// log-sum-exp combine of split-K partials.
hipError_t launch_combine(const CombineParams &c, hipStream_t stream);

}  // namespace attn
