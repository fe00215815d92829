/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention library
 * (libattn_mi355x.so): forward (prefill, split-K decode) and backward.
 *
 * The operation is the attention chain of "Neptune论文浅读：把FlashAttention式融合
 * 放进编译器" (gentlecold.top), section 2: S = scale * Q K^T, then the score
 * modifier (causal mask, additive bias), then the stable softmax of each score
 * row, then P V.  It is computed in one pass over the keys without writing the
 * Lq x Lk score matrix anywhere:
 *   - prefill uses the rolling update of section 5 of those notes (running
 *     max m and sum l per query row, the accumulated sum and output repaired by
 *     exp(m_old - m_new) whenever the max grows, section 3 and section 4);
 *   - decode uses the split-K update of section 6: the keys are cut into
 *     chunks, each chunk yields a local (o, m, l), and a global step repairs
 *     the chunks with the global max and merges them.
 * The variants covered are those listed in section 9 of the notes that change
 * the score only: global (no mask), causal, ALiBi, dense additive bias, and GQA
 * (query heads sharing K/V heads, CMU 15-779 Lecture 11 "Mirage" notes,
 * section 7.1), in prefill and decode form.
 *
 * Conventions shared by every call
 * --------------------------------
 *   Layout       Q [B, Hq, Lq, D]; K, V [B, Hkv, Lk, D]; O [B, Hq, Lq, D]; the
 *                last dimension (d) is contiguous, the b, h, l strides are given
 *                in ELEMENTS.  LSE [B, Hq, Lq] is contiguous fp32.
 *   GQA          Hq % Hkv == 0; query head h reads K/V head h / (Hq / Hkv)
 *                (contiguous groups of query heads share one K/V head).
 *   Score        s_ij = scale * <q_i, k_j> + bias_ij (bias is not scaled).
 *   Causal       aligned to the end of the keys: key j is visible to query row
 *                i iff j <= i + (Lk - Lq).  For Lq == Lk this is the lower
 *                triangle; a single decode query (Lq = 1) sees every key.
 *   ALiBi        bias_ij = -alibi_slopes[h] * |i + (Lk - Lq) - j|.  With the
 *                causal mask and bf16 inputs the bias enters the key-query
 *                product as one more matrix-core step, relative to the position
 *                of each group of 32 rows; its rounding grows with the slope:
 *                for |slope| <= 64 it stays below 1e-3 on LSE and 1.5e-2 on O
 *                against an exact evaluation (ALiBi's own slopes are at most 1).
 *   Output       O_i = sum_j softmax(s_i)_j v_j;  LSE_i = ln sum_j exp(s_ij)
 *                (natural log).  A row with no visible key gets O_i = 0 and
 *                LSE_i = -inf (never NaN).
 *   Arithmetic   bf16 inputs are multiplied on the matrix cores with fp32
 *                accumulation; the softmax, the running max/sum, LSE and all
 *                partials are fp32.  fp32 inputs are computed in fp32.
 *   Pointers     every tensor pointer is a DEVICE pointer owned by the caller;
 *                the library never allocates, frees or synchronises, keeps no
 *                state except a per-device cache of the compute-unit and XCD
 *                counts, and enqueues its kernels on the given HIP stream (a hipStream_t
 *                passed as void*, NULL = the null stream).  Calls return as soon
 *                as the kernels are enqueued.  Calls are thread-safe.
 *   Alignment    q, k, v and o base pointers must be 16-byte aligned and every
 *                b/h/l stride a multiple of 16 bytes' worth of elements.
 *   Errors       arguments are checked on the host before anything is
 *                enqueued; a failed check returns ATTN_ERR_INVALID_ARG (bad
 *                value) or ATTN_ERR_UNSUPPORTED (valid but not implemented:
 *                D not in {64, 128}, dtype combination, alignment; sizes
 *                beyond what the kernels hold: any of B, H, L, D above
 *                2^31 - 1, or products of them past the kernels' 32-bit
 *                grids) and enqueues nothing.  A launch failure returns
 *                ATTN_ERR_HIP; the thread's HIP error state is cleared before
 *                the launch, so the error is the call's own.  No C++
 *                exception crosses this interface.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,
    ATTN_ERR_UNSUPPORTED = 2,
    ATTN_ERR_WORKSPACE = 3,
    ATTN_ERR_HIP = 4
} attn_status;

/* Element types (values of the *_dtype fields). */
enum { ATTN_F32 = 0, ATTN_BF16 = 1 };

/* Score-bias kinds (values of bias_kind). */
enum { ATTN_BIAS_NONE = 0, ATTN_BIAS_DENSE = 1, ATTN_BIAS_ALIBI = 2 };

/*
 * Arguments of one attention forward problem (the problem statement of the
 * Neptune notes, section 2: Q, K, V, scale, mask, bias; section 9: the causal,
 * ALiBi and GQA variants).
 */
typedef struct attn_fwd_args {
    int64_t B, Hq, Hkv, Lq, Lk, D;   /* batch, query heads, K/V heads, query rows, keys, head dim */
    int32_t dtype;                   /* ATTN_F32 or ATTN_BF16: element type of q, k and v */
    int32_t causal;                  /* 0 = every key visible; 1 = end-aligned causal mask */
    const void *q, *k, *v;           /* device pointers */
    int64_t q_strides[3];            /* b, h, l strides of q in elements (d stride is 1) */
    int64_t k_strides[3];
    int64_t v_strides[3];
    float scale;                     /* multiplies <q, k> before the bias is added */
    int32_t bias_kind;               /* ATTN_BIAS_NONE / ATTN_BIAS_DENSE / ATTN_BIAS_ALIBI */
    const void *bias;                /* DENSE: device pointer to the bias, element (b,h,i,j) at
                                        b*bias_strides[0] + h*bias_strides[1] + i*bias_strides[2]
                                        + j*bias_strides[3]; a stride of 0 broadcasts */
    int32_t bias_dtype;              /* ATTN_F32 or ATTN_BF16 */
    int32_t o_dtype;                 /* ATTN_F32 or ATTN_BF16: element type of o */
    int64_t bias_strides[4];
    const float *alibi_slopes;       /* ALIBI: device pointer to Hq fp32 slopes */
    void *o;                         /* device pointer, O [B, Hq, Lq, D] */
    int64_t o_strides[3];            /* b, h, l strides of o in elements */
    float *lse;                      /* device pointer to [B, Hq, Lq] fp32, or NULL */
    /* SoftCap and Window, the two further score modifiers the Neptune notes
       list in section 9 (named there without a formula; these are the plain
       readings).  A zero-filled tail leaves both off. */
    float softcap;                   /* > 0: the scaled score t = scale*<q,k> becomes
                                        softcap * tanh(t / softcap) before the bias is added;
                                        0 = off */
    int32_t window;                  /* 1: only keys p - window_left <= j <= p + window_right
                                        are visible (p = i + Lk - Lq, intersected with the
                                        causal bound); 0 = no window */
    int32_t window_left;             /* keys to the left of p; negative = unbounded */
    int32_t window_right;            /* keys to the right of p; negative = unbounded */
} attn_fwd_args;

/*
 * attn_fwd_prefill -- fused attention forward with the rolling update
 * (Neptune notes, section 5; the loop structure of the CANN FlashAttention
 * post: a query tile stays on chip while K/V tiles stream past it).
 * Writes o and, when lse != NULL, lse.  Any Lq, Lk >= 0.
 */
attn_status attn_fwd_prefill(const attn_fwd_args *a, void *stream);

/*
 * attn_fwd_decode_splitk -- local step of the split-K update (Neptune notes,
 * section 6).  The keys are cut into num_splits chunks
 *     chunk s = [s*C, min((s+1)*C, Lk)),  C = 32 * ceil(Lk / (32 * num_splits)),
 * and for every query row (b, h, i) and chunk s it writes, in fp32,
 *     m_part[b,h,i,s]   a reference value (natural-log units) for the chunk,
 *     l_part[b,h,i,s] = sum_j exp(s_ij - m),
 *     o_part[b,h,i,s,:] = sum_j exp(s_ij - m) v_j      (not normalised),
 * over the visible keys j of the chunk.  A chunk with no visible key gives
 * m = -inf, l = 0, o = 0.  The query heads of one K/V group are processed
 * together so each K/V element is read once per group (Mirage lecture notes,
 * section 7.1).  o_part is [B, Hq, Lq, num_splits, D] and m_part, l_part are
 * [B, Hq, Lq, num_splits], all contiguous device fp32 buffers owned by the
 * caller (attn_decode_partial_bytes gives their total size).  a->o and a->lse
 * are not used.  Any Lq >= 0 (Lq = 1 is the decode case), 1 <= num_splits <= 65535.
 */
attn_status attn_fwd_decode_splitk(const attn_fwd_args *a, int32_t num_splits,
                                   float *o_part, float *m_part, float *l_part, void *stream);

/*
 * attn_splitk_combine -- global step of the split-K update (Neptune notes,
 * section 6, with the repair term exp(r - r') of section 4): for every row,
 *     M = max_s m_s,  w_s = exp(m_s - M),  L = sum_s w_s l_s,
 *     O = sum_s w_s o_s / L,  LSE = M + ln L;
 * a row whose chunks are all empty gets O = 0, LSE = -inf.  The partials are
 * laid out as attn_fwd_decode_splitk writes them (rows = B*Hq*Lq).  o is
 * [B, Hq, Lq, D] with the given strides and element type; lse may be NULL.
 */
attn_status attn_splitk_combine(const float *o_part, const float *m_part, const float *l_part,
                                int64_t B, int64_t Hq, int64_t Lq, int64_t D, int32_t num_splits,
                                void *o, int32_t o_dtype, const int64_t o_strides[3],
                                float *lse, void *stream);

/*
 * attn_decode_choose_splits -- split count for attn_fwd_decode_splitk (pure
 * host function, no HIP call).  Picks the smallest number of key chunks for
 * which the B * Hkv * ceil(Lq*Hq/Hkv / 32) * num_splits workgroups give every
 * one of cu_count compute units a workgroup (each workgroup streams its chunk
 * with enough loads in flight to keep its share of HBM busy), while keeping
 * at least 256 keys per chunk (an
 * under-filled grid is what the Mirage lecture notes, section 7.1, measure as
 * the cost of fixed grid heuristics).  Returns >= 1; 1 when Lk <= 256.
 */
int32_t attn_decode_choose_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                                  int32_t cu_count);

/*
 * Automatic choice of the parallel dimensions
 * -------------------------------------------
 * The prefill kernel parallelises over batch, query head and query rows (one
 * workgroup per 128 rows of one query head, every K/V tile streamed past
 * it); the split-K kernel parallelises over batch, K/V head, the rows of a
 * K/V group (the G query heads of the group times Lq rows, stacked 32 to a
 * workgroup, so each K/V element is read once per group) and key chunks,
 * followed by the combine.  The Mirage lecture notes (section 7.1) observe
 * that fixed choices of these dimensions underfill the GPU for few heads and
 * short query lengths, and that the right choice depends on the problem; the
 * Neptune notes (section 6) trade partial-result storage for parallelism
 * along the keys.
 *
 * attn_fwd_choose_plan picks, from the shapes alone (pure host function):
 *   split-K, when Lq <= 16 and R = B * Hkv * ceil(G * Lq / 32) row blocks
 *            fit on the compute units at once (R <= cu_count), with
 *            num_splits from attn_decode_choose_splits;
 *   split prefill, otherwise, when attn_prefill_choose_splits gives two or
 *            more key chunks (the prefill grid leaves compute units idle, or
 *            the rows are long enough for chunks of 8192 keys), then the
 *            combine;
 *   split-K, otherwise, when R <= cu_count;
 *   prefill, otherwise (and always for fp32 inputs, or shapes the split-K
 *            grid cannot hold).
 * The rule is measured: on MI355X, over 216 shapes (B 1 and 4; Hq/Hkv 8/8,
 * 32/8, 64/8; Lq 1 to 2048; Lk 4096 and 32768; causal and not) the planned
 * path is within 1.093x of the fastest of the three at its best split count
 * (split-K is the fastest for Lq <= 16; the split prefill beats it by up to
 * 2.2x from Lq = 64 on, and the plain prefill by up to 1.8x on small grids).
 */
enum { ATTN_PLAN_PREFILL = 0, ATTN_PLAN_SPLITK = 1, ATTN_PLAN_PREFILL_SPLIT = 2 };

typedef struct attn_fwd_plan {
    int32_t method;                  /* ATTN_PLAN_PREFILL, ATTN_PLAN_SPLITK or ATTN_PLAN_PREFILL_SPLIT */
    int32_t num_splits;              /* split-K and split prefill: key chunks (split-K: 1 = grouped rows,
                                        no split); prefill: 0 */
    size_t workspace_bytes;          /* device workspace attn_fwd needs for this plan (0 for prefill) */
} attn_fwd_plan;

/*
 * attn_fwd_prefill_splitk -- the prefill kernel over key chunks (Neptune
 * notes, section 6: partial results per chunk, merged afterwards): a grid of
 * (128-row query tile, key chunk) workgroups, for grids too small to occupy
 * the device over the query rows alone.  Chunk s holds keys
 *     [s*C, min((s+1)*C, Lk)),  C = 64 * ceil(Lk / (64 * num_splits))
 * (whole 64-key tiles; trailing chunks may be empty).  The partials have the
 * layout and meaning of attn_fwd_decode_splitk's (o_part [B, Hq, Lq,
 * num_splits, D] not normalised, m_part and l_part [B, Hq, Lq, num_splits],
 * m in natural units; a row that sees no key of a chunk gets m = -inf, l = 0,
 * o = 0), so attn_splitk_combine finishes the forward.  Arguments as for
 * attn_fwd_prefill (o, o_strides and lse are not used); bf16 inputs only
 * (ATTN_ERR_UNSUPPORTED otherwise); 1 <= num_splits <= 65535.  The buffers
 * are contiguous device fp32 arrays owned by the caller (o_part 16-byte
 * aligned); nothing is allocated.
 */
attn_status attn_fwd_prefill_splitk(const attn_fwd_args *a, int32_t num_splits,
                                    float *o_part, float *m_part, float *l_part, void *stream);

/*
 * attn_prefill_choose_splits -- key chunks for attn_fwd_prefill_splitk (pure
 * host function): enough (query tile, chunk) workgroups for two per compute
 * unit, B * Hq * ceil(Lq / 128) * num_splits >= 2 * cu_count (<= 0: 256),
 * with at least 1024 keys per chunk; when the unsplit grid already has a
 * workgroup per compute unit, only if the chunks hold 8192 keys or more.
 * Returns 1 (no split) or the chunk count.
 */
int32_t attn_prefill_choose_splits(int64_t B, int64_t Hq, int64_t Lq, int64_t Lk, int32_t cu_count);

/*
 * attn_fwd_choose_plan -- the plan attn_fwd runs for `a` on a device with
 * cu_count compute units (<= 0: 256).  Validates like attn_validate_prefill
 * and writes *plan on success.
 */
attn_status attn_fwd_choose_plan(const attn_fwd_args *a, int32_t cu_count, attn_fwd_plan *plan);

/*
 * attn_fwd -- the forward with the plan chosen for the current device: writes
 * o and, when lse != NULL, lse, exactly as attn_fwd_prefill does (same
 * arguments and conventions).  A split-K plan keeps its partials in the
 * caller's device workspace (16-byte aligned, at least plan.workspace_bytes;
 * its contents on entry do not matter); a smaller workspace returns
 * ATTN_ERR_WORKSPACE and enqueues nothing.  NULL / 0 is fine when the plan is
 * prefill.
 */
attn_status attn_fwd(const attn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_fwd_noalloc -- attn_fwd for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, hosts that forbid
 * hipMalloc): the same plan, kernels and results as attn_fwd, with the
 * split plans' partials in a fixed array that the library holds on each
 * device (ATTN_NOALLOC_SCRATCH_BYTES per device, taken at the first call on
 * that device and kept until the process ends).  Allocates nothing and takes
 * no workspace.  A plan whose partials exceed the array (plan.workspace_bytes
 * > ATTN_NOALLOC_SCRATCH_BYTES) returns ATTN_ERR_WORKSPACE and enqueues
 * nothing; the prefill plan needs no array.  All calls on one device share
 * its array: calls whose execution overlaps on one device (different streams
 * without ordering between them) race on it; calls on one stream are ordered.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
attn_status attn_fwd_noalloc(const attn_fwd_args *a, void *stream);

/* attn_decode_partial_bytes -- bytes of o_part + m_part + l_part for a decode call. */
size_t attn_decode_partial_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int32_t num_splits);

/* attn_device_cu_count -- compute units of HIP device `device` (cached); <= 0 on error. */
int32_t attn_device_cu_count(int32_t device);

/*
 * attn_device_xcd_count -- accelerator complex dies (XCDs) of HIP device
 * `device` (cached; 1 when the runtime reports none); <= 0 on error.  Each
 * XCD has its own L2 cache and the hardware deals workgroups to the XCDs in
 * turn; the kernels order their work by this count so that the K/V of one
 * head stays in one XCD's L2.  Every launching call reads both counts of the
 * current device.
 */
int32_t attn_device_xcd_count(int32_t device);

/*
 * attn_validate_prefill / attn_validate_decode -- the host-side argument
 * check that the corresponding entry point runs before enqueuing anything
 * (pure host functions, no HIP call; usable without a GPU).
 */
attn_status attn_validate_prefill(const attn_fwd_args *a);
attn_status attn_validate_decode(const attn_fwd_args *a, int32_t num_splits,
                                 const float *o_part, const float *m_part, const float *l_part);

/* attn_fwd_args_size -- sizeof(attn_fwd_args), so a binding can check its mirror of the struct. */
size_t attn_fwd_args_size(void);

/*
 * Backward pass
 * -------------
 * The gradients of the forward above with respect to q, k and v, for an
 * output gradient dO.  The pages give the backward only by its shape (the
 * review "Optimal Software Pipelining and Warp Specialization for Tensor Core
 * GPUs", section 7.2: one pass over the tiles with five matrix products and
 * one exponential, recomputing the weights from the saved log-sum-exp instead
 * of storing them); the values are the plain derivatives of the forward
 * definition.  With P_ij = exp(s_ij - LSE_i) (the saved LSE, natural log),
 *     Delta_i = <dO_i, O_i>
 *     dv_j    = sum_i P_ij dO_i
 *     dS_ij   = P_ij (<dO_i, v_j> - Delta_i)           (softmax Jacobian)
 *     dU_ij   = dS_ij (1 - tanh^2(t_ij / c))  with a soft cap c, else dS_ij
 *     dq_i    = scale * sum_j dU_ij k_j,   dk_j = scale * sum_i dU_ij q_i,
 * sums over the visible pairs; a K/V head collects the gradients of every
 * query head of its group.  The bias receives no gradient.  A row with no
 * visible key (LSE = -inf) gets dq = 0 and adds nothing.
 */
typedef struct attn_bwd_args {
    attn_fwd_args fwd;               /* the forward problem as it was run: shapes, q, k, v, scale,
                                        causal, bias, softcap, window.  fwd.o (element type
                                        fwd.o_dtype, strides fwd.o_strides) and fwd.lse are READ:
                                        they must hold that forward's outputs; fwd.lse is required */
    const void *dout;                /* dO [B, Hq, Lq, D], element type fwd.dtype */
    int64_t dout_strides[3];         /* b, h, l strides of dout in elements */
    int32_t grad_dtype;              /* ATTN_F32 or ATTN_BF16: element type of dq, dk and dv */
    int32_t reserved;                /* must be 0 */
    void *dq;                        /* device, dQ [B, Hq, Lq, D], written */
    int64_t dq_strides[3];
    void *dk;                        /* device, dK [B, Hkv, Lk, D], written */
    int64_t dk_strides[3];
    void *dv;                        /* device, dV [B, Hkv, Lk, D], written */
    int64_t dv_strides[3];
    float *workspace;                /* device, attn_bwd_workspace_bytes(B, Hq, Lq) bytes, 16-byte
                                        aligned; its contents on entry do not matter */
} attn_bwd_args;

/*
 * attn_bwd -- writes dq, dk and dv (every element, also those of keys no
 * query sees, which get 0).  bf16 q, k, v and dout only (fp32 inputs return
 * ATTN_ERR_UNSUPPORTED), D in {64, 128}, the alignment rules of the forward
 * for dout, dq, dk and dv.  dq, dk, dv and the workspace must not overlap
 * each other or any input.  Two kernels run on the stream: the first forms
 * Delta per query row together with dq, the second dk and dv; neither uses
 * atomics, so the result is deterministic.
 */
attn_status attn_bwd(const attn_bwd_args *a, void *stream);

/* attn_bwd_workspace_bytes -- workspace size for attn_bwd (2 fp32 per query row). */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq);

/* attn_validate_bwd -- the host-side check attn_bwd runs (pure host function). */
attn_status attn_validate_bwd(const attn_bwd_args *a);

/* attn_bwd_args_size -- sizeof(attn_bwd_args). */
size_t attn_bwd_args_size(void);

/* attn_status_str -- static English text for a status code. */
const char *attn_status_str(attn_status s);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
