// attn_device.h -- device-side helpers shared by the gfx950 attention kernels.
//
// Everything here is CDNA4 (gfx950) specific: wave64, the 32x32x16 bf16 matrix
// core instruction, v_exp_f32 (2^x), v_cvt_pk_bf16_f32 and v_permlane32_swap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// D += A * B on the matrix core, 32x32 output, k = 16, bf16 operands, fp32
// accumulate.  Lane l supplies row (l % 32) of A and column (l % 32) of B, each
// as 8 consecutive k values starting at 8 * (l / 32); accumulator element
// 4*i + j of lane l is row 8*i + 4*(l/32) + j, column l % 32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x held by lane (l ^ 32), using the cross-half swap of gfx950.
// Returns {x[l], x[l^32]} in some order; callers only use symmetric
// combinations (max, sum) of the pair.
__device__ __forceinline__ float xor32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Soft cap of a score x in log2 units: c * tanh(x / c) with c = cap (the cap
// in log2 units) and k2 = 2 * log2(e) / c.  For |y| = |x / c| >= 1/16,
// tanh(y) = 1 - 2 / (e^(2y) + 1) with e^(2y) = 2^(x * k2) (relative error a
// few 1e-6); below that the series tanh(y) = y (1 - y^2/3 + ...) is used,
// where the exp form would cancel (the dropped terms are < 1e-6 relative).
__device__ __forceinline__ float soft_cap(float x, float cap, float k2, float inv_cap) {
    const float y = x * inv_cap;
    const float e2 = __builtin_amdgcn_exp2f(x * k2);
    const float far = fmaf(-2.f * cap, __builtin_amdgcn_rcpf(e2 + 1.f), cap);
    const float near = fmaf(-x * y * y, 0.33333334f, x);
    return fabsf(y) < 0.0625f ? near : far;
}

// The exp form alone, for moderate caps.  Near 0 it cancels, but only in
// relative terms: the absolute error of the capped score stays below c * 6e-7
// (a CPU model over the range checks this), and the softmax only sees
// absolute differences of scores.  Used for caps up to 64 (natural units):
// at most 6e-5 in log2 units, against the exact form's five more vector
// instructions per score.
__device__ __forceinline__ float soft_cap_exp(float x, float cap, float k2) {
    const float e2 = __builtin_amdgcn_exp2f(x * k2);
    return fmaf(-2.f * cap, __builtin_amdgcn_rcpf(e2 + 1.f), cap);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two floats to a packed pair of bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void store16(void *p, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Buffer descriptor over `bytes` bytes from `base`: loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The same descriptor as four words, for inline assembly.
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// Buffer-to-LDS loads: 16 (or 4) bytes per lane from buffer offset voff into
// LDS at m0 + 16 * lane (4 * lane).  The whole offset is the vector offset,
// which the hardware checks against the descriptor's range (loads past it
// read zero); a scalar offset would not be checked.  Inline assembly, so that the
// compiler's wait insertion does not see them: a kernel that uses them waits
// for them itself (wait_all_loads, or counted vmcnt waits).  With the
// compiler's builtin, the compiler drains every load in flight before LDS
// reads it cannot prove independent of the load's target, which serialises
// loading and computing.  The assembly writes M0, which is not in the
// clobber list: M0 is a reserved register, and the compiler neither tracks it
// through inline assembly nor promises to restore it when listed.  So no
// compiler-generated instruction of a file that uses these may touch M0; a
// CPU test checks the generated code of every file that calls them.
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t m0, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rsrc)
                 : "memory");
}
__device__ __forceinline__ void dma4(const i32x4 &rsrc, uint32_t m0, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rsrc)
                 : "memory");
}
// every vector memory load of this wave has landed (also a compiler barrier)
__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char *)p);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 4 bf16 values from LDS through the transposing read: within each group of
// 16 lanes, lane i receives element (i % 4) of the 8-byte words addressed by
// lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// s_waitcnt with vmcnt = 0 and the other counters left alone (gfx9 encoding)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Swap bits 2 and 3 of a row index inside a 32-row block.  Loading key
// perm32(r) into matrix-core row r makes the accumulator of S^T = K Q^T hold,
// in lane l, keys 8*(l/32) + 0..7 in elements 0..7 and 16 + 8*(l/32) + 0..7 in
// elements 8..15 -- exactly the B-operand layout the P V product needs, so P
// never leaves registers.  The map is its own inverse.
__device__ __forceinline__ int perm32(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Work order for a grid of per-head tiles.  The dispatcher hands block b to XCD
// b % X (X = the device's XCD count); block b takes item (b % X) * (n / X) +
// b / X of a head-major list, so each XCD runs a contiguous range of heads and
// a head's K/V stays in that XCD's L2.  `rank` numbers a head's tiles, 0
// first.  With `interleave` (tiles of unequal cost, ranked heaviest first),
// windows of 4 heads, else 2, run their tiles rank by rank across the window:
// with one head at a time the last head's heaviest tiles start when the XCD
// is nearly drained and finish alone.  Windows are used only where they tile
// every XCD's range.
struct WorkItem {
    int head;
    int rank;
};
__device__ __forceinline__ WorkItem xcd_work_item(int per_head, bool interleave, int nxcd) {
    const int n = (int)gridDim.x;
    if (nxcd < 1 || n % nxcd != 0) return {(int)blockIdx.x / per_head, (int)blockIdx.x % per_head};
    const int per_xcd = n / nxcd;
    const int item = (int)(blockIdx.x % nxcd) * per_xcd + (int)(blockIdx.x / nxcd);
    int win = 1;
    if (interleave) win = per_xcd % (4 * per_head) == 0 ? 4 : per_xcd % (2 * per_head) == 0 ? 2 : 1;
    const int span = win * per_head;
    const int w0 = item / span;
    const int idx = item - w0 * span;
    const int rank = idx / win;
    return {w0 * win + (idx - rank * win), rank};
}

}  // namespace attn
