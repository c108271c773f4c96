// vs_internal.h -- declarations shared by the HIP sources of libvs (gfx950).
//
// Packed arg-reduction keys.  A candidate's ranking value e (float, smaller
// is better after the metric's sign is applied) and its index j are packed
// into one uint64 so that the unsigned minimum of packed keys is the
// lexicographic minimum of (e, j): the best value, lowest index on ties.
// That makes the merge of partial winners exact and order-independent, which
// is the associativity argument of "Issue 9-014: Tile Diversity Shader Inner
// Loop For L2 Cache Locality", "Intended Behavior", applied to (value, index)
// pairs.  0xFFFF...F means "no candidate".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vs {

constexpr uint64_t kNoKey = ~0ull;

enum Metric : int { L2SQ_MIN = 0, L2SQ_MAX = 1, COS_MAX = 2, COS_MIN = 3 };

__host__ __device__ constexpr bool metric_is_l2(int m) { return m == L2SQ_MIN || m == L2SQ_MAX; }
__host__ __device__ constexpr bool metric_is_max(int m) { return m == L2SQ_MAX || m == COS_MAX; }

// Order-preserving float -> uint32 map (-0 folded onto +0 first).
__device__ __forceinline__ uint32_t ord_of(float x) {
    x = (x == 0.0f) ? 0.0f : x;
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_of_ord(uint32_t o) {
    const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t pack_key(float e, uint32_t j) {
    return (static_cast<uint64_t>(ord_of(e)) << 32) | j;
}

// Ranking value of one pair from its dot product s (and the candidate's
// squared norm cn for squared L2).  The query's own squared norm is the same
// for every candidate, so it is added back only when the score is reported.
template <int M>
__device__ __forceinline__ float rank_value(float s, float cn) {
    if constexpr (M == L2SQ_MIN) return __builtin_fmaf(-2.0f, s, cn);
    else if constexpr (M == L2SQ_MAX) return __builtin_fmaf(2.0f, s, -cn);
    else if constexpr (M == COS_MAX) return -s;
    else return s;
}

// LDS-DMA (global_load_lds): lane l of the issuing wave writes LDS bytes
// [base + w l, base + w l + w), w = 16 or 4 bytes; lanes that are switched
// off write nothing.
__device__ __forceinline__ void dma16(const float *g, float *lds_base) {
    __builtin_amdgcn_global_load_lds(
        (const void *)g, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const float *g, float *lds_base) {
    __builtin_amdgcn_global_load_lds(
        (const void *)g, (__attribute__((address_space(3))) void *)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(n) for the small counts the slab pipelines need (0 .. 4).
__device__ __forceinline__ void wait_vmcnt(int n) {
    if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
}

// s_waitcnt vmcnt(N) for a compile-time count N (0 .. 63).
template <int N>
__device__ __forceinline__ void wait_vmcnt_n() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (the fence
// waits for every outstanding load, including slab loads meant to stay in
// flight across the barrier); callers make the LDS data they need visible
// with explicit waits before it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- kernels --

struct DenseArgs {
    const float *Q;         // nq x d (unused when gathering)
    const float *C;         // nc x d
    const int32_t *pick;    // gather: query i is row pick[i] of C
    const uint32_t *mask;   // nq x W words, or null
    const float *cn;        // nc squared norms (L2 metrics)
    uint64_t *keys;         // nq packed keys (pre-filled with kNoKey)
    int64_t nq, nc;
    int32_t d;
    int64_t mask_words;     // W
    int64_t n_items;        // query tiles x candidate tiles
    int64_t n_ctiles;
    int32_t grid;           // launched workgroups (for the item split)
    int32_t split;          // 1; 8: candidate tiles split into one range per XCD;
                            // 2: the triangle walk of the symmetric store mode
    float *S;               // score block (store mode): S[q * ld_s + c]
    int64_t ld_s;
};

struct CsrArgs {
    const int32_t *indptr, *indices;
    const float *values;
    const float *CT;        // codebook: feature k of neuron 64 b + j at
                            // CT + b * cstride (bytes) + (k * ldct + j) floats
    const float *cn;        // nc
    uint64_t *keys;         // nq
    int64_t nq, nnz, nc, ldct;
    int64_t cstride;        // bytes between 64-neuron blocks: 256 (plain rows) or d * 256
    int32_t d;
    int64_t n_chunks;       // candidate chunks
};

// Where a dense scan takes its queries from: the rows of a.Q; rows
// a.C[a.pick[i]] with the mask (the diversity step); the rows of a.Q with
// the mask (a step against explicit reference rows).  The masked forms rank
// by COS_MIN.
enum QueryMode : int { kQRows = 0, kQGatherMasked = 1, kQRowsMasked = 2 };

}  // namespace vs

// Host-side launchers: declarations only (kept apart so that adding a
// launcher leaves this file, which the kernels' code depends on, unchanged).
#include "vs_launch.h"
