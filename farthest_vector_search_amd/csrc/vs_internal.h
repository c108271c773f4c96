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
    int32_t split;          // 1, or 8: candidate tiles split into one range per XCD
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

// Launchers (return hipError_t of the launch).  The dominant kernel of each
// entry point is bracketed by the library's timing events when recording.
hipError_t launch_fill_keys(uint64_t *keys, int64_t n, hipStream_t st);
hipError_t launch_row_sqnorms(const float *X, int64_t rows, int32_t d, float *out,
                              hipStream_t st);
// feature k of column j at X[(j / 64) * cs + k * ld + j % 64]
hipError_t launch_col_sqnorms(const float *X, int64_t cols, int64_t ld, int64_t cs, int32_t d,
                              float *out, hipStream_t st);
hipError_t launch_block_codebook(const float *CT, int64_t nc, int64_t ldct, int32_t d, float *CB,
                                 hipStream_t st);
// fp16 codebook, 128-neuron blocks: feature k of neuron 128 b + j at
// CB[(b * d + k) * 128 + j]; from the plain feature-major CT, or (when
// src_blocked64) from the 64-neuron blocked fp32 layout
hipError_t launch_block_codebook_f16(const float *CT, int64_t nc, int64_t ldct, int32_t d,
                                     uint16_t *CB, hipStream_t st, bool src_blocked64 = false);
hipError_t launch_col_sqnorms_f16(const uint16_t *X, int64_t cols, int32_t d, float *out,
                                  hipStream_t st);
hipError_t launch_csr_row_sqnorms(const int32_t *indptr, const float *values, int64_t nq,
                                  int64_t nnz, float *out, hipStream_t st);
// Where a dense scan takes its queries from: the rows of a.Q; rows
// a.C[a.pick[i]] with the mask (the diversity step); the rows of a.Q with
// the mask (a step against explicit reference rows).  The masked forms rank
// by COS_MIN.
enum QueryMode : int { kQRows = 0, kQGatherMasked = 1, kQRowsMasked = 2 };

hipError_t launch_dense(const DenseArgs &a, int metric, int qmode, hipStream_t st, int n_cu);
// Queries-in-registers variant of the dense scan (d <= 256, no gather).
bool qreg_supports(int32_t d);
hipError_t launch_dense_qreg(const DenseArgs &a, int metric, hipStream_t st, int n_cu);
// 16-queries-per-wave variant (d <= 768, d % 4 == 0, 16-byte aligned rows);
// also runs the gathered, masked diversity step.
bool q16_supports(int32_t d, const float *C, const float *Q);
hipError_t launch_dense_q16(const DenseArgs &a, int metric, int qmode, hipStream_t st,
                            int n_cu);
// every dot product Q[q] . C[c] into a.S (same arithmetic as the scans)
hipError_t launch_dense_q16_store(const DenseArgs &a, hipStream_t st, int n_cu);
hipError_t launch_dense_qreg_store(const DenseArgs &a, hipStream_t st, int n_cu);
// per-row best of a score block into packed keys (the unfused comparator)
hipError_t launch_row_argbest(const float *S, int64_t nq, int64_t nc, int64_t ld_s,
                              const float *cn, uint64_t *keys, int metric, hipStream_t st);
// Q[s] += C[pick[s]] for every sequence whose pick is in [0, n)
hipError_t launch_div_accumulate(const float *C, int64_t n, int32_t d, const int32_t *pick,
                                 float *Q, int64_t nseq, hipStream_t st);
// one diversity step from a cached score block G (G[r * ldg + j] = C[r] . C[j]);
// with R (nseq x ldr running sums of Gram rows) the centroid reading:
// R[s] += G[pick[s]], then the masked arg-min of R[s]
hipError_t launch_div_gram_step(const float *G, int64_t n, int64_t ldg, const int32_t *pick,
                                uint32_t *mask, int64_t nseq, int32_t *idx_out,
                                float *score_out, hipStream_t st, float *R = nullptr,
                                int64_t ldr = 0);
// columns 0 .. n-1 of `rows` rows of stride ld set to 0 (a fill kernel, so a
// caller may capture it in a graph)
hipError_t launch_zero_rows(float *p, int64_t rows, int64_t ld, int64_t n, hipStream_t st);
// A whole run from G in one launch (masks of up to 32,768 columns): picks
// [steps x nseq] (and scores, optional) of the per-step kernel, bit for bit.
bool div_gram_run_supports(int64_t n);
hipError_t launch_div_gram_run(const float *G, int64_t n, int64_t ldg, const int32_t *seeds,
                               uint32_t *mask, int64_t nseq, int32_t steps, int32_t *picks,
                               float *scores, hipStream_t st, float *R = nullptr,
                               int64_t ldr = 0);
// CSR scan; `part` holds csr_groups(nc) x nq packed keys of scratch.
int32_t csr_groups(int64_t nc);
hipError_t launch_csr(const CsrArgs &a, int metric, hipStream_t st, int n_cu, uint64_t *part);
// CSR scan over the fp16 128-neuron blocked codebook (a.CT points at it,
// a.ldct = 128, a.cstride = d * 256)
hipError_t launch_csr_f16(const CsrArgs &a, int metric, hipStream_t st, int n_cu, uint64_t *part);
hipError_t launch_finalize(const uint64_t *keys, const float *qn, int64_t nq, int metric,
                           int32_t *idx_out, float *score_out, hipStream_t st);
hipError_t launch_finalize_div(const uint64_t *keys, int64_t nseq, uint32_t *mask,
                               int64_t mask_words, int32_t *idx_out, float *score_out,
                               hipStream_t st);

// Batch SOM update (som.hip).  The codebook and the S / T buffers are
// neuron-major (m * d + k) for dense rows, blocked feature-major
// ((m / 64) * 64 d + k * 64 + m % 64) for CSR rows.
struct SomArgs {
    bool csr;
    const float *X;                       // dense rows, n x d
    const int32_t *indptr, *indices;      // CSR rows
    const float *values;
    int64_t n;
    int32_t d;
    const int32_t *bmu;                   // n
    float *C;                             // codebook, updated in place
    int32_t rows, cols, R;                // map and window radius (R < max(rows, cols))
    double sigma;
    float *S, *T, *den_t, *rden, *g;      // workspace (rden: 1 / denominator, 0 where none)
    int32_t *cnt;
};
hipError_t launch_som_update(const SomArgs &a, hipStream_t st, int n_cu);
hipError_t launch_som_qe(const float *score, int64_t n, double *out, hipStream_t st);

// Timing hook (api.hip).
void timing_before(hipStream_t st, const char *name);
void timing_after(hipStream_t st);

}  // namespace vs
