// vs_launch.h -- host-side launchers of libvs's kernels (declarations only;
// included by vs_internal.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vs {

struct DenseArgs;
struct CsrArgs;

// Launchers (return hipError_t of the launch).  The dominant kernel of each
// entry point is bracketed by the library's timing events when recording.
hipError_t launch_fill_keys(uint64_t *keys, int64_t n, hipStream_t st);
// Dense search prologue in one launch: candidate norms (cn may be null),
// query norms (qn may be null) and the nq packed keys reset.
hipError_t launch_dense_prep(const float *C, int64_t nc, float *cn, const float *Q, int64_t nq,
                             float *qn, int32_t d, uint64_t *keys, hipStream_t st);
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
hipError_t launch_dense(const DenseArgs &a, int metric, int qmode, hipStream_t st, int n_cu);
// Queries-in-registers variant of the dense scan (d <= 256, no gather).
bool qreg_supports(int32_t d);
hipError_t launch_dense_qreg(const DenseArgs &a, int metric, hipStream_t st, int n_cu);
// 16-queries-per-wave variant (d <= 768, d % 4 == 0, 16-byte aligned rows);
// also runs the gathered, masked diversity step.
bool q16_supports(int32_t d, const float *C, const float *Q);
// Dense search of a small problem in two launches (bmu_small.hip): nq <=
// kSmallMaxQueries, nc <= kSmallMaxCandidates, d <= 256; small_supports adds
// d % 4 == 0 and 16-byte aligned rows.  Its workspace (small_workspace bytes
// at part): small_part_keys packed keys (nq * ceil(nc / 32), rounded up to
// 32), then nq query norms; every entry is written before it is read.
constexpr int64_t kSmallMaxQueries = 1024;
constexpr int64_t kSmallMaxCandidates = 2048;
int64_t small_part_keys(int64_t nq, int64_t nc);
size_t small_workspace(int64_t nq, int64_t nc);
bool small_shape(int64_t nq, int64_t nc, int32_t d);
bool small_supports(int64_t nq, int64_t nc, int32_t d, const float *Q, const float *C);
hipError_t launch_dense_small(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                              int metric, uint64_t *part, int32_t *idx_out, float *score_out,
                              hipStream_t st);
hipError_t launch_dense_q16(const DenseArgs &a, int metric, int qmode, hipStream_t st,
                            int n_cu);
// every dot product Q[q] . C[c] into a.S (same arithmetic as the scans)
// symmetric (Q == C, nq == nc): only the tiles at or right of each query
// tile's own rows are computed; those right of them also write their
// transpose, so every entry is written once
hipError_t launch_dense_q16_store(const DenseArgs &a, hipStream_t st, int n_cu,
                                  bool symmetric = false);
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
// reset: set every key back to "no candidate" once read (the next step of a
// run then needs no reset launch)
hipError_t launch_finalize_div(uint64_t *keys, int64_t nseq, uint32_t *mask,
                               int64_t mask_words, int32_t *idx_out, float *score_out,
                               hipStream_t st, bool reset);

// Batch SOM update (som.hip).  The codebook and the S / T buffers are
// neuron-major (m * d + k) for dense rows, blocked feature-major
// ((m / 64) * 64 d + k * 64 + m % 64) for CSR rows.
struct SomArgs {
    bool csr;
    const float *X;                       // dense rows, n x d
    const int32_t *indptr, *indices;      // CSR rows
    const float *values;
    int64_t nnz;                          // CSR entries the caller's arrays hold
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
