/*
 * vs.h -- C ABI of libvs: masked arg-reduction scans on AMD MI355X (gfx950).
 *
 * For every query vector the library finds the best row of a candidate
 * table -- nearest or farthest by squared Euclidean distance, or most/least
 * similar by cosine on unit-norm rows -- optionally skipping candidates a
 * per-query bit mask excludes, with the lowest candidate index winning ties.
 *
 * Sources (web pages, cited by title and section):
 *  [BMU] "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof,
 *        Measured Against a Symmetrically Tuned Baseline" (summary),
 *        section 3 "Background: the design being tuned": the best-matching
 *        unit of each article is its closest neuron; sparse articles against
 *        a feature-major codebook; the arg-reduction runs inside the
 *        contraction, and no matrix of scores is ever written out.
 *  [DIV] "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache
 *        Locality", "Current Behavior" and "Intended Behavior": per sequence,
 *        the unmasked candidate most different from the reference vector,
 *        which is then masked; a tiled scan must give the same winner as
 *        the untiled one.
 *
 * Conventions shared by every entry point
 *  - Device pointers are HIP device pointers owned by the caller.  The
 *    library never allocates, frees or retains them after the call's work
 *    has completed on `stream`.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Every call is asynchronous: it validates its arguments on the host,
 *    enqueues kernels on `stream` and returns.  Outputs are valid once the
 *    stream reaches the call.  Calls on one stream are ordered, so results
 *    of one call may feed the next without a host synchronisation.
 *  - Matrices are row-major and contiguous (row stride = number of columns).
 *    Any d >= 1 works; 16-byte vector loads are used when d % 4 == 0 and the
 *    matrix pointers are 16-byte aligned, 4-byte loads otherwise.
 *  - Inputs are assumed finite; NaN/Inf inputs give unspecified winners.
 *  - `workspace` is caller-provided device memory of at least the size the
 *    matching *_workspace() query returns, 256-byte aligned.  Its contents
 *    need no initialisation and are clobbered.  Two calls in flight at the
 *    same time must not share a workspace.
 *  - Return value: a vs_status.  The library never aborts, prints or throws.
 *    Arguments are checked before anything is enqueued; a failed check
 *    enqueues nothing.  A HIP launch failure returns VS_ERR_HIP and the HIP
 *    error code is kept, per calling thread, for vs_last_hip_error().
 *  - A query whose every candidate is masked gets index -1 and score NaN;
 *    this is not an error.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    on every call, independent of how the work is split across the GPU.
 *    The one exception is the SOM batch update (vs_som_update*, and the
 *    epochs that run it), whose per-neuron sums use float atomics: their
 *    last bits may differ from run to run (see there).
 */
#ifndef VS_H
#define VS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VS_OK = 0,
    VS_ERR_NULL = 1,        /* a required pointer is NULL                    */
    VS_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be,
                               or too large for 32-bit indices              */
    VS_ERR_METRIC = 3,      /* unknown metric code                           */
    VS_ERR_WORKSPACE = 4,   /* workspace smaller than *_workspace() returns  */
    VS_ERR_ALIGN = 5,       /* float/int pointer not 4-byte aligned, or
                               workspace not 256-byte aligned               */
    VS_ERR_INDEX = 6,       /* an index argument is out of range             */
    VS_ERR_UNSUPPORTED = 7, /* no GPU of a supported architecture            */
    VS_ERR_HIP = 8          /* a HIP call failed; see vs_last_hip_error()    */
} vs_status;

typedef enum {
    VS_L2SQ_MIN = 0, /* nearest by squared L2 (the BMU)              [BMU] */
    VS_L2SQ_MAX = 1, /* farthest by squared L2                             */
    VS_COS_MAX = 2,  /* most similar: rows unit-norm, score = dot          */
    VS_COS_MIN = 3   /* most different: rows unit-norm, score = dot [DIV]  */
} vs_metric;

/*
 * Dense search [BMU].
 *   Q          nq x d float32, queries.
 *   C          nc x d float32, candidates (codebook, one neuron per row).
 *   metric     a vs_metric.  COS_* assume unit-norm rows and rank by q.c.
 *   idx_out    int32[nq]: winning candidate per query (lowest index on ties).
 *   score_out  float32[nq] (may be NULL): squared distance of the winner
 *              (|q|^2 + |c|^2 - 2 q.c, clamped at 0) for L2SQ_*, q.c for COS_*.
 * nq == 0 is a no-op.  nc must be in [1, 2^31-1], d in [1, 2^20].
 * Workspace (vs_bmu_search_workspace): 8 nq bytes of packed keys, plus for
 * L2SQ_* 4 nq + 4 nc bytes of squared norms, each part rounded up to 256;
 * a search small enough for the two-launch small path (nq <= 1,024,
 * nc <= 2,048, d <= 256) needs instead, if that is more, its partial keys
 * (8 nq ceil(nc / 32) bytes, rounded up to 256) and 4 nq bytes of query
 * norms (rounded up to 256).  Its contents on entry do not
 * matter: every call writes what it reads.
 */
size_t vs_bmu_search_workspace(int64_t nq, int64_t nc, int32_t d, int32_t metric);
int vs_bmu_search(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                  int32_t metric, int32_t *idx_out, float *score_out, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * vs_bmu_search with no device allocation and no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results (bit for bit) as vs_bmu_search; the workspace is a
 * file-scope device array of the library, 8 MiB on every GPU the library
 * runs on, held until the process ends.  Limit: the workspace
 * vs_bmu_search_workspace(nq, nc, d, metric) would report must be at most
 * 8,388,608 bytes (for squared L2 about 12 nq + 4 nc bytes, each part
 * rounded up to 256: e.g. nq = 65,536 with nc up to 1,900,544; for cosine
 * 8 nq bytes; every small-path search fits), else VS_ERR_WORKSPACE before
 * anything is enqueued.  No
 * hipMalloc, hipFree or other allocating call is made; the first call on a
 * device looks up the array's device address once (hipGetSymbolAddress).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (each call rewrites what it reads before reading it), so calls
 * that overlap on one GPU -- concurrent streams, or threads -- race and
 * must be serialised by the caller.
 */
int vs_bmu_search_noalloc(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                          int32_t metric, int32_t *idx_out, float *score_out, void *stream);

/*
 * Unfused comparator for the dense search [BMU, section 3 (the unfused
 * GEMM-then-argmin path the fused search is measured against) and section 4]:
 * the same MFMA arithmetic writes the whole score block S[q * ld_s + c] =
 * Q[q] . C[c], then one pass per query ranks its row with the metric's rule.
 * Results equal vs_bmu_search's bit for bit.  Exists to measure what fusion
 * saves; S is caller-owned scratch of nq * ld_s floats (ld_s >= nc,
 * ld_s % 4 == 0, 16-byte aligned), overwritten.  Other arguments and the
 * workspace as for vs_bmu_search.  Needs d <= 256, or d <= 768 with d % 4 == 0
 * and 16-byte aligned Q and C (else VS_ERR_UNSUPPORTED).
 */
int vs_bmu_search_unfused(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                          int32_t metric, int32_t *idx_out, float *score_out, float *S,
                          int64_t ld_s, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sparse-query search over a feature-major codebook [BMU, section 3 and
 * section 4 "The levers"].
 *   indptr     int32[nq+1], indices int32[nnz], values float32[nnz]: CSR
 *              queries over d features.  Column indices must be unique within
 *              a row (their order is free).  Rows may be empty.
 *   CT         feature-major codebook: d rows of nc float32, row k holding
 *              feature k of every neuron (column j is neuron j).
 *   ldct       row stride of CT in elements (>= nc).  Rows are read in slices
 *              of a few neurons; a stride that is a multiple of a large power
 *              of two (e.g. nc = 65,536 unpadded) maps every row's slice onto
 *              the same cache sets, so pad it (e.g. ldct = nc + 64) for speed.
 *   metric, idx_out, score_out as for vs_bmu_search.
 * Device-side guard: a row whose indptr range is not inside [0, nnz] or
 * that holds a column index outside [0, d) is not scanned; it gets index -1
 * and score NaN.  Nothing outside the arrays is ever read.
 */
size_t vs_bmu_search_csr_workspace(int64_t nq, int64_t nc, int32_t d, int32_t metric);
int vs_bmu_search_csr(const int32_t *indptr, const int32_t *indices, const float *values,
                      int64_t nq, int64_t nnz, const float *CT, int64_t nc, int64_t ldct,
                      int32_t d, int32_t metric, int32_t *idx_out, float *score_out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * 64-neuron blocked codebook layout for the sparse-query search [BMU,
 * section 3 (feature-major storage) and section 4 "The levers" (neuron-axis
 * chunking)].  Feature k of neuron 64 b + j (0 <= j < 64) is stored at
 * CB[(b * d + k) * 64 + j]: each block is a d x 64 feature-major matrix, so
 * the codebook slice one 64-neuron chunk of the search reads is contiguous
 * (a few large pages) instead of d row segments spread over the whole
 * feature-major array, which costs address-translation misses.
 *   vs_csr_blocked_bytes   size of CB in bytes: ceil(nc / 64) * 64 * d * 4
 *                          (0 for invalid sizes).  Host-only.
 *   vs_csr_block_codebook  writes CB from a feature-major CT (d rows of nc,
 *                          row stride ldct >= nc); columns past nc in the
 *                          last block are written as 0.  CB is caller-owned
 *                          device memory of vs_csr_blocked_bytes bytes;
 *                          CT and CB must not overlap.
 *   vs_bmu_search_csr_blocked  vs_bmu_search_csr over CB; same arguments
 *                          otherwise (workspace: vs_bmu_search_csr_workspace)
 *                          and bit-identical results.
 */
size_t vs_csr_blocked_bytes(int64_t nc, int32_t d);
int vs_csr_block_codebook(const float *CT, int64_t nc, int64_t ldct, int32_t d, float *CB,
                          void *stream);
int vs_bmu_search_csr_blocked(const int32_t *indptr, const int32_t *indices,
                              const float *values, int64_t nq, int64_t nnz, const float *CB,
                              int64_t nc, int32_t d, int32_t metric, int32_t *idx_out,
                              float *score_out, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * fp16 storage of the sparse-query search's codebook, fp32 arithmetic
 * ["Issue 9-014", "FP16 storage (compounding optimization)": store the table
 * in half precision, load FP16 and compute FP32; BMU, section 4 "The levers"
 * (vectorised loads)].  The codebook is held as IEEE binary16 in a
 * 128-neuron blocked layout: feature k of neuron 128 b + j (0 <= j < 128) at
 * CB16[(b * d + k) * 128 + j].  Every value is widened exactly to fp32 before
 * it is multiplied, and sums, norms and scores are fp32, so the results are
 * those of vs_bmu_search_csr over the fp16-rounded codebook, bit for bit;
 * the codebook bytes (the scan's roof) are halved.
 *   vs_csr_blocked_f16_bytes   size of CB16 in bytes: ceil(nc / 128) * 128
 *                              * d * 2 (0 for invalid sizes).  Host-only.
 *   vs_csr_block_codebook_f16  writes CB16 from a feature-major fp32 CT (d
 *                              rows of nc, row stride ldct >= nc), rounding
 *                              to nearest even; columns past nc are 0.
 *                              CB16 must be 16-byte aligned, caller-owned.
 *   vs_bmu_search_csr_blocked_f16  the search over CB16; other arguments and
 *                              workspace as for vs_bmu_search_csr.
 */
size_t vs_csr_blocked_f16_bytes(int64_t nc, int32_t d);
int vs_csr_block_codebook_f16(const float *CT, int64_t nc, int64_t ldct, int32_t d,
                              uint16_t *CB16, void *stream);
/*
 * The same fp16 128-neuron blocked copy, made from the 64-neuron blocked fp32
 * codebook CB (the layout vs_csr_block_codebook writes and the SOM update
 * keeps) instead of the plain feature-major one: bit-identical to
 * vs_csr_block_codebook_f16 of the same values.  CB16 16-byte aligned,
 * vs_csr_blocked_f16_bytes(nc, d) bytes.
 */
int vs_csr_blocked_to_f16(const float *CB, int64_t nc, int32_t d, uint16_t *CB16, void *stream);
int vs_bmu_search_csr_blocked_f16(const int32_t *indptr, const int32_t *indices,
                                  const float *values, int64_t nq, int64_t nnz,
                                  const uint16_t *CB16, int64_t nc, int32_t d, int32_t metric,
                                  int32_t *idx_out, float *score_out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * One step of the greedy diversity sequence [DIV] for nseq sequences at once.
 *   C          n x d float32, unit-norm rows (the embedding table).
 *   last_pick  int32[nseq]: each sequence's reference row (its last pick).
 *   mask_bits  uint32[nseq][W], W = ceil(n/32), in/out: bit j (word j/32,
 *              bit j%32, least significant first) set = row j excluded.
 *              Bits at or above n are never read.
 *   idx_out    int32[nseq]: the unmasked row with the smallest cosine to the
 *              reference (lowest index on ties); its bit is then set in the
 *              sequence's mask.  -1 if every row is masked or last_pick is
 *              outside [0, n) (then the mask is left unchanged).
 *   score_out  float32[nseq] or NULL: cosine (dot) of the pick.
 * idx_out may alias last_pick, so a chain of steps can reuse one buffer.
 */
size_t vs_diversity_step_workspace(int64_t n, int32_t d, int64_t nseq);
int vs_diversity_step(const float *C, int64_t n, int32_t d, const int32_t *last_pick,
                      uint32_t *mask_bits, int64_t nseq, int32_t *idx_out, float *score_out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * A whole diversity run [DIV "Current Behavior": the driver repeats the
 * step, each iteration's picks becoming the next one's references]: `steps`
 * calls of vs_diversity_step chained on the stream, step t's last_pick
 * being step t-1's picks (seeds for t = 0).  mask_bits as for the step (the
 * seeds' bits set by the caller), updated in place; picks_out int32[steps x
 * nseq] (row t = step t), scores_out float32[steps x nseq] or NULL.  Same
 * workspace as vs_diversity_step.  Results equal those of the steps called
 * one by one, bit for bit.
 */
int vs_diversity_run(const float *C, int64_t n, int32_t d, const int32_t *seeds,
                     uint32_t *mask_bits, int64_t nseq, int32_t steps, int32_t *picks_out,
                     float *scores_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The diversity step against explicit reference rows [DIV "Current
 * Behavior"; "FP16 storage (compounding optimization)" ranks candidates
 * against the sequence's centroid].
 *   vs_diversity_step_ref    as vs_diversity_step, with sequence s ranked
 *                            against Q[s] (nseq x d, float32, row-major)
 *                            instead of C[last_pick[s]]: the unmasked row j
 *                            of C with the smallest C[j] . Q[s] (lowest index
 *                            on ties) is picked and its bit set.  C's rows
 *                            unit-norm: that is the smallest cosine to Q[s],
 *                            for any positive scale of Q[s].  score_out =
 *                            C[pick] . Q[s].  Workspace as vs_diversity_step.
 *   vs_diversity_accumulate  Q[s] += C[pick[s]] for every s whose pick is in
 *                            [0, n) (others unchanged): with Q[s] started at
 *                            the seed's row it holds the sum of the sequence
 *                            so far, i.e. its centroid times a positive count,
 *                            so a chain step_ref / accumulate is the centroid
 *                            reading.  No workspace.
 */
int vs_diversity_step_ref(const float *C, int64_t n, int32_t d, const float *Q,
                          uint32_t *mask_bits, int64_t nseq, int32_t *idx_out, float *score_out,
                          void *workspace, size_t workspace_bytes, void *stream);
int vs_diversity_accumulate(const float *C, int64_t n, int32_t d, const int32_t *pick, float *Q,
                            int64_t nseq, void *stream);
/*
 *   vs_diversity_run_ref     a whole centroid-reading run with explicit
 *                            references, as vs_diversity_run: Q (nseq x d
 *                            float32, caller-owned) is set to the seeds' rows,
 *                            then each step is vs_diversity_step_ref followed
 *                            by vs_diversity_accumulate of its picks; on
 *                            return Q holds each sequence's sum of rows.
 *                            Workspace as vs_diversity_step.
 */
int vs_diversity_run_ref(const float *C, int64_t n, int32_t d, const int32_t *seeds, float *Q,
                         uint32_t *mask_bits, int64_t nseq, int32_t steps, int32_t *picks_out,
                         float *scores_out, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * The diversity step from a cached Gram matrix [DIV "Current Behavior"; the
 * reference of a step is the sequence's last pick, so every score a run can
 * need is an entry of G = C C^T].
 *   vs_diversity_gram       writes G[r * ldg + j] = C[r] . C[j] (fp32) for
 *                           r, j < n, by the same MFMA arithmetic and
 *                           per-pair order as vs_diversity_step, so each
 *                           entry equals bit for bit the dot product that
 *                           call ranks.  C is n x d, unit-norm rows; needs
 *                           d % 4 == 0, d <= 768 and C 16-byte aligned
 *                           (else VS_ERR_UNSUPPORTED).  G is caller-owned,
 *                           n * ldg floats, 16-byte aligned; ldg >= n and
 *                           ldg % 4 == 0; columns n .. ldg-1 are not written.
 *   vs_diversity_step_gram  one step for nseq sequences from G: arguments,
 *                           mask semantics and results as vs_diversity_step
 *                           (bit-identical picks, scores and masks); reads
 *                           one row of G per sequence.  No workspace.
 */
int vs_diversity_gram(const float *C, int64_t n, int32_t d, float *G, int64_t ldg,
                      void *stream);
/*
 *   vs_diversity_step_gram_sum  the centroid reading from G [DIV, "FP16
 *                           storage (compounding optimization)": the
 *                           reference is the sequence's centroid].  C's rows
 *                           unit-norm: C[j] . sum_p C[p] = sum_p G[p][j], so
 *                           a run keeps R (nseq x ldr float32, ldr >= n,
 *                           ldr % 4 == 0, 16-byte aligned, all zero before
 *                           its first step) and each call first adds the
 *                           reference's row, R[s] += G[last_pick[s]] (for
 *                           the first step last_pick is the seed), then picks
 *                           the unmasked j with the smallest R[s][j] (lowest
 *                           index on ties), sets its bit, and reports
 *                           score_out = R[s][pick].  Columns already masked
 *                           are never candidates again and their entries of
 *                           R[s] hold unspecified values (the scan works on
 *                           groups of four columns and skips a group only
 *                           when all four are masked).  last_pick outside
 *                           [0, n): -1, mask and R[s] unchanged.  No
 *                           workspace.
 */
int vs_diversity_step_gram_sum(const float *G, int64_t n, int64_t ldg, const int32_t *last_pick,
                               float *R, int64_t ldr, uint32_t *mask_bits, int64_t nseq,
                               int32_t *idx_out, float *score_out, void *stream);
/*
 *   vs_diversity_run_gram   a whole run from G, as vs_diversity_run: with R
 *                           NULL the last-pick reading (vs_diversity_step_gram
 *                           per step), else the centroid reading
 *                           (vs_diversity_step_gram_sum per step; R as there,
 *                           cleared by this call before the first step).
 */
int vs_diversity_run_gram(const float *G, int64_t n, int64_t ldg, const int32_t *seeds,
                          float *R, int64_t ldr, uint32_t *mask_bits, int64_t nseq,
                          int32_t steps, int32_t *picks_out, float *scores_out, void *stream);
int vs_diversity_step_gram(const float *G, int64_t n, int64_t ldg, const int32_t *last_pick,
                           uint32_t *mask_bits, int64_t nseq, int32_t *idx_out,
                           float *score_out, void *stream);

/*
 * SOM epoch around the BMU search [BMU section 3: each input's closest
 * neuron is found first, then that neuron and its neighbours are updated;
 * the update rule is not given there, these calls take the batch map].
 * The map is rows x cols neurons, planar; neuron m sits at grid row m / cols,
 * column m % cols.  The neighbourhood weight of a BMU b on neuron m is
 * h = exp(-(dy^2 + dx^2) / (2 sigma^2)) of their grid offset inside the
 * square window max(|dy|, |dx|) <= radius, 0 outside, and the update is
 *     w_m <- sum_i h(bmu_i, m) x_i / sum_i h(bmu_i, m)
 * for every neuron whose denominator is > 0 (the others keep their weights).
 * Inputs whose BMU lies outside [0, rows*cols) pull nothing.  sigma > 0 and
 * finite; radius >= 0 and, unless 0, <= 8 sigma (so every weight in the
 * window stays a normal fp32 number); else VS_ERR_SHAPE.  Arithmetic is
 * fp32 with float atomics for the per-neuron sums: results agree with the
 * exact update to a few units of fp32 rounding per summed term, and their
 * last bits can differ from run to run.
 *   vs_som_update      dense rows X (n x d) and bmu int32[n]; C (rows*cols x
 *                      d, neuron-major) is updated in place.
 *   vs_som_update_csr  CSR rows (as vs_bmu_search_csr; entries with a
 *                      column outside [0, d) are skipped, and a row whose
 *                      span indptr[i] .. indptr[i+1] is not inside
 *                      [0, nnz] pulls nothing, whatever its BMU; nothing
 *                      outside the arrays is read); CB is the
 *                      64-neuron blocked codebook of vs_csr_block_codebook,
 *                      updated in place.
 *   vs_som_qe          quantisation error: mean over the n inputs of
 *                      sqrt(max(score, 0)), score = squared distance to the
 *                      BMU as the searches return it; summed in double in a
 *                      fixed order; NaN for n = 0.  qe_out: one double in
 *                      device memory (8-byte aligned).
 *   vs_som_epoch       dense rows: vs_bmu_search (squared L2) into bmu_out /
 *                      score_out (caller-owned int32[n] / float32[n], may be
 *                      NULL when n = 0), then
 *                      vs_som_qe into qe_out (may be NULL), then
 *                      vs_som_update of C.
 *   vs_som_epoch_csr   the same for CSR rows over the blocked codebook CB
 *                      (vs_bmu_search_csr_blocked, vs_som_update_csr).
 * Workspace: 256-byte aligned, at least the matching *_workspace() bytes
 * (two rows*cols x d float buffers plus O(rows*cols); the epochs add the
 * search's).  The workspace functions return 0 for invalid sizes.
 */
size_t vs_som_update_workspace(int32_t map_rows, int32_t map_cols, int32_t d);
int vs_som_update(const float *X, int64_t n, int32_t d, const int32_t *bmu, float *C,
                  int32_t map_rows, int32_t map_cols, float sigma, int32_t radius,
                  void *workspace, size_t workspace_bytes, void *stream);
int vs_som_update_csr(const int32_t *indptr, const int32_t *indices, const float *values,
                      int64_t n, int64_t nnz, const int32_t *bmu, float *CB, int32_t map_rows,
                      int32_t map_cols, int32_t d, float sigma, int32_t radius, void *workspace,
                      size_t workspace_bytes, void *stream);
int vs_som_qe(const float *score, int64_t n, double *qe_out, void *stream);
size_t vs_som_epoch_workspace(int64_t n, int32_t map_rows, int32_t map_cols, int32_t d);
int vs_som_epoch(const float *X, int64_t n, int32_t d, float *C, int32_t map_rows,
                 int32_t map_cols, float sigma, int32_t radius, int32_t *bmu_out,
                 float *score_out, double *qe_out, void *workspace, size_t workspace_bytes,
                 void *stream);
size_t vs_som_epoch_csr_workspace(int64_t n, int32_t map_rows, int32_t map_cols, int32_t d);
int vs_som_epoch_csr(const int32_t *indptr, const int32_t *indices, const float *values,
                     int64_t n, int64_t nnz, float *CB, int32_t map_rows, int32_t map_cols,
                     int32_t d, float sigma, int32_t radius, int32_t *bmu_out, float *score_out,
                     double *qe_out, void *workspace, size_t workspace_bytes, void *stream);
/*
 *   vs_som_epoch_csr_f16  the CSR epoch with the search over an fp16 copy of
 *                      the codebook [Issue "FP16 storage (compounding
 *                      optimization)": load half, compute fp32]:
 *                      vs_csr_blocked_to_f16 of CB into CB16 (caller-owned,
 *                      vs_csr_blocked_f16_bytes), vs_bmu_search_csr_blocked_f16,
 *                      vs_som_qe, then vs_som_update_csr of the fp32 CB.  BMUs
 *                      and the error are those of the fp16-rounded codebook;
 *                      the update keeps full fp32 weights.  Workspace as
 *                      vs_som_epoch_csr.
 */
int vs_som_epoch_csr_f16(const int32_t *indptr, const int32_t *indices, const float *values,
                         int64_t n, int64_t nnz, float *CB, uint16_t *CB16, int32_t map_rows,
                         int32_t map_cols, int32_t d, float sigma, int32_t radius,
                         int32_t *bmu_out, float *score_out, double *qe_out, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Squared L2 norms of candidates, float32, fixed summation order (the same
 * values the searches use).  feature_major == 0: C is nc x d (row j);
 * otherwise C is d x nc (column j).  norms_out is float32[nc].
 * [Issue 9-014, "FP16 storage path": the norm accumulators of the distance
 * loop stay fp32 whatever the storage type; "From 80x to 385x ...",
 * section 3: squared-L2 BMU search, the codebook held feature-major.  The
 * pages compute the norms inside the scan; this call hoists the candidates'
 * norms out of it so the scan ranks by |c|^2 - 2 q.c.]
 */
int vs_candidate_norms(const float *C, int64_t nc, int32_t d, int32_t feature_major,
                       float *norms_out, void *stream);

/*
 * Candidate tile rows that fit a cache with headroom: floor(cache_bytes *
 * 0.85 / (d * bytes_per_value)), at least 1 ["Issue 9-014", "Intended
 * Behavior" and "Suggested Implementation Steps"].  Host-only.  Returns 0
 * for invalid arguments.
 */
int64_t vs_tile_rows(int64_t cache_bytes, int32_t d, int32_t bytes_per_value);

/*
 * Measurement hook (host-only bookkeeping, no device memory): while enabled,
 * the dominant kernel of each call is bracketed by a pair of HIP events on
 * the call's stream.  vs_timing_enable(max_launches) (re)starts recording
 * for up to max_launches launches (0 disables); vs_timing_read() waits for
 * the recorded events, returns the summed kernel time in milliseconds and the
 * number of launches, and stops recording.  Kernel names: see
 * vs_timing_kernel_name().
 */
int vs_timing_enable(int32_t max_launches);
int vs_timing_read(double *total_ms, int64_t *launches);
const char *vs_timing_kernel_name(void);

const char *vs_status_str(int status);
int vs_last_hip_error(void);
const char *vs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VS_H */
