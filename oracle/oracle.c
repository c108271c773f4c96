/*
 * oracle.c -- plain, slow CPU reference for the masked arg-reduction scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file; only the test-suite, the smoke check and the CPU leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library: every quantity is recomputed here from its definition in double
 * precision, one query at a time, candidates visited in ascending index order.
 *
 * What it computes (sources are web pages; cited by title and section):
 *
 *  - Best-matching-unit search: for every query, the candidate (neuron) that
 *    is closest to it, found exactly by brute force.  "From 80x to 385x: A
 *    Best-Matching-Unit Search at the L2 Roof ..." (summary), section 3
 *    "Background: the design being tuned": the BMU of each article is its
 *    closest neuron, the exact argmin does not depend on how the codebook is
 *    stored.
 *  - Farthest / most-different candidate: the diversity-sequence shader keeps,
 *    per sequence, the candidate with the largest cosine distance to its
 *    reference, skipping masked candidates.  "Issue 9-014: Tile Diversity
 *    Shader Inner Loop For L2 Cache Locality", sections "Current Behavior" and
 *    "Intended Behavior".  Largest cosine distance == smallest cosine, so the
 *    same scan with the order reversed covers it (metric COS_MIN).
 *  - SOM batch update and quantisation error around the BMU search (the
 *    same paper, section 3); see the notes at orc_som_update below.
 *  - The running best across the whole candidate range is a plain max/min:
 *    the same issue, "Intended Behavior" (associativity of max) and
 *    "Suggested Implementation Steps" (per-thread running best that is never
 *    reset).  Here there is one running best per query over all candidates.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - ties: the lowest candidate index wins (strict "<" in ascending order);
 *  - mask: bit j of a row of 32-bit words, least significant bit first, set
 *    means "excluded"; W = ceil(n/32) words per sequence;
 *  - cosine is the true cosine q.c / (|q| |c|) evaluated in double;
 *  - squared L2 is the direct form sum_k (q_k - c_k)^2 in double, k ascending;
 *  - the diversity reference vector is the sequence's last pick.
 *
 * Metric codes (same numbering as the public header, restated here on
 * purpose so the two sides share nothing):
 *   0 = squared L2, smallest wins      1 = squared L2, largest wins
 *   2 = cosine, largest wins           3 = cosine, smallest wins
 *
 * Non-vacuity: building with -DORC_MUTANT=<n> plants one deliberate mistake
 * (see the MUTANT notes below); the pins in tests/test_oracle.py must catch
 * every one of them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORC_MUTANT
#define ORC_MUTANT 0
#endif

enum { ORC_L2SQ_MIN = 0, ORC_L2SQ_MAX = 1, ORC_COS_MAX = 2, ORC_COS_MIN = 3 };

int orc_mutant(void) { return ORC_MUTANT; }

/* ---------------------------------------------------------------- pairs -- */

/* squared Euclidean distance, direct form, k ascending */
static double sq_l2(const float *q, const float *c, int64_t d)
{
    double s = 0.0;
    int64_t kend = d;
#if ORC_MUTANT == 4 /* MUTANT 4: drop the last coordinate */
    kend = d > 1 ? d - 1 : d;
#endif
    for (int64_t k = 0; k < kend; ++k) {
        double t = (double)q[k] - (double)c[k];
        s += t * t;
    }
    return s;
}

/* true cosine similarity */
static double cosine(const float *q, const float *c, int64_t d)
{
    double qq = 0.0, cc = 0.0, qc = 0.0;
    for (int64_t k = 0; k < d; ++k) {
        double a = (double)q[k], b = (double)c[k];
        qq += a * a;
        cc += b * b;
        qc += a * b;
    }
#if ORC_MUTANT == 6 /* MUTANT 6: forget to normalise */
    return qc;
#else
    return qc / (sqrt(qq) * sqrt(cc));
#endif
}

static double pair_value(const float *q, const float *c, int64_t d, int metric)
{
    return (metric == ORC_L2SQ_MIN || metric == ORC_L2SQ_MAX) ? sq_l2(q, c, d)
                                                              : cosine(q, c, d);
}

/* order key: smaller is better */
static double order_key(double s, int metric)
{
#if ORC_MUTANT == 3 /* MUTANT 3: treat every metric as "smallest wins" */
    (void)metric;
    return s;
#else
    return (metric == ORC_L2SQ_MIN || metric == ORC_COS_MIN) ? s : -s;
#endif
}

static int is_masked(const uint32_t *mask_row, int64_t j)
{
#if ORC_MUTANT == 5 /* MUTANT 5: ignore the mask */
    (void)mask_row;
    (void)j;
    return 0;
#else
    return mask_row != NULL && ((mask_row[j >> 5] >> (j & 31)) & 1u);
#endif
}

/* ------------------------------------------------------- running best -- */

typedef struct {
    double best, second; /* order keys */
    double value;        /* metric value of the best */
    int32_t idx;
} run_best;

static void rb_init(run_best *r)
{
    r->best = INFINITY;
    r->second = INFINITY;
    r->value = NAN;
    r->idx = -1;
}

/* Candidates must be offered in ascending index order. */
static void rb_offer(run_best *r, double key, double value, int64_t j)
{
#if ORC_MUTANT == 1 /* MUTANT 1: ties go to the highest index */
    if (key <= r->best) {
#else
    if (key < r->best) {
#endif
        r->second = r->best;
        r->best = key;
        r->value = value;
        r->idx = (int32_t)j;
    } else if (key < r->second) {
        r->second = key;
    }
}

static void rb_emit(const run_best *r, int32_t *idx, double *value, double *gap)
{
    *idx = r->idx;
    *value = r->value;
    /* top-two gap in key units; +inf when fewer than two candidates exist */
    *gap = (r->idx < 0 || isinf(r->second)) ? INFINITY : r->second - r->best;
}

/* ----------------------------------------------------------- dense scan -- */

/*
 * Dense scan: Q is nq x d, C is nc x d, both row-major fp32.  mask (nullable)
 * is nq rows of W = ceil(nc/32) words.  Outputs per query: winning index
 * (-1 when every candidate is masked), its metric value (NaN then) and the
 * top-two gap of the order key.
 */
void orc_dense(const float *Q, const float *C, int64_t nq, int64_t nc, int64_t d,
               int metric, const uint32_t *mask, int32_t *idx, double *value,
               double *gap)
{
    const int64_t W = (nc + 31) / 32;
    int64_t jend = nc;
#if ORC_MUTANT == 2 /* MUTANT 2: drop the last candidate (ragged-tail bug) */
    jend = nc > 1 ? nc - 1 : nc;
#endif
    for (int64_t i = 0; i < nq; ++i) {
        const float *q = Q + i * d;
        const uint32_t *mrow = mask ? mask + i * W : NULL;
        run_best r;
        rb_init(&r);
        for (int64_t j = 0; j < jend; ++j) {
            if (is_masked(mrow, j))
                continue;
            double s = pair_value(q, C + j * d, d, metric);
            rb_offer(&r, order_key(s, metric), s, j);
        }
        rb_emit(&r, idx + i, value + i, gap + i);
    }
}

/* metric value of given (query, candidate) pairs */
void orc_pair_values(const float *Q, const float *C, int64_t d, int metric,
                     int64_t npairs, const int64_t *qi, const int64_t *cj,
                     double *value)
{
    for (int64_t p = 0; p < npairs; ++p) {
#if ORC_MUTANT == 17 /* MUTANT 17: query and candidate indices exchanged */
        value[p] = pair_value(Q + cj[p] * d, C + qi[p] * d, d, metric);
#elif ORC_MUTANT == 18 /* MUTANT 18: candidate rows one float too short */
        value[p] = pair_value(Q + qi[p] * d, C + cj[p] * (d > 1 ? d - 1 : d), d, metric);
#else
        value[p] = pair_value(Q + qi[p] * d, C + cj[p] * d, d, metric);
#endif
    }
}

/* squared norms of rows (feature_major == 0: X is rows x d) or of columns
 * (feature_major != 0: X is d x rows, one column per candidate) */
void orc_sqnorms(const float *X, int64_t rows, int64_t d, int feature_major,
                 double *out)
{
    for (int64_t j = 0; j < rows; ++j) {
        double s = 0.0;
        for (int64_t k = 0; k < d; ++k) {
            double v = feature_major ? (double)X[k * rows + j] : (double)X[j * d + k];
            s += v * v;
        }
        out[j] = s;
    }
}

/* ------------------------------------------------------------- CSR scan -- */

/*
 * Sparse queries in CSR (indptr[nq+1], indices, values; column indices unique
 * within a row) against a feature-major codebook CT (d x nc, column j is
 * candidate j), as in the feature-major codebook of "From 80x to 385x ...",
 * section 3.  col_sq[j] = sum_k CT[k][j]^2 (from orc_sqnorms, feature-major).
 *
 * Squared L2 is still the plain definition sum_k (q_k - c_kj)^2: coordinates
 * where q is zero contribute c_kj^2, so
 *     s_j = col_sq[j] + sum_{(k,v) in row} ((v - c_kj)^2 - c_kj^2).
 * Cosine is (sum v c_kj) / (|q| sqrt(col_sq[j])).
 * acc has room for nc doubles (caller-provided scratch).
 */
void orc_csr(const int32_t *indptr, const int32_t *indices, const float *values,
             int64_t nq, const float *CT, int64_t nc, int64_t d, int metric,
             const double *col_sq, double *acc, int32_t *idx, double *value,
             double *gap)
{
    (void)d;
    const int is_l2 = (metric == ORC_L2SQ_MIN || metric == ORC_L2SQ_MAX);
    for (int64_t i = 0; i < nq; ++i) {
        double qq = 0.0;
        for (int64_t j = 0; j < nc; ++j)
#if ORC_MUTANT == 7 /* MUTANT 7: forget the untouched coordinates' |c|^2 */
            acc[j] = 0.0;
#else
            acc[j] = is_l2 ? col_sq[j] : 0.0;
#endif
        for (int64_t p = indptr[i]; p < indptr[i + 1]; ++p) {
            const double v = (double)values[p];
            const float *row = CT + (int64_t)indices[p] * nc;
            qq += v * v;
            if (is_l2) {
                for (int64_t j = 0; j < nc; ++j) {
                    const double c = (double)row[j];
                    acc[j] += (v - c) * (v - c) - c * c;
                }
            } else {
                for (int64_t j = 0; j < nc; ++j)
                    acc[j] += v * (double)row[j];
            }
        }
        run_best r;
        rb_init(&r);
        for (int64_t j = 0; j < nc; ++j) {
            double s = is_l2 ? acc[j] : acc[j] / (sqrt(qq) * sqrt(col_sq[j]));
            rb_offer(&r, order_key(s, metric), s, j);
        }
        rb_emit(&r, idx + i, value + i, gap + i);
    }
}

/* ---------------------------------------------------- diversity sequence -- */

/*
 * Greedy diversity sequence, run directly (no cache).  "Issue 9-014",
 * "Current Behavior": per iteration every sequence scans all candidate rows,
 * skips the ones its mask excludes and keeps the most different one; the
 * pick is then excluded for the rest of that sequence.  Reference vector:
 * the sequence's last pick; the seed is excluded before the first step.
 * picks/values are nseq x T (row-major); a step with nothing left gives -1.
 * mask_scratch needs W = ceil(n/32) words.
 */
void orc_div_run(const float *C, int64_t n, int64_t d, int64_t nseq, int T,
                 const int32_t *seeds, int32_t *picks, double *values,
                 uint32_t *mask_scratch)
{
    const int64_t W = (n + 31) / 32;
    for (int64_t s = 0; s < nseq; ++s) {
        memset(mask_scratch, 0, (size_t)W * sizeof(uint32_t));
        int32_t last = seeds[s];
#if ORC_MUTANT != 8 /* MUTANT 8: the seed is not excluded */
        mask_scratch[last >> 5] |= 1u << (last & 31);
#endif
        for (int t = 0; t < T; ++t) {
            run_best r;
            rb_init(&r);
            if (last >= 0) {
                for (int64_t j = 0; j < n; ++j) {
                    if (is_masked(mask_scratch, j))
                        continue;
                    double s_ = cosine(C + (int64_t)last * d, C + j * d, d);
                    rb_offer(&r, order_key(s_, ORC_COS_MIN), s_, j);
                }
            }
            picks[s * T + t] = r.idx;
            values[s * T + t] = r.value;
            if (r.idx >= 0)
                mask_scratch[r.idx >> 5] |= 1u << (r.idx & 31);
            last = r.idx;
        }
    }
}

/* rows [r0, r1) of the cosine Gram matrix G[i][j] = cos(C_i, C_j), n columns */
void orc_gram_cos(const float *C, int64_t n, int64_t d, int64_t r0, int64_t r1,
                  double *G)
{
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = 0; j < n; ++j)
            G[(i - r0) * n + j] = cosine(C + i * d, C + j * d, d);
}

/*
 * Replay of a recorded diversity run (e.g. one produced by the GPU) against
 * the cosine Gram matrix G (n x n, from orc_gram_cos).  For each sequence s
 * and step t the replay starts from the recorded prefix (seed plus recorded
 * picks before t), so one near-tie cannot cascade, and reports what the exact
 * step would have chosen: bidx, its cosine (best_value) and the top-two gap.
 * It also reports the cosine of the recorded pick (pick_value) and whether
 * the recorded pick was a legal choice (pick_ok: in range and not yet
 * excluded).  Arrays are nseq x T.  seen_scratch needs W = ceil(n/32) words.
 */
void orc_div_replay(const double *G, int64_t n, int64_t nseq, int T,
                    const int32_t *seeds, const int32_t *picks, int32_t *bidx,
                    double *best_value, double *gap, double *pick_value,
                    int32_t *pick_ok, uint32_t *seen_scratch)
{
    const int64_t W = (n + 31) / 32;
    for (int64_t s = 0; s < nseq; ++s) {
        memset(seen_scratch, 0, (size_t)W * sizeof(uint32_t));
        int32_t last = seeds[s];
#if ORC_MUTANT != 8
        seen_scratch[last >> 5] |= 1u << (last & 31);
#endif
        for (int t = 0; t < T; ++t) {
            const int64_t o = s * T + t;
            run_best r;
            rb_init(&r);
            if (last >= 0 && last < n) {
                const double *g = G + (int64_t)last * n;
                for (int64_t j = 0; j < n; ++j) {
                    if (is_masked(seen_scratch, j))
                        continue;
                    rb_offer(&r, order_key(g[j], ORC_COS_MIN), g[j], j);
                }
            }
            rb_emit(&r, bidx + o, best_value + o, gap + o);
            const int32_t p = picks[o];
            const int ok = p >= 0 && p < n && !((seen_scratch[p >> 5] >> (p & 31)) & 1u);
            pick_ok[o] = ok;
            pick_value[o] = (ok && last >= 0 && last < n) ? G[(int64_t)last * n + p] : NAN;
            if (p >= 0 && p < n)
#if ORC_MUTANT != 9 /* MUTANT 9: the replay forgets to exclude the pick */
                seen_scratch[p >> 5] |= 1u << (p & 31);
#else
                ;
#endif
            last = p;
        }
    }
}

/* ------------------------------------------------------ SOM batch update -- */
/*
 * One batch update of a self-organizing map around the BMU search.  "From
 * 80x to 385x ...", section 3 (workload): the search for every article's
 * BMU comes first; the update of the BMU and of the neurons around it on
 * the map follows.
 * The pages name no update rule; the readings taken here (all listed in the
 * design notes) are the batch map of the SOM literature:
 *  - the map is rows x cols, planar (no wrap-around); neuron m sits at grid
 *    row m / cols, column m % cols;
 *  - the neighbourhood weight of a BMU b on a neuron m is the Gaussian
 *    h(b, m) = exp(-(dy^2 + dx^2) / (2 sigma^2)) of their grid offset
 *    (dy, dx), taken as 0 outside the square window max(|dy|, |dx|) <= R;
 *  - every input pulls with weight h(bmu_i, m) at once:
 *        w_m <- sum_i h(bmu_i, m) x_i / sum_i h(bmu_i, m),
 *    and a neuron whose denominator is 0 keeps its weights;
 *  - an input whose BMU index lies outside [0, rows*cols) pulls nothing.
 * Inputs are CSR rows (a dense matrix is the CSR matrix holding every
 * entry); a column repeated within a row adds its values.  The definition is
 * evaluated directly, one requested neuron at a time, inputs in ascending
 * order, in double.  For each neuron the function also returns its
 * denominator and, per feature, sum_i h |x_ik| / den (the magnitude the
 * floating-point error of any summation order scales with; 0 when den = 0).
 *
 * MUTANT 10: window one step too narrow;  MUTANT 11: exp(-r^2 / sigma^2);
 * MUTANT 12: grid row taken as m / rows;   MUTANT 13: weights not normalised
 * by the Gaussian (den counts inputs).
 */
void orc_som_update(const int64_t *indptr, const int32_t *indices, const float *values,
                    int64_t n_in, int32_t d, const int32_t *bmu, int32_t rows, int32_t cols,
                    double sigma, int32_t radius, const int32_t *neurons, int64_t m,
                    const float *old_rows, double *w_out, double *mass_out, double *den_out)
{
    const int64_t nc = (int64_t)rows * cols;
#if ORC_MUTANT == 10
    const int64_t R = (int64_t)radius - 1;
#else
    const int64_t R = radius;
#endif
    for (int64_t t = 0; t < m; ++t) {
        const int64_t nm = neurons[t];
#if ORC_MUTANT == 12
        const int64_t ym = nm / rows, xm = nm % cols;
#else
        const int64_t ym = nm / cols, xm = nm % cols;
#endif
        double *num = w_out + t * d;
        double *mass = mass_out + t * d;
        for (int32_t k = 0; k < d; ++k)
            num[k] = mass[k] = 0.0;
        double den = 0.0;
        for (int64_t i = 0; i < n_in; ++i) {
            const int64_t b = bmu[i];
            if (b < 0 || b >= nc)
                continue;
#if ORC_MUTANT == 12
            const int64_t dy = b / rows - ym, dx = b % cols - xm;
#else
            const int64_t dy = b / cols - ym, dx = b % cols - xm;
#endif
            if (llabs(dy) > R || llabs(dx) > R)
                continue;
            const double r2 = (double)(dy * dy + dx * dx);
#if ORC_MUTANT == 11
            const double h = exp(-r2 / (sigma * sigma));
#else
            const double h = exp(-r2 / (2.0 * sigma * sigma));
#endif
#if ORC_MUTANT == 13
            den += 1.0;
#else
            den += h;
#endif
            for (int64_t p = indptr[i]; p < indptr[i + 1]; ++p) {
                const double v = (double)values[p];
                num[indices[p]] += h * v;
                mass[indices[p]] += h * fabs(v);
            }
        }
        den_out[t] = den;
        for (int32_t k = 0; k < d; ++k) {
            if (den > 0.0) {
                num[k] /= den;
                mass[k] /= den;
            } else {
                num[k] = (double)old_rows[t * d + k];
                mass[k] = 0.0;
            }
        }
    }
}

/*
 * Quantisation error of a map: the mean, over the inputs, of the Euclidean
 * distance from each input to its BMU's weight vector, measured before the
 * update ("From 80x to 385x ...", section 3 records it as the map's quality
 * figure; the mean Euclidean distance is the usual SOM definition, a
 * reading).  d2 holds each input's exact squared distance to its BMU (the
 * value the scans above return for squared L2); n = 0 gives NaN.
 * MUTANT 14: averages the squared distances.
 */
double orc_mean_sqrt(const double *d2, int64_t n)
{
    if (n <= 0)
        return NAN;
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
#if ORC_MUTANT == 14
        s += d2[i];
#else
        s += sqrt(d2[i] > 0.0 ? d2[i] : 0.0);
#endif
    return s / (double)n;
}

/* ------------------------------------------- centroid-reference diversity -- */
/*
 * The diversity run with the sequence's centroid as the reference: "Issue
 * 9-014 ...", "FP16 storage (compounding optimization)" speaks of the
 * candidate most different from the centroid.  Reading: after the seed and t
 * picks, the reference is the mean of those t+1 rows; each step takes the
 * unmasked row with the smallest true cosine to it (lowest index on ties) and
 * masks it.  A zero centroid has no direction: every candidate then scores 0
 * (so the lowest unmasked index wins).  Everything in double.
 *
 * MUTANT 15: the centroid leaves out the seed;  MUTANT 16: the centroid is
 * not accumulated (only the last pick is kept).
 */
static double cosine_ref(const float *c, const double *ref, int64_t d)
{
    double rr = 0.0, cc = 0.0, rc = 0.0;
    for (int64_t k = 0; k < d; ++k) {
        const double b = (double)c[k];
        rr += ref[k] * ref[k];
        cc += b * b;
        rc += ref[k] * b;
    }
    if (rr == 0.0 || cc == 0.0)
        return 0.0;
    return rc / (sqrt(rr) * sqrt(cc));
}

/* sum <- sum + row (double), or sum <- row when `reset` */
static void acc_row(double *sum, const float *row, int64_t d, int reset)
{
    for (int64_t k = 0; k < d; ++k)
        sum[k] = (reset ? 0.0 : sum[k]) + (double)row[k];
}

/* centroid of the seed and the first t picks of a prefix (invalid picks skipped) */
static void prefix_centroid(const float *C, int64_t n, int64_t d, int32_t seed,
                            const int32_t *picks, int t, double *cent)
{
    int64_t cnt = 0;
    for (int64_t k = 0; k < d; ++k)
        cent[k] = 0.0;
#if ORC_MUTANT != 15
    if (seed >= 0 && seed < n) {
        acc_row(cent, C + (int64_t)seed * d, d, 0);
        ++cnt;
    }
#endif
    for (int i = 0; i < t; ++i) {
        const int32_t p = picks[i];
        if (p < 0 || p >= n)
            continue;
#if ORC_MUTANT == 16
        acc_row(cent, C + (int64_t)p * d, d, 1);
        cnt = 1;
#else
        acc_row(cent, C + (int64_t)p * d, d, 0);
        ++cnt;
#endif
    }
    if (cnt > 0)
        for (int64_t k = 0; k < d; ++k)
            cent[k] /= (double)cnt;
}

/* nseq x T picks and cosines (to the centroid at that step) of the centroid run */
void orc_div_run_centroid(const float *C, int64_t n, int64_t d, int64_t nseq, int T,
                          const int32_t *seeds, int32_t *picks, double *values,
                          uint32_t *mask_scratch, double *cent)
{
    const int64_t W = (n + 31) / 32;
    for (int64_t s = 0; s < nseq; ++s) {
        memset(mask_scratch, 0, (size_t)W * sizeof(uint32_t));
        const int32_t seed = seeds[s];
        if (seed >= 0 && seed < n)
            mask_scratch[seed >> 5] |= 1u << (seed & 31);
        int32_t *ps = picks + s * T;
        for (int t = 0; t < T; ++t) {
            run_best r;
            rb_init(&r);
            prefix_centroid(C, n, d, seed, ps, t, cent);
            if (seed >= 0 && seed < n) {
                for (int64_t j = 0; j < n; ++j) {
                    if (is_masked(mask_scratch, j))
                        continue;
                    const double v = cosine_ref(C + j * d, cent, d);
                    rb_offer(&r, order_key(v, ORC_COS_MIN), v, j);
                }
            }
            ps[t] = r.idx;
            values[s * T + t] = r.value;
            if (r.idx >= 0)
                mask_scratch[r.idx >> 5] |= 1u << (r.idx & 31);
        }
    }
}

/*
 * Replay of a recorded centroid run: as orc_div_replay, with the reference of
 * step t the centroid of the recorded prefix (seed and recorded picks before
 * t).  Outputs per (sequence, step): the exact best index, its cosine, the
 * top-two gap, the recorded pick's cosine and whether that pick was legal.
 */
void orc_div_replay_centroid(const float *C, int64_t n, int64_t d, int64_t nseq, int T,
                             const int32_t *seeds, const int32_t *picks, int32_t *bidx,
                             double *best_value, double *gap, double *pick_value,
                             int32_t *pick_ok, uint32_t *seen_scratch, double *cent)
{
    const int64_t W = (n + 31) / 32;
    for (int64_t s = 0; s < nseq; ++s) {
        memset(seen_scratch, 0, (size_t)W * sizeof(uint32_t));
        const int32_t seed = seeds[s];
        const int seed_ok = seed >= 0 && seed < n;
        if (seed_ok)
            seen_scratch[seed >> 5] |= 1u << (seed & 31);
        const int32_t *ps = picks + s * T;
        for (int t = 0; t < T; ++t) {
            const int64_t o = s * T + t;
            run_best r;
            rb_init(&r);
            prefix_centroid(C, n, d, seed, ps, t, cent);
            if (seed_ok) {
                for (int64_t j = 0; j < n; ++j) {
                    if (is_masked(seen_scratch, j))
                        continue;
                    const double v = cosine_ref(C + j * d, cent, d);
                    rb_offer(&r, order_key(v, ORC_COS_MIN), v, j);
                }
            }
            rb_emit(&r, bidx + o, best_value + o, gap + o);
            const int32_t p = ps[t];
            const int ok = seed_ok && p >= 0 && p < n &&
                           !((seen_scratch[p >> 5] >> (p & 31)) & 1u);
            pick_ok[o] = ok;
            pick_value[o] = ok ? cosine_ref(C + (int64_t)p * d, cent, d) : NAN;
            if (p >= 0 && p < n)
                seen_scratch[p >> 5] |= 1u << (p & 31);
        }
    }
}
