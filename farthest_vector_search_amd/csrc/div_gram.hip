// div_gram.hip -- the diversity step from a cached Gram matrix.
//
// "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
// "Current Behavior": every step ranks, for each sequence, all unmasked rows
// by their cosine to the sequence's reference and picks the most different
// one.  With the last pick as the reference, every score a run can need is
// an entry of the table's Gram matrix G = C C^T, so G is computed once (by
// the same MFMA arithmetic as the per-step scan, so each entry equals, bit
// for bit, the dot product the scan would rank) and a step becomes a masked
// arg-min over one row of G per sequence: an HBM-bound read of n floats
// instead of a d-long dot product per candidate.
//
// Lanes read the reference's row four floats at a time (lane l of a wave:
// columns 4 l .. 4 l + 3 of each 256-column segment the wave owns), skip
// masked and padded columns, keep the lowest value with strict "<" (so the
// lowest index among equal values), then (value, index) pairs are merged
// lexicographically.  -0 and +0 compare equal and the score is reported
// with the sign folded, as the packed-key path does; NaN is never picked.
// A lane whose four columns are all masked does not load them, so as a run
// fills its masks (a full-length run ends with every bit set) the HBM bytes
// of a step fall with the number of candidates left.
#include "vs_internal.h"

namespace vs {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One workgroup of kWPS waves per sequence: wave w scans the 256-column
// segments w, w + kWPS, ... (so a step has kWPS x nseq waves in flight to
// hide the row loads' latency), then the waves' (value, index) pairs are
// merged through LDS; the order of a lexicographic minimum is immaterial, so
// the pick equals the one-wave scan's.
//
// SUM: the centroid reading.  C's rows are unit-norm, so the cosine to a
// sequence's centroid ranks candidates as C[j] . sum_p C[p] = sum_p G[p][j]
// does (p over the sequence's rows so far); R[s] keeps that running sum of
// Gram rows.  A step first adds the reference's row, R[s] += G[pick[s]],
// then takes the masked arg-min of R[s].  Masked columns are never candidates
// again, so their entries of R[s] are left unspecified: a group of four
// columns is skipped only when all four are masked, otherwise the whole
// group's sums are read and updated.
constexpr int kWPS = 4;

template <bool SUM>
__global__ __launch_bounds__(64 * kWPS) void k_div_gram_step(const float *__restrict__ G,
                                                            int64_t n, int64_t ldg,
                                                            const int32_t *__restrict__ pick,
                                                            uint32_t *__restrict__ mask,
                                                            int64_t nseq,
                                                            int32_t *__restrict__ idx_out,
                                                            float *__restrict__ score_out,
                                                            float *__restrict__ R, int64_t ldr) {
    __shared__ float s_best[kWPS];
    __shared__ int64_t s_idx[kWPS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t W = (n + 31) / 32;
    // sequences s = blockIdx.x, + gridDim.x, ...: every branch below is
    // uniform over the workgroup, so all its waves meet every barrier
    for (int64_t s = blockIdx.x; s < nseq; s += gridDim.x) {
        const int64_t r = pick[s];
        if (r < 0 || r >= n) {  // no reference: no pick, mask unchanged
            if (threadIdx.x == 0) {
                idx_out[s] = -1;
                if (score_out) score_out[s] = __builtin_nanf("");
            }
            continue;
        }
        const float *row = G + r * ldg;
        const uint32_t *mrow = mask + s * W;
        float best = __builtin_inff();
        int64_t bidx = -1;
        // the mask word of the next segment is fetched one iteration ahead
        // (unconditionally, at a clamped in-range column, so that the compiler's
        // wait before the row load does not also wait for it): a segment's row
        // load never waits for its own mask load
        constexpr int64_t kStep = 256 * kWPS;
        int64_t j0 = 256 * (int64_t)wave + 4 * (int64_t)lane;
        uint32_t mw = mrow[(j0 < n ? j0 : n - 1) >> 5];
        for (; j0 < n; j0 += kStep) {
            const int64_t jn = j0 + kStep;
            const uint32_t mw_next = mrow[(jn < n ? jn : n - 1) >> 5];
            // j0 % 32 <= 28: the four columns' bits sit in one mask word
            const int64_t left = n - j0;
            uint32_t live4 = ~(mw >> (j0 & 31)) & 0xFu;
            mw = mw_next;
            if (left < 4) live4 &= (1u << left) - 1u;
            if (live4 == 0) continue;
            // ld % 4 == 0 and G 16-byte aligned: columns j0 .. j0 + 3 are in the
            // row's padded storage even past n
            f32x4 v = *reinterpret_cast<const f32x4 *>(row + j0);
        if constexpr (SUM) {
            // ldr % 4 == 0 and R 16-byte aligned, as for G
            f32x4 *rp = reinterpret_cast<f32x4 *>(R + s * ldr + j0);
            v += *rp;
            *rp = v;
        }
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = v[e];
                if (((live4 >> e) & 1u) && x < best) {
                    best = x;
                    bidx = j0 + e;
                }
            }
        }
        auto better = [](float ob, int64_t oi, float b, int64_t i) {
            return oi >= 0 && (i < 0 || ob < b || (ob == b && oi < i));
        };
    #pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ob = __shfl_xor(best, off);
            const int64_t oi = __shfl_xor(bidx, off);
            if (better(ob, oi, best, bidx)) {
                best = ob;
                bidx = oi;
            }
        }
        if (lane == 0) {
            s_best[wave] = best;
            s_idx[wave] = bidx;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < kWPS; ++w)
                if (better(s_best[w], s_idx[w], best, bidx)) {
                    best = s_best[w];
                    bidx = s_idx[w];
                }
            if (bidx < 0) {
                idx_out[s] = -1;
                if (score_out) score_out[s] = __builtin_nanf("");
            } else {
                idx_out[s] = (int32_t)bidx;
                if (score_out) score_out[s] = best == 0.0f ? 0.0f : best;
                mask[s * W + (bidx >> 5)] |= 1u << (bidx & 31);
            }
        }
        __syncthreads();  // s_best / s_idx are rewritten by the next sequence
    }
}

hipError_t launch_div_gram_step(const float *G, int64_t n, int64_t ldg, const int32_t *pick,
                                uint32_t *mask, int64_t nseq, int32_t *idx_out,
                                float *score_out, hipStream_t st, float *R, int64_t ldr) {
    if (nseq <= 0) return hipSuccess;
    const unsigned grid = (unsigned)(nseq < (1 << 20) ? nseq : (1 << 20));
    if (R) {
        timing_before(st, "k_div_gram_step<sum>");
        hipLaunchKernelGGL(k_div_gram_step<true>, dim3(grid), dim3(64 * kWPS), 0, st, G, n, ldg,
                           pick, mask, nseq, idx_out, score_out, R, ldr);
    } else {
        timing_before(st, "k_div_gram_step");
        hipLaunchKernelGGL(k_div_gram_step<false>, dim3(grid), dim3(64 * kWPS), 0, st, G, n, ldg,
                           pick, mask, nseq, idx_out, score_out, R, ldr);
    }
    const hipError_t err = hipGetLastError();
    timing_after(st);
    return err;
}

// A whole run in one launch: one workgroup of kWPS waves per sequence
// (grid-stride over sequences) takes all `steps` steps of its sequence, the
// pick of step t becoming the reference of step t + 1.  Sequences never
// interact, so no step needs a grid-wide barrier, and the launch gap between
// per-step kernels disappears.  The sequence's mask row (W <= kRunWords
// words) lives in LDS for the run and is written back at its end.  Each
// step is the per-step kernel's scan: the same columns per lane (visited in
// ascending order, two segments per iteration so that two row loads are in
// flight), the same strict compares and lexicographic merge, and with SUM
// the same one add per live column and step, so picks, scores, masks and R
// are those of the per-step kernel, bit for bit.  A reference outside
// [0, n) (or a step that finds no unmasked column) makes that step and all
// later ones report -1 (score NaN) with mask and R unchanged, as a chain of
// per-step calls does.
constexpr int kRunWords = 1024;  // mask rows of up to 32,768 columns

template <bool SUM>
__global__ __launch_bounds__(64 * kWPS) void k_div_gram_run(
    const float *__restrict__ G, int64_t n, int64_t ldg, const int32_t *__restrict__ seeds,
    uint32_t *__restrict__ mask, int64_t nseq, int32_t steps, int32_t *__restrict__ picks,
    float *__restrict__ scores, float *__restrict__ R, int64_t ldr) {
    __shared__ uint32_t s_mask[kRunWords];
    __shared__ float s_best[kWPS];
    __shared__ int32_t s_idx[kWPS];
    __shared__ int32_t s_ref;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t nn = (int32_t)n;
    const int32_t W = (nn + 31) / 32;
    constexpr int32_t kStep = 256 * kWPS;
    auto live_of = [&](int32_t j) -> uint32_t {  // live columns j .. j + 3 (bit e: column j + e)
        if (j >= nn) return 0u;
        // j % 32 <= 28: the four columns' bits sit in one mask word
        uint32_t live4 = ~(s_mask[j >> 5] >> (j & 31)) & 0xFu;
        const int32_t left = nn - j;
        if (left < 4) live4 &= (1u << left) - 1u;
        return live4;
    };
    for (int64_t s = blockIdx.x; s < nseq; s += gridDim.x) {
        uint32_t *mrow = mask + s * W;
        for (int32_t i = threadIdx.x; i < W; i += 64 * kWPS) s_mask[i] = mrow[i];
        int32_t r = seeds[s];
        __syncthreads();
        for (int32_t t = 0; t < steps; ++t) {
            if (r < 0 || r >= nn) {  // uniform: no reference from here on
                for (int32_t u = t + (int32_t)threadIdx.x; u < steps; u += 64 * kWPS) {
                    picks[(int64_t)u * nseq + s] = -1;
                    if (scores) scores[(int64_t)u * nseq + s] = __builtin_nanf("");
                }
                break;
            }
            const float *row = G + (int64_t)r * ldg;
            float *rrow = SUM ? R + s * ldr : nullptr;
            float best = __builtin_inff();
            int32_t bidx = -1;
            for (int32_t j0 = 256 * wave + 4 * lane; j0 < nn; j0 += 2 * kStep) {
                const int32_t j1 = j0 + kStep;
                const uint32_t la = live_of(j0), lb = live_of(j1);
                // ld % 4 == 0 and G 16-byte aligned: columns j .. j + 3 are in
                // the row's padded storage even past n
                f32x4 va = {0.0f, 0.0f, 0.0f, 0.0f}, vb = va;
                if (la) va = *reinterpret_cast<const f32x4 *>(row + j0);
                if (lb) vb = *reinterpret_cast<const f32x4 *>(row + j1);
                if constexpr (SUM) {
                    if (la) {
                        f32x4 *rp = reinterpret_cast<f32x4 *>(rrow + j0);
                        va += *rp;
                        *rp = va;
                    }
                    if (lb) {
                        f32x4 *rp = reinterpret_cast<f32x4 *>(rrow + j1);
                        vb += *rp;
                        *rp = vb;
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (((la >> e) & 1u) && va[e] < best) {
                        best = va[e];
                        bidx = j0 + e;
                    }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (((lb >> e) & 1u) && vb[e] < best) {
                        best = vb[e];
                        bidx = j1 + e;
                    }
            }
            auto better = [](float ob, int32_t oi, float b, int32_t i) {
                return oi >= 0 && (i < 0 || ob < b || (ob == b && oi < i));
            };
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ob = __shfl_xor(best, off);
                const int32_t oi = __shfl_xor(bidx, off);
                if (better(ob, oi, best, bidx)) {
                    best = ob;
                    bidx = oi;
                }
            }
            if (lane == 0) {
                s_best[wave] = best;
                s_idx[wave] = bidx;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                for (int w = 1; w < kWPS; ++w)
                    if (better(s_best[w], s_idx[w], best, bidx)) {
                        best = s_best[w];
                        bidx = s_idx[w];
                    }
                picks[(int64_t)t * nseq + s] = bidx;
                if (scores)
                    scores[(int64_t)t * nseq + s] =
                        bidx < 0 ? __builtin_nanf("") : (best == 0.0f ? 0.0f : best);
                if (bidx >= 0) s_mask[bidx >> 5] |= 1u << (bidx & 31);
                s_ref = bidx;
            }
            __syncthreads();
            r = s_ref;  // read before thread 0 rewrites it, behind the next step's first barrier
        }
        __syncthreads();
        for (int32_t i = threadIdx.x; i < W; i += 64 * kWPS) mrow[i] = s_mask[i];
        __syncthreads();  // s_mask is reloaded for the next sequence
    }
}

bool div_gram_run_supports(int64_t n) { return n >= 1 && (n + 31) / 32 <= kRunWords; }

hipError_t launch_div_gram_run(const float *G, int64_t n, int64_t ldg, const int32_t *seeds,
                               uint32_t *mask, int64_t nseq, int32_t steps, int32_t *picks,
                               float *scores, hipStream_t st, float *R, int64_t ldr) {
    if (nseq <= 0 || steps <= 0) return hipSuccess;
    const unsigned grid = (unsigned)(nseq < (1 << 20) ? nseq : (1 << 20));
    if (R) {
        timing_before(st, "k_div_gram_run<sum>");
        hipLaunchKernelGGL(k_div_gram_run<true>, dim3(grid), dim3(64 * kWPS), 0, st, G, n, ldg,
                           seeds, mask, nseq, steps, picks, scores, R, ldr);
    } else {
        timing_before(st, "k_div_gram_run");
        hipLaunchKernelGGL(k_div_gram_run<false>, dim3(grid), dim3(64 * kWPS), 0, st, G, n, ldg,
                           seeds, mask, nseq, steps, picks, scores, R, ldr);
    }
    const hipError_t err = hipGetLastError();
    timing_after(st);
    return err;
}

__global__ __launch_bounds__(256) void k_zero_rows(float *__restrict__ p, int64_t rows,
                                                  int64_t ld, int64_t n) {
    const int64_t total = rows * ld;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride)
        if (i % ld < n) p[i] = 0.0f;
}

hipError_t launch_zero_rows(float *p, int64_t rows, int64_t ld, int64_t n, hipStream_t st) {
    const int64_t total = rows * ld;
    if (total <= 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const unsigned grid = (unsigned)(want < 16384 ? want : 16384);
    hipLaunchKernelGGL(k_zero_rows, dim3(grid), dim3(256), 0, st, p, rows, ld, n);
    return hipGetLastError();
}

}  // namespace vs
