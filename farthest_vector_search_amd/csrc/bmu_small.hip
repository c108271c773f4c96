// bmu_small.hip -- the dense search of a small problem in two launches.
//
// A search far too small to fill the chip (the 32 x 32 map: 256 queries x
// 1,024 neurons, d = 64) is bound by launch latency and by the chain of
// dependent memory reads inside each launch, not by the MFMA pipe.  The
// general path takes three launches (norms and key reset, scan, finalize);
// this one takes two and keeps no state between calls:
//  1. k_small_scan: one wave per (block of 32 queries, group of 32
//     candidates).  The wave loads all its operands straight from global
//     memory at once (no LDS staging, no barrier), runs the MFMAs, sums the
//     candidates' (and, in one wave per query block, the queries') squared
//     norms from the same registers, ranks, and writes the group's best
//     packed key of every query to its own slot part[query][group]: each
//     slot is written exactly once per call, so nothing needs resetting.
//  2. k_small_finalize: per query (one wave, one group per lane), the
//     minimum packed key over the groups (lowest index on ties, as in every
//     merge of the library) and the reported (index, score).
//
// Same numbers as the general dense path, bit for bit: the dot products run
// through the same v_mfma_f32_32x32x2f32 sequence as bmu_qreg.hip (chunk c of
// 8 features, lane half h feeding features 8c+4h..8c+4h+3, zeros past d, the
// same number of chunks); the norms are summed in the order of prep.hip's
// row routine (half_tree below); ranking, (value, lowest index) selection,
// packing and the final score use the shared routines.  Sources, by page
// title and section: "From 80x to 385x: A Best-Matching-Unit Search at the
// L2 Roof ..." (summary), section 3 (the argmin fused into the scan); "Issue
// 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality", "Intended
// Behavior" (partial winners of candidate tiles merged by an associative
// minimum).
#include "vs_internal.h"
#include "vs_score.h"

namespace vs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kSmallMaxD = 256;
static_assert((kSmallMaxCandidates + 31) / 32 <= 64, "the finalize gives each group one lane");

// The 16-byte quad at feature k of a row (rows 16-byte aligned, d % 4 == 0),
// or zeros past d or for a missing row (ok false).  The load itself is
// unconditional and stays inside the row (row is a valid row, k clamped to
// d - 4), so the compiler can issue a slab's loads together.
__device__ __forceinline__ f32x4 quad(const float *row, bool ok, int32_t k, int32_t d) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(row + (k < d ? k : d - 4));
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    return (ok && k < d) ? v : z;
}

// Squared norms with the bits of prep.hip's wave-wide row routine, from
// the quads a lane already holds as MFMA operands.  There lane g sums the
// quad at feature 4g with four FMAs in element order (d <= 256: one quad per
// lane, 0 past d), and the 64 lane sums are combined by a butterfly (partner
// g ^ s, s = 32, 16, ..., 1).  Here lane half h holds the quads g = 2j + h
// (j = the chunk) of its row: the butterfly levels s = 32 .. 2 pair quads of
// the same h, so they run in the lane on j (partner j ^ s/2), and the last
// level (s = 1) adds the other half's sum (lane ^ 32).  All sums are >= +0,
// so skipping levels whose partners are all zero (quads past d) changes no
// bit.  NJ: chunks held, rounded up to a power of two.
template <int NJ, int NCH>
__device__ __forceinline__ float half_tree(const f32x4 (&x)[NCH]) {
    float v[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        float acc = 0.0f;
        if (j < NCH) {
            acc = __builtin_fmaf(x[j].x, x[j].x, acc);
            acc = __builtin_fmaf(x[j].y, x[j].y, acc);
            acc = __builtin_fmaf(x[j].z, x[j].z, acc);
            acc = __builtin_fmaf(x[j].w, x[j].w, acc);
        }
        v[j] = acc;
    }
#pragma unroll
    for (int s = NJ / 2; s >= 1; s >>= 1) {
#pragma unroll
        for (int j = 0; j < s; ++j) v[j] = v[j] + v[j + s];
    }
    return v[0];
}

}  // namespace

// NSLAB = ceil(d / 64): the scan runs 8 NSLAB chunks of 8 features, as the
// general kernel does over its NSLAB slabs of 64 features.
template <int M, int NSLAB>
__global__ __launch_bounds__(256) void k_small_scan(const float *__restrict__ Q,
                                                    const float *__restrict__ C, int64_t nq,
                                                    int64_t nc, int32_t d, int32_t nqb,
                                                    int32_t ncg, uint64_t *__restrict__ part,
                                                    float *__restrict__ qn) {
    constexpr int NCH = 8 * NSLAB;
    constexpr int NJ = NCH <= 8 ? 8 : (NCH <= 16 ? 16 : 32);
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= (int64_t)nqb * ncg) return;  // whole waves; the kernel has no barrier
    const int32_t qb = (int32_t)(gw / ncg), cg = (int32_t)(gw - (int64_t)qb * ncg);
    const int64_t q = (int64_t)qb * 32 + l32;
    const int64_t base = (int64_t)cg * 32;
    // missing rows read row 0 (nq, nc >= 1) and are zeroed
    const bool q_ok = q < nq, c_ok = base + l32 < nc;
    const float *qrow = Q + (q_ok ? q : 0) * d;
    const float *crow = C + (c_ok ? base + l32 : 0) * d;

    // every operand quad is loaded before the first MFMA: one memory latency
    f32x4 qv[NCH], xv[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int32_t k = 8 * c + 4 * h;
        qv[c] = quad(qrow, q_ok, k, d);
        xv[c] = quad(crow, c_ok, k, d);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xv[c][e], qv[c][e], acc, 0, 0, 0);
    }
    // squared norms of candidate row l32 and (one wave per query block) of
    // query row l32, while the MFMAs run
    float cn_row = 0.0f;
    if constexpr (metric_is_l2(M)) {
        const float mine = half_tree<NJ, NCH>(xv);
        cn_row = mine + __shfl_xor(mine, 32);
        if (qn != nullptr && cg == 0) {
            const float qm = half_tree<NJ, NCH>(qv);
            const float qs = qm + __shfl_xor(qm, 32);
            if (h == 0 && q_ok) qn[q] = qs;
        }
    }
    // Accumulator register i: candidate row 8(i/4) + 4h + i%4 of the group,
    // query column l32.  Rows rise with i, and strict "<" keeps the lowest
    // row among equal values.
    const int64_t live = nc - base;  // rows r < live exist
    float best = __builtin_inff();
    int32_t bidx = -1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * h + (i & 3);
        const float cn = metric_is_l2(M) ? __shfl(cn_row, r) : 0.0f;
        const float v = rank_value<M>(acc[i], cn);
        if (r < live && v < best) {
            best = v;
            bidx = (int32_t)(base + r);
        }
    }
    // the two lane halves hold the same query's other rows
    const float oe = __shfl_xor(best, 32);
    const int32_t oi = __shfl_xor(bidx, 32);
    if (oi >= 0 && (bidx < 0 || oe < best || (oe == best && oi < bidx))) {
        best = oe;
        bidx = oi;
    }
    if (h == 0 && q_ok)
        part[q * ncg + cg] = bidx >= 0 ? pack_key(best, (uint32_t)bidx) : kNoKey;
}

// One wave per query: lane g reads group g's key (ncg <= 64), a butterfly
// takes their minimum, lane 0 writes the result.
template <int M>
__global__ __launch_bounds__(256) void k_small_finalize(const uint64_t *__restrict__ part,
                                                        int32_t ncg, const float *__restrict__ qn,
                                                        int64_t nq, int32_t *__restrict__ idx_out,
                                                        float *__restrict__ score_out) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= nq) return;  // whole waves
    uint64_t k = lane < ncg ? part[i * ncg + lane] : kNoKey;
    const float qni = (metric_is_l2(M) && score_out) ? qn[i] : 0.0f;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const uint64_t o = __shfl_xor(k, s);
        k = o < k ? o : k;
    }
    if (lane == 0) write_result<M>(k, qni, idx_out + i, score_out ? score_out + i : nullptr);
}

int64_t small_part_keys(int64_t nq, int64_t nc) {
    // nq * ceil(nc / 32) keys, rounded up to a multiple of 32 (256 bytes)
    return (nq * ((nc + 31) / 32) + 31) / 32 * 32;
}

size_t small_workspace(int64_t nq, int64_t nc) {
    return (size_t)small_part_keys(nq, nc) * 8u + ((size_t)nq * 4u + 255u) / 256u * 256u;
}

bool small_shape(int64_t nq, int64_t nc, int32_t d) {
    return nq >= 1 && nq <= kSmallMaxQueries && nc >= 1 && nc <= kSmallMaxCandidates && d >= 1 &&
           d <= kSmallMaxD;
}

bool small_supports(int64_t nq, int64_t nc, int32_t d, const float *Q, const float *C) {
    const bool al = (reinterpret_cast<uintptr_t>(Q) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(C) & 15) == 0;
    return small_shape(nq, nc, d) && d % 4 == 0 && al;
}

template <int M, int NSLAB>
static void launch_small_m(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                           uint64_t *part, int32_t *idx_out, float *score_out, hipStream_t st) {
    const int32_t nqb = (int32_t)((nq + 31) / 32), ncg = (int32_t)((nc + 31) / 32);
    const int64_t waves = (int64_t)nqb * ncg;
    // the query norms follow the partial keys in the workspace
    float *qn = (metric_is_l2(M) && score_out)
                    ? reinterpret_cast<float *>(part + small_part_keys(nq, nc))
                    : nullptr;
    timing_before(st, "k_small_scan");
    hipLaunchKernelGGL((k_small_scan<M, NSLAB>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       st, Q, C, nq, nc, d, nqb, ncg, part, qn);
    timing_after(st);
    hipLaunchKernelGGL((k_small_finalize<M>), dim3((unsigned)((nq + 3) / 4)), dim3(256), 0, st,
                       part, ncg, qn, nq, idx_out, score_out);
}

template <int M>
static void launch_small_slabs(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                               uint64_t *part, int32_t *idx_out, float *score_out,
                               hipStream_t st) {
    switch ((d + 63) / 64) {
    case 1: launch_small_m<M, 1>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    case 2: launch_small_m<M, 2>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    case 3: launch_small_m<M, 3>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    default: launch_small_m<M, 4>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    }
}

hipError_t launch_dense_small(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                              int metric, uint64_t *part, int32_t *idx_out, float *score_out,
                              hipStream_t st) {
    switch (metric) {
    case L2SQ_MIN: launch_small_slabs<L2SQ_MIN>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    case L2SQ_MAX: launch_small_slabs<L2SQ_MAX>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    case COS_MAX: launch_small_slabs<COS_MAX>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    default: launch_small_slabs<COS_MIN>(Q, C, nq, nc, d, part, idx_out, score_out, st); break;
    }
    return hipGetLastError();
}

}  // namespace vs
