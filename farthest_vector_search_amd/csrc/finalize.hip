// finalize.hip -- turn each query's merged packed key into (index, score).
//
// The scan leaves, per query, the minimum packed key over every candidate
// tile (value bits high, index low).  Here the winner's index is unpacked and
// its score rebuilt: squared L2 adds the query's own squared norm back
// (|q|^2 + |c|^2 - 2 q.c) and clamps at 0; cosine reports q.c.  For the
// diversity step the pick is also excluded from its sequence from now on, by
// setting its bit in that sequence's mask ("Issue 9-014: Tile Diversity
// Shader Inner Loop For L2 Cache Locality", "Current Behavior": the mask
// grows as picks accumulate).
#include "vs_internal.h"
#include "vs_score.h"

namespace vs {

template <int M>
__global__ __launch_bounds__(256) void k_finalize(const uint64_t *__restrict__ keys,
                                                 const float *__restrict__ qn, int64_t nq,
                                                 int32_t *__restrict__ idx_out,
                                                 float *__restrict__ score_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nq) return;
    const float qni = (metric_is_l2(M) && score_out) ? qn[i] : 0.0f;
    write_result<M>(keys[i], qni, idx_out + i, score_out ? score_out + i : nullptr);
}

// reset != 0: the key is set back to "no candidate" once read, so the next
// step of a run needs no separate reset launch.
__global__ __launch_bounds__(256) void k_finalize_div(uint64_t *__restrict__ keys,
                                                     int64_t nseq, uint32_t *__restrict__ mask,
                                                     int64_t mask_words,
                                                     int32_t *__restrict__ idx_out,
                                                     float *__restrict__ score_out, int reset) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nseq) return;
    const uint64_t k = keys[s];
    if (reset && k != kNoKey) keys[s] = kNoKey;
    if (k == kNoKey) {
        idx_out[s] = -1;
        if (score_out) score_out[s] = __builtin_nanf("");
        return;
    }
    const uint32_t j = (uint32_t)(k & 0xffffffffu);
    idx_out[s] = (int32_t)j;
    if (score_out) score_out[s] = float_of_ord((uint32_t)(k >> 32));  // COS_MIN: value = q.c
    // one thread per sequence owns that sequence's mask row
    mask[s * mask_words + (j >> 5)] |= 1u << (j & 31);
}

hipError_t launch_finalize(const uint64_t *keys, const float *qn, int64_t nq, int metric,
                           int32_t *idx_out, float *score_out, hipStream_t st) {
    if (nq <= 0) return hipSuccess;
    const dim3 grid((unsigned)((nq + 255) / 256)), block(256);
    switch (metric) {
    case L2SQ_MIN: hipLaunchKernelGGL(k_finalize<L2SQ_MIN>, grid, block, 0, st, keys, qn, nq, idx_out, score_out); break;
    case L2SQ_MAX: hipLaunchKernelGGL(k_finalize<L2SQ_MAX>, grid, block, 0, st, keys, qn, nq, idx_out, score_out); break;
    case COS_MAX: hipLaunchKernelGGL(k_finalize<COS_MAX>, grid, block, 0, st, keys, qn, nq, idx_out, score_out); break;
    default: hipLaunchKernelGGL(k_finalize<COS_MIN>, grid, block, 0, st, keys, qn, nq, idx_out, score_out); break;
    }
    return hipGetLastError();
}

hipError_t launch_finalize_div(uint64_t *keys, int64_t nseq, uint32_t *mask,
                               int64_t mask_words, int32_t *idx_out, float *score_out,
                               hipStream_t st, bool reset) {
    if (nseq <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_finalize_div, dim3((unsigned)((nseq + 255) / 256)), dim3(256), 0, st,
                       keys, nseq, mask, mask_words, idx_out, score_out, reset ? 1 : 0);
    return hipGetLastError();
}

// Second pass of the unfused comparator: one wave per query reads its row
// of the score block (16-byte loads, lane l: columns 256 i + 4 l .. + 3),
// ranks each dot product with the metric's rule (the fused epilogue's own
// rank_value), keeps the lowest value with the lowest index, and writes the
// query's packed key; k_finalize then produces (index, score) as for the
// fused scan.  The keys equal the fused scan's bit for bit.
template <int M>
__global__ __launch_bounds__(256) void k_row_argbest(const float *__restrict__ S, int64_t nq,
                                                    int64_t nc, int64_t ld_s,
                                                    const float *__restrict__ cn,
                                                    uint64_t *__restrict__ keys) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int64_t q = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (q >= nq) return;
    const float *row = S + q * ld_s;
    float best = __builtin_inff();
    int64_t bidx = -1;
    for (int64_t j0 = 4 * (int64_t)lane; j0 < nc; j0 += 256) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(row + j0);  // ld_s % 4 == 0
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (j0 + e < nc) {
                const float r = rank_value<M>(v[e], metric_is_l2(M) ? cn[j0 + e] : 0.0f);
                if (r < best) {
                    best = r;
                    bidx = j0 + e;
                }
            }
        }
    }
    uint64_t k = bidx >= 0 ? pack_key(best, (uint32_t)bidx) : kNoKey;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(k, off);
        k = o < k ? o : k;
    }
    if (lane == 0) keys[q] = k;
}

hipError_t launch_row_argbest(const float *S, int64_t nq, int64_t nc, int64_t ld_s,
                              const float *cn, uint64_t *keys, int metric, hipStream_t st) {
    if (nq <= 0) return hipSuccess;
    const dim3 grid((unsigned)((nq + 3) / 4)), block(256);
    switch (metric) {
    case L2SQ_MIN: hipLaunchKernelGGL(k_row_argbest<L2SQ_MIN>, grid, block, 0, st, S, nq, nc, ld_s, cn, keys); break;
    case L2SQ_MAX: hipLaunchKernelGGL(k_row_argbest<L2SQ_MAX>, grid, block, 0, st, S, nq, nc, ld_s, cn, keys); break;
    case COS_MAX: hipLaunchKernelGGL(k_row_argbest<COS_MAX>, grid, block, 0, st, S, nq, nc, ld_s, cn, keys); break;
    default: hipLaunchKernelGGL(k_row_argbest<COS_MIN>, grid, block, 0, st, S, nq, nc, ld_s, cn, keys); break;
    }
    return hipGetLastError();
}

}  // namespace vs
