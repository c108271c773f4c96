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

namespace vs {

template <int M>
__global__ __launch_bounds__(256) void k_finalize(const uint64_t *__restrict__ keys,
                                                 const float *__restrict__ qn, int64_t nq,
                                                 int32_t *__restrict__ idx_out,
                                                 float *__restrict__ score_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nq) return;
    const uint64_t k = keys[i];
    if (k == kNoKey) {
        idx_out[i] = -1;
        if (score_out) score_out[i] = __builtin_nanf("");
        return;
    }
    idx_out[i] = (int32_t)(uint32_t)(k & 0xffffffffu);
    if (score_out) {
        const float e = float_of_ord((uint32_t)(k >> 32));
        const float key = metric_is_max(M) ? -e : e;
        float s;
        if constexpr (metric_is_l2(M)) {
            s = qn[i] + key;
            s = s > 0.0f ? s : 0.0f;
        } else {
            s = key;
        }
        score_out[i] = s;
    }
}

__global__ __launch_bounds__(256) void k_finalize_div(const uint64_t *__restrict__ keys,
                                                     int64_t nseq, uint32_t *__restrict__ mask,
                                                     int64_t mask_words,
                                                     int32_t *__restrict__ idx_out,
                                                     float *__restrict__ score_out) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nseq) return;
    const uint64_t k = keys[s];
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

hipError_t launch_finalize_div(const uint64_t *keys, int64_t nseq, uint32_t *mask,
                               int64_t mask_words, int32_t *idx_out, float *score_out,
                               hipStream_t st) {
    if (nseq <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_finalize_div, dim3((unsigned)((nseq + 255) / 256)), dim3(256), 0, st,
                       keys, nseq, mask, mask_words, idx_out, score_out);
    return hipGetLastError();
}

}  // namespace vs
