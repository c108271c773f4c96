// div_ref.hip -- the running reference of a centroid-reference diversity run.
//
// "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
// "FP16 storage (compounding optimization)", ranks candidates against the
// sequence's centroid.  Every row of the table is unit-norm, so the cosine
// to the centroid orders candidates exactly as the dot product with the sum
// of the sequence's rows does (the centroid is that sum over a positive
// count); the run keeps that sum per sequence, in fp32, and after each step
// adds the pick's row to it.  One wave per sequence, lanes along the
// features.
#include "vs_internal.h"

namespace vs {

__global__ __launch_bounds__(256) void k_div_accumulate(const float *__restrict__ C, int64_t n,
                                                        int32_t d,
                                                        const int32_t *__restrict__ pick,
                                                        float *__restrict__ Q, int64_t nseq) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * 4;
    for (int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); s < nseq; s += waves) {
        const int64_t p = pick[s];
        if (p < 0 || p >= n) continue;  // no pick: the reference stays
        const float *c = C + p * d;
        float *q = Q + s * d;
        for (int k = lane; k < d; k += 64) q[k] += c[k];
    }
}

hipError_t launch_div_accumulate(const float *C, int64_t n, int32_t d, const int32_t *pick,
                                 float *Q, int64_t nseq, hipStream_t st) {
    if (nseq <= 0) return hipSuccess;
    const int64_t want = (nseq + 3) / 4;
    const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(k_div_accumulate, dim3(grid), dim3(256), 0, st, C, n, d, pick, Q, nseq);
    return hipGetLastError();
}

}  // namespace vs
