// bmu_csr.hip -- sparse (CSR) queries against a feature-major codebook,
// fused with the arg-reduction.
//
// Source: "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof ..."
// (summary), section 3 (codebook stored feature-major, weight columns read
// once and reused, argmin fused so no score block is stored) and section 4
// (levers: articles per tile, neuron-axis chunking, vectorised loads).
//
// For a query with non-zeros (k, v) the dot product with neuron n is
// sum v * CT[k][n]; with the codebook feature-major, the neurons of one
// feature are contiguous, so a wave that owns a chunk of consecutive neurons
// reads each needed codebook row segment with fully coalesced loads
// (16-byte loads when the layout allows: "vectorised loads").  The work
// items are (neuron chunk, query) pairs in chunk-major order, so the waves
// running at one time share one chunk of the codebook (neuron-axis
// chunking), and the XCD-aware renumbering keeps an XCD's waves on
// neighbouring queries of that chunk.
//
// Per item a wave accumulates the dot products of its neurons in CSR order
// (a fixed order), ranks them (|c|^2 - 2 q.c for squared L2, +-q.c for
// cosine), reduces over its lanes to one (value, index) pair with the lowest
// index on ties, and merges it into the query's packed key with atomicMin.
// Rows with an out-of-range indptr span or column index are skipped whole
// (nothing outside the arrays is read) and keep the "no candidate" key.
#include "vs_internal.h"

namespace vs {

template <int NPL>
struct VecT;
template <>
struct VecT<1> { typedef float T; };
template <>
struct VecT<2> { typedef float T __attribute__((ext_vector_type(2))); };
template <>
struct VecT<4> { typedef float T __attribute__((ext_vector_type(4))); };

template <int NPL>
__device__ __forceinline__ void load_n(const float *p, float (&out)[NPL]) {
    if constexpr (NPL == 1) {
        out[0] = *p;
    } else {
        const typename VecT<NPL>::T v = *reinterpret_cast<const typename VecT<NPL>::T *>(p);
#pragma unroll
        for (int j = 0; j < NPL; ++j) out[j] = v[j];
    }
}

template <int M, int NPL>
__global__ __launch_bounds__(256) void k_bmu_csr(const CsrArgs a) {
    constexpr int NCW = 64 * NPL;  // neurons per wave item
    const int lane = threadIdx.x & 63;
    int g = blockIdx.x;
    const int G = gridDim.x;
    if ((G & 7) == 0) g = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
    const int64_t W = (int64_t)G * 4;
    const int64_t w = (int64_t)g * 4 + (threadIdx.x >> 6);
    const int64_t nq = a.nq, nc = a.nc;
    const int32_t d = a.d;

    for (int64_t item = w; item < a.n_items; item += W) {
        const int64_t chunk = item / nq;
        const int64_t q = item - chunk * nq;
        const int64_t n0 = chunk * NCW + (int64_t)lane * NPL;
        const bool live = n0 < nc;  // NPL > 1 only when nc % NPL == 0
        int64_t b = a.indptr[q], e = a.indptr[q + 1];
        bool ok = b >= 0 && e >= b && e <= a.nnz;
        if (!ok) b = e = 0;

        float acc[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) acc[j] = 0.0f;
        const float *base = a.CT + (live ? n0 : 0);

        int64_t p = b;
        for (; p + 4 <= e; p += 4) {
            int32_t k[4];
            float v[4], c[4][NPL];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                k[u] = a.indices[p + u];
                v[u] = a.values[p + u];
                if ((uint32_t)k[u] >= (uint32_t)d) {
                    ok = false;
                    k[u] = 0;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (live) load_n<NPL>(base + (int64_t)k[u] * nc, c[u]);
                else
#pragma unroll
                    for (int j = 0; j < NPL; ++j) c[u][j] = 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < NPL; ++j) acc[j] = __builtin_fmaf(v[u], c[u][j], acc[j]);
        }
        for (; p < e; ++p) {
            int32_t k = a.indices[p];
            const float v = a.values[p];
            if ((uint32_t)k >= (uint32_t)d) {
                ok = false;
                k = 0;
            }
            float c[NPL];
            if (live) load_n<NPL>(base + (int64_t)k * nc, c);
            else
#pragma unroll
                for (int j = 0; j < NPL; ++j) c[j] = 0.0f;
#pragma unroll
            for (int j = 0; j < NPL; ++j) acc[j] = __builtin_fmaf(v, c[j], acc[j]);
        }
        if (!ok) continue;  // same decision on every lane of the wave

        float be = __builtin_inff();
        int32_t bi = -1;
        if (live) {
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const int64_t n = n0 + j;
                if (n < nc) {
                    const float cnn = metric_is_l2(M) ? a.cn[n] : 0.0f;
                    const float r = rank_value<M>(acc[j], cnn);
                    if (r < be) {
                        be = r;
                        bi = (int32_t)n;
                    }
                }
            }
        }
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) {
            const float oe = __shfl_xor(be, s);
            const int32_t oi = __shfl_xor(bi, s);
            if (oi >= 0 && (bi < 0 || oe < be || (oe == be && oi < bi))) {
                be = oe;
                bi = oi;
            }
        }
        if (lane == 0 && bi >= 0)
            atomicMin(reinterpret_cast<unsigned long long *>(a.keys + q),
                      (unsigned long long)pack_key(be, (uint32_t)bi));
    }
}

template <int NPL>
static void dispatch_metric(const CsrArgs &a, int metric, dim3 grid, hipStream_t st) {
    switch (metric) {
    case L2SQ_MIN: hipLaunchKernelGGL((k_bmu_csr<L2SQ_MIN, NPL>), grid, dim3(256), 0, st, a); break;
    case L2SQ_MAX: hipLaunchKernelGGL((k_bmu_csr<L2SQ_MAX, NPL>), grid, dim3(256), 0, st, a); break;
    case COS_MAX: hipLaunchKernelGGL((k_bmu_csr<COS_MAX, NPL>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((k_bmu_csr<COS_MIN, NPL>), grid, dim3(256), 0, st, a); break;
    }
}

hipError_t launch_csr(const CsrArgs &a0, int metric, hipStream_t st, int n_cu) {
    CsrArgs a = a0;
    const bool vec4 = (a.nc % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.CT) & 15) == 0);
    const int npl = vec4 ? 4 : 1;
    const int64_t ncw = 64 * npl;
    a.n_chunks = (a.nc + ncw - 1) / ncw;
    a.n_items = a.n_chunks * a.nq;
    const int64_t cap = (int64_t)(n_cu > 0 ? n_cu : 256) * 8;  // 8 workgroups (32 waves) per CU
    const int64_t wg_needed = (a.n_items + 3) / 4;
    int64_t grid = wg_needed < cap ? wg_needed : cap;
    if (grid >= 8) grid &= ~int64_t(7);
    if (grid < 1) grid = 1;
    timing_before(st, "k_bmu_csr");
    if (vec4) dispatch_metric<4>(a, metric, dim3((unsigned)grid), st);
    else dispatch_metric<1>(a, metric, dim3((unsigned)grid), st);
    const hipError_t err = hipGetLastError();
    timing_after(st);
    return err;
}

}  // namespace vs
