// prep.hip -- squared-norm precompute and key initialisation (gfx950).
//
// The squared-L2 ranking uses |q|^2 + |c|^2 - 2 q.c; |c|^2 is the same for
// every query, so it is computed once per call here instead of inside the
// scan (the diversity shader of "Issue 9-014: Tile Diversity Shader Inner
// Loop For L2 Cache Locality", "FP16 storage path", keeps norm accumulators
// inside its inner loop).  Every norm is summed in one fixed order that does
// not depend on alignment, table size or launch shape, so a candidate's
// norm -- and with it every ranking value -- is identical on every call.
#include "vs_internal.h"

namespace vs {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_fill_keys(uint64_t *keys, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) keys[i] = kNoKey;
}

// One wave per row.  Lane l owns the 4-element groups starting at 4l + 256i
// and accumulates them in index order; the 64 lane sums are then combined by
// a fixed butterfly.  The vector and scalar variants read the same elements
// in the same order.  Every row norm of the library comes from this routine.
template <bool VEC>
__device__ __forceinline__ float row_sqnorm(const float *__restrict__ x, int32_t d, int lane) {
    float acc = 0.0f;
    for (int32_t k = 4 * lane; k < d; k += 256) {
        if constexpr (VEC) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(x + k);
            acc = __builtin_fmaf(v.x, v.x, acc);
            acc = __builtin_fmaf(v.y, v.y, acc);
            acc = __builtin_fmaf(v.z, v.z, acc);
            acc = __builtin_fmaf(v.w, v.w, acc);
        } else {
            for (int e = 0; e < 4; ++e) {
                if (k + e < d) {
                    const float v = x[k + e];
                    acc = __builtin_fmaf(v, v, acc);
                }
            }
        }
    }
    for (int s = 32; s >= 1; s >>= 1) acc += __shfl_xor(acc, s);
    return acc;
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_row_sqnorms(const float *__restrict__ X, int64_t rows,
                                                    int32_t d, float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float acc = row_sqnorm<VEC>(X + row * (int64_t)d, d, lane);
    if (lane == 0) out[row] = acc;
}

// Everything the dense search needs before its scan, in one launch: the
// candidates' squared norms (workgroups [0, bc)), the queries' (next bq
// workgroups; skipped when qn is null) and the packed keys reset to "no
// candidate" (the last bk workgroups).  Same per-row routine, so the norms
// equal k_row_sqnorms' bit for bit.
template <bool VECC, bool VECQ>
__global__ __launch_bounds__(256) void k_dense_prep(const float *__restrict__ C, int64_t nc,
                                                   float *__restrict__ cn,
                                                   const float *__restrict__ Q, int64_t nq,
                                                   float *__restrict__ qn, int32_t d,
                                                   uint64_t *__restrict__ keys, int64_t bc,
                                                   int64_t bq) {
    const int lane = threadIdx.x & 63;
    const int64_t b = blockIdx.x;
    if (b < bc) {
        const int64_t row = b * 4 + (threadIdx.x >> 6);
        if (row >= nc) return;
        const float acc = row_sqnorm<VECC>(C + row * (int64_t)d, d, lane);
        if (lane == 0) cn[row] = acc;
    } else if (b < bc + bq) {
        const int64_t row = (b - bc) * 4 + (threadIdx.x >> 6);
        if (row >= nq) return;
        const float acc = row_sqnorm<VECQ>(Q + row * (int64_t)d, d, lane);
        if (lane == 0) qn[row] = acc;
    } else {
        const int64_t i = (b - bc - bq) * 256 + threadIdx.x;
        if (i < nq) keys[i] = kNoKey;
    }
}

// Feature-major X: column j's squared norm, feature k of column j at
// X[(j / 64) * cs + k * ld + j % 64] (cs = 64 for plain rows of stride ld;
// cs = d * 64, ld = 64 for the 64-column blocked layout).  A workgroup owns
// 64 columns (VEC: 256, four per lane); its 16 waves each sum one contiguous
// range of features in order, then wave 0 adds the 16 partial sums in wave
// order.  Vector width does not change any column's order of summation.
constexpr int kColWaves = 16;

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// four consecutive values widened to fp32 (fp16 exactly)
template <typename T>
__device__ __forceinline__ f32x4 load4_f32(const T *p) {
    if constexpr (sizeof(T) == 2) {
        const f16x4 h = *reinterpret_cast<const f16x4 *>(p);
        return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    } else {
        return *reinterpret_cast<const f32x4 *>(p);
    }
}

// T = float, or _Float16 for the fp16 blocked codebook (CB = 128, with
// 128-column blocks); plain fp32 layouts use CB = 64.
template <typename T, bool VEC, int CB = 64>
__global__ __launch_bounds__(64 * kColWaves) void k_col_sqnorms(const T *__restrict__ X,
                                                               int64_t cols, int64_t ld,
                                                               int64_t cs, int32_t d,
                                                               float *__restrict__ out) {
    constexpr int W = VEC ? 4 : 1;
    __shared__ f32x4 part[kColWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * W;
    const int32_t k0 = (int32_t)((int64_t)d * wave / kColWaves);
    const int32_t k1 = (int32_t)((int64_t)d * (wave + 1) / kColWaves);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c0 < cols) {
        const T *x = X + (c0 / CB) * cs + (c0 % CB);
        if constexpr (VEC) {
#pragma unroll 8
            for (int32_t k = k0; k < k1; ++k) {
                const f32x4 v = load4_f32(x + (int64_t)k * ld);
                acc.x = __builtin_fmaf(v.x, v.x, acc.x);
                acc.y = __builtin_fmaf(v.y, v.y, acc.y);
                acc.z = __builtin_fmaf(v.z, v.z, acc.z);
                acc.w = __builtin_fmaf(v.w, v.w, acc.w);
            }
        } else {
#pragma unroll 8
            for (int32_t k = k0; k < k1; ++k) {
                const float v = (float)x[(int64_t)k * ld];
                acc.x = __builtin_fmaf(v, v, acc.x);
            }
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && c0 < cols) {
        f32x4 s = part[0][lane];
        for (int w = 1; w < kColWaves; ++w) s += part[w][lane];
        if constexpr (VEC) {
            *reinterpret_cast<f32x4 *>(out + c0) = s;
        } else {
            out[c0] = s.x;
        }
    }
}

// Squared norm of each CSR row, summed in storage order.  Rows whose range
// is not inside [0, nnz] get NaN (they are not scanned either).
__global__ __launch_bounds__(256) void k_csr_row_sqnorms(const int32_t *__restrict__ indptr,
                                                        const float *__restrict__ values,
                                                        int64_t nq, int64_t nnz,
                                                        float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nq) return;
    const int64_t b = indptr[i], e = indptr[i + 1];
    if (b < 0 || e < b || e > nnz) {
        out[i] = __builtin_nanf("");
        return;
    }
    float acc = 0.0f;
    for (int64_t p = b; p < e; ++p) acc = __builtin_fmaf(values[p], values[p], acc);
    out[i] = acc;
}

static inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_fill_keys(uint64_t *keys, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_keys, dim3(blocks_for(n, 256)), dim3(256), 0, st, keys, n);
    return hipGetLastError();
}

hipError_t launch_row_sqnorms(const float *X, int64_t rows, int32_t d, float *out,
                              hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const bool vec = (d % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    if (vec)
        hipLaunchKernelGGL(k_row_sqnorms<true>, dim3(blocks_for(rows, 4)), dim3(256), 0, st, X,
                           rows, d, out);
    else
        hipLaunchKernelGGL(k_row_sqnorms<false>, dim3(blocks_for(rows, 4)), dim3(256), 0, st, X,
                           rows, d, out);
    return hipGetLastError();
}

hipError_t launch_dense_prep(const float *C, int64_t nc, float *cn, const float *Q, int64_t nq,
                             float *qn, int32_t d, uint64_t *keys, hipStream_t st) {
    if (nq <= 0) return hipSuccess;
    const int64_t bc = cn ? blocks_for(nc, 4) : 0;
    const int64_t bq = qn ? blocks_for(nq, 4) : 0;
    const int64_t bk = blocks_for(nq, 256);
    const dim3 grid((unsigned)(bc + bq + bk)), block(256);
    auto vec = [d](const float *X) {
        return (d % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    };
    const bool vc = cn && vec(C), vq = qn && vec(Q);
    if (vc && vq)
        hipLaunchKernelGGL((k_dense_prep<true, true>), grid, block, 0, st, C, nc, cn, Q, nq, qn, d,
                           keys, bc, bq);
    else if (vc)
        hipLaunchKernelGGL((k_dense_prep<true, false>), grid, block, 0, st, C, nc, cn, Q, nq, qn,
                           d, keys, bc, bq);
    else if (vq)
        hipLaunchKernelGGL((k_dense_prep<false, true>), grid, block, 0, st, C, nc, cn, Q, nq, qn,
                           d, keys, bc, bq);
    else
        hipLaunchKernelGGL((k_dense_prep<false, false>), grid, block, 0, st, C, nc, cn, Q, nq, qn,
                           d, keys, bc, bq);
    return hipGetLastError();
}

hipError_t launch_col_sqnorms(const float *X, int64_t cols, int64_t ld, int64_t cs, int32_t d,
                              float *out, hipStream_t st) {
    if (cols <= 0) return hipSuccess;
    const bool vec = (cols % 4 == 0) && (ld % 4 == 0) && (cs % 4 == 0) &&
                     ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
    if (vec)
        hipLaunchKernelGGL((k_col_sqnorms<float, true>), dim3(blocks_for(cols, 256)),
                           dim3(64 * kColWaves), 0, st, X, cols, ld, cs, d, out);
    else
        hipLaunchKernelGGL((k_col_sqnorms<float, false>), dim3(blocks_for(cols, 64)),
                           dim3(64 * kColWaves), 0, st, X, cols, ld, cs, d, out);
    return hipGetLastError();
}

// 64-column blocked copy of a feature-major codebook: CB[b][k][j] =
// CT[k * ldct + 64 b + j] for 64 b + j < nc, 0 for the padding columns of the
// last block.  One thread per 4 values (VEC) or per value; both sides move
// in 256-byte row segments.
template <bool VEC>
__global__ __launch_bounds__(256) void k_block_codebook(const float *__restrict__ CT, int64_t nc,
                                                       int64_t ldct, int32_t d, int64_t total,
                                                       float *__restrict__ CB) {
    constexpr int W = VEC ? 4 : 1;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * W;
    for (int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * W; e < total; e += stride) {
        const int64_t j = e & 63, k = (e >> 6) % d, b = (e >> 6) / d;
        const int64_t n = b * 64 + j;
        if constexpr (VEC) {
            f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (n < nc) v = *reinterpret_cast<const f32x4 *>(CT + k * ldct + n);  // nc % 4 == 0
            *reinterpret_cast<f32x4 *>(CB + e) = v;
        } else {
            CB[e] = n < nc ? CT[k * ldct + n] : 0.0f;
        }
    }
}

// Column norms of the fp16 128-column blocked codebook (feature k of column
// j at X[(j / 128) * d * 128 + k * 128 + j % 128]).
hipError_t launch_col_sqnorms_f16(const uint16_t *X, int64_t cols, int32_t d, float *out,
                                  hipStream_t st) {
    if (cols <= 0) return hipSuccess;
    const _Float16 *Xh = reinterpret_cast<const _Float16 *>(X);
    const int64_t cs = (int64_t)d * 128;
    const bool vec = (cols % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 7) == 0) &&
                     ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
    if (vec)
        hipLaunchKernelGGL((k_col_sqnorms<_Float16, true, 128>), dim3(blocks_for(cols, 256)),
                           dim3(64 * kColWaves), 0, st, Xh, cols, (int64_t)128, cs, d, out);
    else
        hipLaunchKernelGGL((k_col_sqnorms<_Float16, false, 128>), dim3(blocks_for(cols, 64)),
                           dim3(64 * kColWaves), 0, st, Xh, cols, (int64_t)128, cs, d, out);
    return hipGetLastError();
}

// 128-column blocked fp16 copy of a feature-major fp32 codebook: CB[b][k][j]
// = fp16(CT[k * ldct + 128 b + j]) (round to nearest even) for 128 b + j < nc,
// 0 past nc.  One thread per value.
// SRC64: the source is the 64-neuron blocked fp32 layout (feature k of
// neuron n at CT[(n / 64) * 64 d + k * 64 + n % 64]) instead of the plain
// feature-major one; the fp16 values are the same roundings either way.
template <bool SRC64>
__global__ __launch_bounds__(256) void k_block_codebook_f16(const float *__restrict__ CT, int64_t nc,
                                                           int64_t ldct, int32_t d, int64_t total,
                                                           _Float16 *__restrict__ CB) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t j = e & 127, k = (e >> 7) % d, b = (e >> 7) / d;
        const int64_t n = b * 128 + j;
        const int64_t src = SRC64 ? (n >> 6) * 64 * (int64_t)d + k * 64 + (n & 63) : k * ldct + n;
        CB[e] = n < nc ? (_Float16)CT[src] : (_Float16)0.0f;
    }
}

// Four neurons per thread: one 16-byte load of four consecutive neurons'
// values (they are contiguous in both source layouts, which the launcher
// checks for the plain one) and one 8-byte store of their halves.
template <bool SRC64>
__global__ __launch_bounds__(256) void k_block_codebook_f16_x4(const float *__restrict__ CT,
                                                              int64_t nc, int64_t ldct, int32_t d,
                                                              int64_t total4,
                                                              _Float16 *__restrict__ CB) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e4 < total4; e4 += stride) {
        const int64_t j = (e4 & 31) * 4, bk = e4 >> 5;
        const int64_t k = bk % d, b = bk / d;
        const int64_t n = b * 128 + j;
        f16x4 h = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
        if (n < nc) {  // nc % 4 == 0: all four neurons exist
            const int64_t src =
                SRC64 ? (n >> 6) * 64 * (int64_t)d + k * 64 + (n & 63) : k * ldct + n;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(CT + src);
            h = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        }
        *reinterpret_cast<f16x4 *>(CB + e4 * 4) = h;
    }
}

hipError_t launch_block_codebook_f16(const float *CT, int64_t nc, int64_t ldct, int32_t d,
                                     uint16_t *CB, hipStream_t st, bool src_blocked64) {
    const int64_t total = (nc + 127) / 128 * 128 * (int64_t)d;
    const bool vec = nc % 4 == 0 && (src_blocked64 || ldct % 4 == 0) &&
                     ((reinterpret_cast<uintptr_t>(CT) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(CB) & 7) == 0);
    if (vec) {
        int64_t blocks = (total / 4 + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        if (src_blocked64)
            hipLaunchKernelGGL(k_block_codebook_f16_x4<true>, dim3((unsigned)blocks), dim3(256), 0,
                               st, CT, nc, ldct, d, total / 4, reinterpret_cast<_Float16 *>(CB));
        else
            hipLaunchKernelGGL(k_block_codebook_f16_x4<false>, dim3((unsigned)blocks), dim3(256), 0,
                               st, CT, nc, ldct, d, total / 4, reinterpret_cast<_Float16 *>(CB));
        return hipGetLastError();
    }
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (src_blocked64)
        hipLaunchKernelGGL(k_block_codebook_f16<true>, dim3((unsigned)blocks), dim3(256), 0, st, CT,
                           nc, ldct, d, total, reinterpret_cast<_Float16 *>(CB));
    else
        hipLaunchKernelGGL(k_block_codebook_f16<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                           CT, nc, ldct, d, total, reinterpret_cast<_Float16 *>(CB));
    return hipGetLastError();
}

hipError_t launch_block_codebook(const float *CT, int64_t nc, int64_t ldct, int32_t d, float *CB,
                                 hipStream_t st) {
    const int64_t total = (nc + 63) / 64 * 64 * (int64_t)d;
    const bool vec = nc % 4 == 0 && ldct % 4 == 0 &&
                     ((reinterpret_cast<uintptr_t>(CT) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(CB) & 15) == 0);
    const int64_t per = vec ? 4 : 1;
    int64_t blocks = (total / per + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (vec)
        hipLaunchKernelGGL(k_block_codebook<true>, dim3((unsigned)blocks), dim3(256), 0, st, CT,
                           nc, ldct, d, total, CB);
    else
        hipLaunchKernelGGL(k_block_codebook<false>, dim3((unsigned)blocks), dim3(256), 0, st, CT,
                           nc, ldct, d, total, CB);
    return hipGetLastError();
}

hipError_t launch_csr_row_sqnorms(const int32_t *indptr, const float *values, int64_t nq,
                                  int64_t nnz, float *out, hipStream_t st) {
    if (nq <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_csr_row_sqnorms, dim3(blocks_for(nq, 256)), dim3(256), 0, st, indptr,
                       values, nq, nnz, out);
    return hipGetLastError();
}

}  // namespace vs
