// som.hip -- batch SOM update and quantisation error around the BMU search.
//
// "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof", section 3
// (workload): each input's closest neuron is found first, then that neuron
// and its neighbours on the map are updated.  The update here is the batch
// map: neuron m at grid (m / cols, m % cols) of a planar rows x cols map
// becomes sum_i h(bmu_i, m) x_i / sum_i h(bmu_i, m) with the Gaussian
// h = exp(-(dy^2 + dx^2) / (2 sigma^2)) of the grid offset inside the square
// window max(|dy|, |dx|) <= R (0 outside); a neuron with zero denominator
// keeps its weights.
//
// The Gaussian of a square window factorises, h = g(dy) g(dx) with
// g(t) = exp(-t^2 / (2 sigma^2)), so the update runs as
//   1. S[b] = sum of the inputs whose BMU is b, N[b] = their count
//      (fp32 / int32 atomics; the float sums' last bits depend on the order
//      in which the atomics land);
//   2. a pass along the map's columns:  T(m) = sum_t g(t) S(m + t)
//      and the same over N;
//   3. a pass along the map's rows:     num(m) = sum_t g(t) T(m + t cols),
//      fused with the division into the codebook: num * (1 / den), the
//      reciprocal taken once per neuron by the denominator's second pass
//      (0 where den = 0: those neurons keep their weights).
// Both passes only sum over offsets that stay on the map (the planar edge).
// For window radii 1 .. 8 both passes run as one sweep over the map
// (k_som_smooth_blk, k_som_smooth_nm) that holds the pending outputs in a
// ring of registers; the two-pass kernels take R = 0 and R > 8.
//
// Element (neuron m, feature k) of the codebook and of the S / T buffers:
//   neuron-major (dense rows):  m * d + k
//   blocked feature-major (the sparse search's layout, 64-neuron blocks):
//                               (m / 64) * 64 d + k * 64 + m % 64
// Threads run along the contiguous axis (k, resp. m within a block), so every
// load and store of a pass is coalesced; the window's other taps are re-reads
// of lines the neighbouring waves just fetched (L1 / L2 hits).
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "vs_internal.h"

namespace vs {

namespace {

constexpr int kThreads = 256;

template <bool BLOCKED>
__device__ __forceinline__ int64_t at(int64_t m, int64_t k, int32_t d) {
    if constexpr (BLOCKED) return (m >> 6) * 64 * (int64_t)d + k * 64 + (m & 63);
    else return m * d + k;
}

__global__ __launch_bounds__(kThreads) void k_som_zero(float *p, int64_t n4, int32_t *cnt,
                                                       int64_t nc) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride)
        reinterpret_cast<f32x4 *>(p)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nc; i += stride) cnt[i] = 0;
}

// g[t] = exp(-t^2 / (2 sigma^2)), t = 0 .. count-1, evaluated in double and
// rounded once.
__global__ void k_som_gauss(float *g, int32_t count, double sigma) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < count) g[t] = (float)exp(-((double)t * (double)t) / (2.0 * sigma * sigma));
}

// Dense rows: one wave per input, lanes along the features.
__global__ __launch_bounds__(kThreads) void k_som_scatter_rows(const float *__restrict__ X,
                                                               int64_t n, int32_t d,
                                                               const int32_t *__restrict__ bmu,
                                                               int64_t nc, float *S,
                                                               int32_t *cnt) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t i = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); i < n;
         i += waves) {
        const int64_t b = bmu[i];
        if (b < 0 || b >= nc) continue;
        const float *x = X + i * d;
        float *s = S + b * d;
        for (int k = lane; k < d; k += 64) unsafeAtomicAdd(s + k, x[k]);
        if (lane == 0) atomicAdd(cnt + b, 1);
    }
}

// CSR rows: one wave per input, lanes along its stored entries; entries with
// a column outside [0, d) are skipped, and a row whose span is not inside
// [0, nnz] pulls nothing (nothing outside the caller's arrays is read).
__global__ __launch_bounds__(kThreads) void k_som_scatter_csr(
    const int32_t *__restrict__ indptr, const int32_t *__restrict__ indices,
    const float *__restrict__ values, int64_t nnz, int64_t n, int32_t d,
    const int32_t *__restrict__ bmu, int64_t nc, float *S, int32_t *cnt) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t i = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); i < n;
         i += waves) {
        const int64_t b = bmu[i];
        if (b < 0 || b >= nc) continue;
        const int64_t lo = indptr[i], hi = indptr[i + 1];
        if (lo < 0 || hi < lo || hi > nnz) continue;
        for (int64_t p = lo + lane; p < hi; p += 64) {
            const int32_t k = indices[p];
            if (k >= 0 && k < d) unsafeAtomicAdd(S + at<true>(b, k, d), values[p]);
        }
        if (lane == 0) atomicAdd(cnt + b, 1);
    }
}

// The neuron-major layout's two passes (dense rows).  Threads of a workgroup are
// split into groups of sg = min(256, d rounded up to a power of two) lanes;
// each group takes one neuron and runs along its features, so every tap is a
// coalesced row segment and the neuron's grid position and window are worked
// out once per neuron.  XCD x (workgroups blockIdx % 8 == x) owns map rows
// [x * rpx, (x + 1) * rpx) and its workgroups sweep them in an order that
// keeps the window's taps in that XCD's L2: row by row for the pass along
// map rows (taps m + t), in strips of kStrip columns, row by row within a
// strip, for the pass along map columns (taps m + t cols).  ALONG_X selects
// the pass; FINAL: out(m, k) = acc * rden[m] written where rden[m] > 0.
constexpr int kStrip = 32;

template <bool ALONG_X, bool FINAL>
__global__ __launch_bounds__(kThreads) void k_som_pass_nm(const float *__restrict__ in,
                                                          float *__restrict__ out, int32_t d,
                                                          int32_t sg, int32_t rows, int32_t cols,
                                                          int32_t rpx, int32_t R,
                                                          const float *__restrict__ g,
                                                          const float *__restrict__ rden) {
    const int per = kThreads / sg;  // neurons per workgroup step
    const int sub = (int)threadIdx.x / sg, kk = (int)threadIdx.x - sub * sg;
    const int xcd = (int)(blockIdx.x & 7);
    const int64_t wg = blockIdx.x >> 3, n_wg = gridDim.x >> 3;
    const int32_t y0 = xcd * rpx;
    const int32_t nstrip = (cols + kStrip - 1) / kStrip;
    // positions of this XCD's sweep (with holes past the map's edges)
    const int64_t npos = ALONG_X ? (int64_t)rpx * cols : (int64_t)nstrip * rpx * kStrip;
    for (int64_t p0 = wg * per; p0 < npos; p0 += n_wg * per) {
        const int64_t pos_i = p0 + sub;
        if (pos_i >= npos) continue;
        int32_t y, x;
        if constexpr (ALONG_X) {
            y = y0 + (int32_t)(pos_i / cols);
            x = (int32_t)(pos_i % cols);
        } else {
            const int64_t strip = pos_i / ((int64_t)rpx * kStrip);
            const int64_t rem = pos_i - strip * rpx * kStrip;
            y = y0 + (int32_t)(rem / kStrip);
            x = (int32_t)(strip * kStrip + rem % kStrip);
        }
        if (y >= rows || x >= cols) continue;
        const int64_t m = (int64_t)y * cols + x;
        float rd = 1.0f;
        if constexpr (FINAL) {
            rd = rden[m];
            if (!(rd > 0.0f)) continue;  // no input in the window: the neuron keeps its weights
        }
        const int32_t pos = ALONG_X ? x : y, ext = ALONG_X ? cols : rows;
        const int64_t step = ALONG_X ? 1 : cols;
        const int lo = pos < R ? -pos : -R;
        const int hi = ext - 1 - pos < R ? ext - 1 - pos : R;
        const float *src = in + m * d;
        const int64_t sd = step * d;  // floats between successive taps
        for (int k = kk; k < d; k += sg) {
            // taps kTB at a time, loads first: the window's loads are in
            // flight together instead of one round trip per tap
            constexpr int kTB = 8;
            float acc = 0.0f;
            int t = lo;
            // A batch's taps past the window read tap hi again with weight 0:
            // for finite data that adds exactly 0, and a non-finite tap hi is
            // summed with its own weight anyway.  (Guarding the add with a
            // branch or a select measured 30-50 % slower: the compiler then
            // waits for each load before the next.)
            for (; t <= hi; t += kTB) {
                float v[kTB];
#pragma unroll
                for (int i = 0; i < kTB; ++i) {
                    const int ti = t + i <= hi ? t + i : hi;
                    v[i] = src[(int64_t)ti * sd + k];
                }
#pragma unroll
                for (int i = 0; i < kTB; ++i) {
                    const int ti = t + i;
                    const float w = ti <= hi ? g[ti < 0 ? -ti : ti] : 0.0f;
                    acc = __builtin_fmaf(w, v[i], acc);
                }
            }
            out[m * d + k] = FINAL ? acc * rd : acc;
        }
    }
}

// The blocked layout's two passes.  A workgroup owns one 64-neuron block (lane =
// neuron) and 4 x kKV features (kKV per wave); each thread works out its
// neuron's grid position and window once, then for every tap reads kKV
// features of the tap neuron -- kKV loads, each a coalesced 256-byte row of a
// block.  Workgroups are numbered XCD by XCD: workgroup i runs on XCD i % 8
// and XCD x owns a contiguous eighth of the blocks, sweeping all of its blocks
// at one feature chunk before the next, so the neighbouring blocks a window
// reaches are (mostly) fetched into the same XCD's L2.
constexpr int kKV = 8;

template <bool ALONG_X, bool FINAL>
__global__ __launch_bounds__(kThreads) void k_som_pass_blk(const float *__restrict__ in,
                                                           float *__restrict__ out, int32_t nc,
                                                           int32_t d, int32_t rows, int32_t cols,
                                                           int32_t R, int32_t per_xcd,
                                                           const float *__restrict__ g,
                                                           const float *__restrict__ rden) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t lin = blockIdx.x, r = lin >> 3;
    const int32_t blk = (lin & 7) * per_xcd + r % per_xcd;
    const int32_t kbase = ((r / per_xcd) * 4 + wave) * kKV;
    const int64_t m64 = (int64_t)blk * 64 + lane;
    if (m64 >= nc || kbase >= d) return;
    const int32_t m = (int32_t)m64;
    float rd = 1.0f;
    if constexpr (FINAL) {
        rd = rden[m];
        if (!(rd > 0.0f)) return;  // no input in the window: the neuron keeps its weights
    }
    const int32_t y = m / cols, x = m - y * cols;
    const int32_t pos = ALONG_X ? x : y, ext = ALONG_X ? cols : rows;
    const int32_t step = ALONG_X ? 1 : cols;
    const int lo = pos < R ? -pos : -R;
    const int hi = ext - 1 - pos < R ? ext - 1 - pos : R;
    const int64_t D64 = 64 * (int64_t)d;
    const int nk = d - kbase < kKV ? d - kbase : kKV;
    float acc[kKV];
#pragma unroll
    for (int i = 0; i < kKV; ++i) acc[i] = 0.0f;
    for (int t = lo; t <= hi; ++t) {
        const int32_t n2 = m + t * step;
        const float *p = in + (int64_t)(n2 >> 6) * D64 + (n2 & 63) + (int64_t)kbase * 64;
        const float gt = g[t < 0 ? -t : t];
        if (nk == kKV) {
#pragma unroll
            for (int i = 0; i < kKV; ++i) acc[i] = __builtin_fmaf(gt, p[i * 64], acc[i]);
        } else {
            for (int i = 0; i < nk; ++i) acc[i] = __builtin_fmaf(gt, p[i * 64], acc[i]);
        }
    }
    float *o = out + (int64_t)blk * D64 + lane + (int64_t)kbase * 64;
#pragma unroll
    for (int i = 0; i < kKV; ++i)
        if (i < nk) o[i * 64] = FINAL ? acc[i] * rd : acc[i];
}

// Both passes in one sweep (blocked layout, window radius R <= 8 known at
// compile time).  A wave owns kSF consecutive features k0 .. k0+kSF-1 and a
// strip of 64 map columns x0 .. x0+63 and walks down the map one row at a
// time; the features' rows of one block are adjacent in memory, so a row's
// loads and stores cover kSF x 256 contiguous bytes instead of 256 bytes
// 4 MiB apart (d = 16,384), and they share the row's denominators.  Per
// feature:
//   - the row's 64 values plus R halo columns on each side (0 off the map)
//     go to a per-wave LDS row, from which each lane sums its column's
//     window along the row: X(y', x) = sum_t g(t) S(y', x + t);
//   - X(y', x) is added, weighted g(s), to the pending outputs of rows
//     y' - s, s = -R .. R, held in a ring of 2R+1 registers (the row loop is
//     unrolled by 2R+1 so every ring slot is a fixed register);
//   - once row y' is in, output row y' - R has all its terms: it is divided
//     by its denominator and stored (or left alone when that is 0).
// S is read once (plus the halo columns) and the codebook written once; no
// intermediate buffer.  The next row's loads are issued before the current
// row is summed.
// Calls f(integral_constant<int, U>) for U = B .. E-1 (compile-time unrolling).
template <int B, int E>
struct Unroll {
    template <class F>
    __device__ __forceinline__ static void run(F &f) {
        f(std::integral_constant<int, B>{});
        Unroll<B + 1, E>::run(f);
    }
};
template <int E>
struct Unroll<E, E> {
    template <class F>
    __device__ __forceinline__ static void run(F &) {}
};

#ifndef VS_SOM_BLK_F
#define VS_SOM_BLK_F 4
#endif
constexpr int kSF = VS_SOM_BLK_F;  // features per wave of the blocked sweep

template <int R, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void k_som_smooth_blk(
    const float *__restrict__ S, float *__restrict__ C, int32_t d, int32_t rows, int32_t cols,
    int32_t ntx, int64_t n_items, const float *__restrict__ g, const float *__restrict__ rden) {
    constexpr int P = 2 * R + 1;
    constexpr int W = 64 + 2 * R;
    constexpr int F = kSF;
    __shared__ float buf[kThreads / 64][F][W];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t item = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    if (item >= n_items) return;
    // strips fastest: the waves of a workgroup sweep neighbouring strips of
    // the same F features together, so each one's halo columns are lines
    // another has just fetched (ordering features fastest instead measured
    // 23 % slower)
    const int32_t kg = (int32_t)(item / ntx);
    const int32_t x0 = (int32_t)(item - (int64_t)kg * ntx) * 64;
    const int32_t k0 = kg * F;
    const int64_t D64 = 64 * (int64_t)d;
    const float *Sk = S + (int64_t)k0 * 64;
    float *Ck = C + (int64_t)k0 * 64;
    // feature k0 + f sits 64 f floats after feature k0 in every block;
    // features past d re-read feature d - 1 and are not stored
    int32_t fo[F];
#pragma unroll
    for (int f = 0; f < F; ++f) fo[f] = (k0 + f < d ? f : d - 1 - k0) * 64;
    const int nf = d - k0 < F ? d - k0 : F;  // features stored

    // each lane loads its own column and, lanes < 2R, one halo column:
    // left halo x0-R+lane (slot lane), right halo x0+64+lane-R (slot 64+lane)
    const int32_t xc = x0 + lane;
    const bool c_ok = xc < cols;
    const int32_t xh = lane < R ? x0 - R + lane : x0 + 64 + (lane - R);
    const bool h_ok = lane < 2 * R && xh >= 0 && xh < cols;
    const int hslot = lane < R ? lane : 64 + lane;
    // clamped (always in-bounds) columns, so every load is unconditional
    const int32_t xcl = c_ok ? xc : cols - 1;
    const int32_t xhl = h_ok ? xh : (xh < 0 ? 0 : cols - 1);
    // ALIGNED (cols % 64 == 0): a map row is cols / 64 whole blocks, so row y
    // of a column sits y * (cols / 64) * 64 d floats after row 0
    const int64_t rs = (int64_t)(cols >> 6) * D64;
    auto at_rc = [&](int32_t y, int32_t x) -> int64_t {
        if constexpr (ALIGNED) {
            return (int64_t)y * rs + ((int64_t)(x >> 6) * D64 + (x & 63));
        } else {
            const int32_t n = y * cols + x;
            return (int64_t)(n >> 6) * D64 + (n & 63);
        }
    };

    // ALIGNED: uniform row pointers, each advanced by one map row per step
    // (no per-row 64-bit products), and per-lane offsets inside a row; every
    // column of the strip is on the map (c_ok), and a halo lane's offset is
    // taken from its row's own block (the neighbouring blocks of one map row
    // are adjacent in this layout)
    const int64_t blk0 = (int64_t)(x0 >> 6) * D64;
    int64_t hoff = lane;  // lanes without a halo column read their own
    if (h_ok) hoff = lane < R ? (int64_t)(64 - R + lane) - D64 : D64 + (lane - R);
    const float *pn = Sk + blk0 + (rows > 1 ? rs : 0);  // row min(yy + 1, rows - 1)
    const float *pr = rden + x0;                        // row clamp(yy + 1 - R, 0, rows - 1)
    float *po = Ck + blk0;                              // output row yy - R

    float gw[R + 1];
#pragma unroll
    for (int i = 0; i <= R; ++i) gw[i] = g[i];
    float acc[F][P];
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
        for (int i = 0; i < P; ++i) acc[f][i] = 0.0f;

    float vc[F], vh[F];
#pragma unroll
    for (int f = 0; f < F; ++f) {
        if constexpr (ALIGNED) {
            vc[f] = Sk[fo[f] + blk0 + lane];
            vh[f] = Sk[fo[f] + blk0 + hoff];
        } else {
            vc[f] = Sk[fo[f] + at_rc(0, xcl)];
            vh[f] = Sk[fo[f] + at_rc(0, xhl)];
        }
    }
    // 1 / denominator of the output row finished after the current input row
    // (row yy - R; none for yy < R)
    float rnext = 0.0f;
    int32_t base = 0;
    // one input row; u = yy mod P is a compile-time constant
    auto step = [&](auto U) {
        constexpr int u = decltype(U)::value;
        const int32_t yy = base + u;
        if (yy < rows) {
            float cc[F], hh[F];
#pragma unroll
            for (int f = 0; f < F; ++f) {
                cc[f] = c_ok ? vc[f] : 0.0f;
                hh[f] = h_ok ? vh[f] : 0.0f;
            }
            const float rd = rnext;
            if constexpr (ALIGNED) {
#pragma unroll
                for (int f = 0; f < F; ++f) vc[f] = pn[fo[f] + lane];
#pragma unroll
                for (int f = 0; f < F; ++f) vh[f] = pn[fo[f] + hoff];
                rnext = pr[lane];
                if (yy + 2 < rows) pn += rs;
                if (yy + 2 - R >= 1 && yy + 2 - R <= rows - 1) pr += cols;
            } else {
                const int32_t yn = yy + 1 < rows ? yy + 1 : rows - 1;
                const int64_t an = at_rc(yn, xcl), hn = at_rc(yn, xhl);
#pragma unroll
                for (int f = 0; f < F; ++f) vc[f] = Sk[fo[f] + an];
#pragma unroll
                for (int f = 0; f < F; ++f) vh[f] = Sk[fo[f] + hn];
                int32_t yd1 = yy + 1 - R;
                yd1 = yd1 < 0 ? 0 : (yd1 >= rows ? rows - 1 : yd1);
                rnext = rden[(int64_t)yd1 * cols + xcl];
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int f = 0; f < F; ++f) {
                buf[wave][f][R + lane] = cc[f];
                if (lane < 2 * R) buf[wave][f][hslot] = hh[f];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            float X[F];
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const float *row = buf[wave][f];
                float x = gw[0] * row[R + lane];
#pragma unroll
                for (int t = 1; t <= R; ++t)
                    x = __builtin_fmaf(gw[t], row[R + lane - t] + row[R + lane + t], x);
                X[f] = x;
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int sft = -R; sft <= R; ++sft) {
                const int q = (u + sft + 2 * P) % P;  // constant once unrolled
#pragma unroll
                for (int f = 0; f < F; ++f)
                    acc[f][q] = __builtin_fmaf(gw[sft < 0 ? -sft : sft], X[f], acc[f][q]);
            }
            constexpr int qd = (u - R + 2 * P) % P;
            const int32_t yd = yy - R;
            if constexpr (ALIGNED) {
                if (yd >= 0) {
                    if (rd > 0.0f) {
#pragma unroll
                        for (int f = 0; f < F; ++f)
                            if (f < nf) po[fo[f] + lane] = acc[f][qd] * rd;
                    }
                    po += rs;
                }
            } else {
                if (yd >= 0 && c_ok && rd > 0.0f) {
                    const int64_t ao = at_rc(yd, xc);
#pragma unroll
                    for (int f = 0; f < F; ++f)
                        if (f < nf) Ck[fo[f] + ao] = acc[f][qd] * rd;
                }
            }
#pragma unroll
            for (int f = 0; f < F; ++f) acc[f][qd] = 0.0f;
        }
    };
    for (; base < rows; base += P) Unroll<0, P>::run(step);
    // the last R output rows have no further input rows
    for (int j = 0; j < R; ++j) {
        const int32_t y = rows - R + j;
        if (y < 0 || !c_ok) continue;
        const int q = y % P;
        const float rd = rden[(int64_t)y * cols + xc];
        if (!(rd > 0.0f)) continue;
        const int64_t ao = at_rc(y, xc);
#pragma unroll
        for (int f = 0; f < F; ++f) {
            float v = 0.0f;
#pragma unroll
            for (int qq = 0; qq < P; ++qq) v = qq == q ? acc[f][qq] : v;
            if (f < nf) Ck[fo[f] + ao] = v * rd;
        }
    }
}

// Both passes in one sweep for the neuron-major layout (dense rows, window
// radius R <= 8 known at compile time).  A wave owns 64 consecutive features
// (one per lane, so a neuron's segment is one 256-byte load), a strip of kSW
// map columns x0 .. x0+kSW-1 and a band of output rows [ya, yb), and walks
// the input rows ya-R .. yb+R-1 that lie on the map:
//   - the row's kSW + 2R neurons (0 off the map) are loaded into registers,
//     where every column's window along the row is summed:
//     X(y', x) = sum_t g(t) S(y', x + t);
//   - X(y', x) is added, weighted g(s), to the pending outputs of rows
//     y' - s in a ring of 2R+1 registers per column (the row loop is unrolled
//     by 2R+1, so every ring slot is a fixed register);
//   - once row y' is in, output row y' - R has all its terms; inside the band
//     it is multiplied by its reciprocal denominator and stored (or left
//     alone where the denominator is 0).
// The four waves of a workgroup take four adjacent strips, so most halo
// columns are lines a neighbouring wave has just fetched; the bands' halo
// rows are read twice.  No intermediate buffer: S is read about once and the
// codebook written once.
constexpr int kSW = 8;  // map columns per wave
#ifndef VS_SOM_SMOOTH_WAVES
#define VS_SOM_SMOOTH_WAVES 2048
#endif
constexpr int64_t kSmoothWaves = VS_SOM_SMOOTH_WAVES;  // target wave count of a launch
// Below this many waves the sweep cannot hide its row-by-row load latency
// (the 32 x 32 map, 16 waves: 36 us against 28 us for the two passes) and
// the two-pass kernels run instead.  VS_SOM_SMOOTH=sweep|passes forces one.
constexpr int64_t kSmoothMinWaves = 256;

template <int R>
__global__ __launch_bounds__(kThreads) void k_som_smooth_nm(
    const float *__restrict__ S, float *__restrict__ C, int32_t d, int32_t rows, int32_t cols,
    int32_t nkc, int32_t nsg, int32_t band, int64_t n_items, const float *__restrict__ g,
    const float *__restrict__ rden) {
    constexpr int P = 2 * R + 1;
    constexpr int NH = kSW + 2 * R;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // the grid is a multiple of 8: XCD x (blockIdx % 8) takes a contiguous
    // run of items, so the strips of neighbouring workgroups share an L2
    const int64_t G8 = gridDim.x >> 3;
    const int64_t item = (int64_t)(blockIdx.x & 7) * G8 + (blockIdx.x >> 3);
    if (item >= n_items) return;
    // item = (band, feature chunk, group of 4 strips), strips fastest
    const int32_t sg = (int32_t)(item % nsg);
    const int64_t rest = item / nsg;
    const int32_t kc = (int32_t)(rest % nkc);
    const int32_t bnd = (int32_t)(rest / nkc);
    const int32_t x0 = (sg * 4 + wave) * kSW;
    if (x0 >= cols) return;  // whole wave (no barriers in this kernel)
    const int32_t ya = bnd * band;
    const int32_t yb = ya + band < rows ? ya + band : rows;
    const int32_t ys = ya - R > 0 ? ya - R : 0;       // first input row
    const int32_t ye = yb + R < rows ? yb + R : rows;  // input rows end

    const int32_t k = kc * 64 + lane;
    const bool k_ok = k < d;
    const int32_t kl = k_ok ? k : d - 1;  // loads stay inside the row
    float gw[R + 1];
#pragma unroll
    for (int i = 0; i <= R; ++i) gw[i] = g[i];

    // raw loads of input row y (columns clamped onto the map; the columns
    // off the map are zeroed where the values are used)
    auto load_row = [&](int32_t y, float(&h)[NH]) {
        const float *row = S + (int64_t)y * cols * d + kl;
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const int32_t x = x0 - R + i;
            const int32_t xc = x < 0 ? 0 : (x >= cols ? cols - 1 : x);
            h[i] = row[(int64_t)xc * d];
        }
    };
    float hn[NH];
    load_row(ys, hn);
    float acc[kSW][P];
#pragma unroll
    for (int j = 0; j < kSW; ++j)
#pragma unroll
        for (int q = 0; q < P; ++q) acc[j][q] = 0.0f;

    int32_t base = ys;
    // one input row yy; its ring position u = (yy - ys) mod P is a
    // compile-time constant (output row y sits in slot (y - ys) mod P)
    auto step = [&](auto U) {
        constexpr int u = decltype(U)::value;
        const int32_t yy = base + u;
        if (yy < ye) {
            float h[NH];
#pragma unroll
            for (int i = 0; i < NH; ++i) {
                const int32_t x = x0 - R + i;
                h[i] = (x >= 0 && x < cols) ? hn[i] : 0.0f;
            }
            // output row of this step: its reciprocal denominators, then
            // the next input row's loads, all issued before the sums
            const int32_t yo = yy - R;
            float rq[kSW];
            {
                const int64_t ro = (int64_t)(yo > 0 ? yo : 0) * cols;
#pragma unroll
                for (int j = 0; j < kSW; ++j) {
                    const int32_t xo = x0 + j < cols ? x0 + j : cols - 1;
                    rq[j] = rden[ro + xo];
                }
            }
            load_row(yy + 1 < ye ? yy + 1 : yy, hn);
            asm volatile("" ::: "memory");
            float X[kSW];
#pragma unroll
            for (int j = 0; j < kSW; ++j) {
                float x = gw[0] * h[R + j];
#pragma unroll
                for (int t = 1; t <= R; ++t) x = __builtin_fmaf(gw[t], h[R + j - t] + h[R + j + t], x);
                X[j] = x;
            }
#pragma unroll
            for (int sft = -R; sft <= R; ++sft) {
                const int q = (u + sft + 2 * P) % P;  // constant once unrolled
#pragma unroll
                for (int j = 0; j < kSW; ++j)
                    acc[j][q] = __builtin_fmaf(gw[sft < 0 ? -sft : sft], X[j], acc[j][q]);
            }
            constexpr int qd = (u - R + 2 * P) % P;
            if (yo >= ya) {  // (yo < yb always: yy < ye <= yb + R)
                float *out = C + ((int64_t)yo * cols + x0) * d + k;
#pragma unroll
                for (int j = 0; j < kSW; ++j)
                    if (x0 + j < cols && k_ok && rq[j] > 0.0f) out[(int64_t)j * d] = acc[j][qd] * rq[j];
            }
#pragma unroll
            for (int j = 0; j < kSW; ++j) acc[j][qd] = 0.0f;
        }
    };
    for (; base < ye; base += P) Unroll<0, P>::run(step);
    // the map's last R rows have no further input rows: they are complete
    // now (only when the band reaches the map's end)
    if (ye == rows) {
        for (int32_t yo = rows - R > ya ? rows - R : ya; yo < yb; ++yo) {
            const int q = (yo - ys) % P;
            float *out = C + ((int64_t)yo * cols + x0) * d + k;
#pragma unroll
            for (int j = 0; j < kSW; ++j) {
                float v = 0.0f;
#pragma unroll
                for (int qq = 0; qq < P; ++qq) v = qq == q ? acc[j][qq] : v;
                if (x0 + j < cols && k_ok) {
                    const float rd = rden[(int64_t)yo * cols + x0 + j];
                    if (rd > 0.0f) out[(int64_t)j * d] = v * rd;
                }
            }
        }
    }
}

// The same two passes over the counts (one "feature", int32 input first);
// the second writes 1 / den (0 where den = 0).
template <bool ALONG_X, typename TIn>
__global__ __launch_bounds__(kThreads) void k_som_den_pass(const TIn *__restrict__ in,
                                                           float *__restrict__ out, int64_t nc,
                                                           int32_t rows, int32_t cols, int32_t R,
                                                           const float *__restrict__ g) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t m = (int64_t)blockIdx.x * kThreads + threadIdx.x; m < nc; m += stride) {
        const int64_t y = m / cols, x = m - y * cols;
        const int64_t pos = ALONG_X ? x : y, ext = ALONG_X ? cols : rows;
        const int64_t step = ALONG_X ? 1 : cols;
        const int lo = (int)(pos < R ? -pos : -R);
        const int hi = (int)(ext - 1 - pos < R ? ext - 1 - pos : R);
        float acc = 0.0f;
        for (int t = lo; t <= hi; ++t)
            acc = __builtin_fmaf(g[t < 0 ? -t : t], (float)in[m + t * step], acc);
        out[m] = ALONG_X ? acc : (acc > 0.0f ? 1.0f / acc : 0.0f);
    }
}

// Quantisation error: mean over the inputs of sqrt(max(score, 0)), summed in
// double by one workgroup in a fixed order (so the result is reproducible).
__global__ __launch_bounds__(1024) void k_som_qe(const float *__restrict__ score, int64_t n,
                                                 double *out) {
    __shared__ double part[1024];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) {
        const double v = (double)score[i];
        s += sqrt(v > 0.0 ? v : 0.0);
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 512; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = n > 0 ? part[0] / (double)n : __builtin_nan("");
}

unsigned grid_for(int64_t work, int n_cu) {
    const int64_t want = (work + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)n_cu * 32;
    return (unsigned)(want < 1 ? 1 : (want < cap ? want : cap));
}

}  // namespace

hipError_t launch_som_update(const SomArgs &a, hipStream_t st, int n_cu) {
    const bool blocked = a.csr;
    const int64_t nc = (int64_t)a.rows * a.cols;
    const int64_t elems = blocked ? ((nc + 63) / 64) * 64 * (int64_t)a.d : nc * (int64_t)a.d;
    const int32_t R = a.R;
    hipError_t err;

    // S is allocated in whole 256-byte units, so rounding up to float4 stays inside it
    const int64_t n4 = (elems + 3) / 4;
    hipLaunchKernelGGL(k_som_zero, dim3(grid_for(n4 > nc ? n4 : nc, n_cu)), dim3(kThreads), 0,
                       st, a.S, n4, a.cnt, nc);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_som_gauss, dim3((R + 1 + 255) / 256), dim3(256), 0, st, a.g, R + 1,
                       a.sigma);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.n > 0) {
        const dim3 gs(grid_for(a.n * 64, n_cu));  // one wave per input
        if (blocked)
            hipLaunchKernelGGL(k_som_scatter_csr, gs, dim3(kThreads), 0, st, a.indptr, a.indices,
                               a.values, a.nnz, a.n, a.d, a.bmu, nc, a.S, a.cnt);
        else
            hipLaunchKernelGGL(k_som_scatter_rows, gs, dim3(kThreads), 0, st, a.X, a.n, a.d,
                               a.bmu, nc, a.S, a.cnt);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const dim3 gd(grid_for(nc, n_cu));
    hipLaunchKernelGGL((k_som_den_pass<true, int32_t>), gd, dim3(kThreads), 0, st, a.cnt, a.den_t,
                       nc, a.rows, a.cols, R, a.g);
    hipLaunchKernelGGL((k_som_den_pass<false, float>), gd, dim3(kThreads), 0, st, a.den_t, a.rden,
                       nc, a.rows, a.cols, R, a.g);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // neuron-major sweep: bands of at least 8 rows, as many as bring the
    // waves to about kSmoothWaves (more waves keep more loads in flight; each
    // band re-reads 2R halo rows)
    const int32_t nm_kc = (a.d + 63) / 64;
    const int32_t nm_sg = ((a.cols + kSW - 1) / kSW + 3) / 4;
    const int64_t per_band = (int64_t)nm_kc * nm_sg * 4;
    int64_t nb = (kSmoothWaves + per_band - 1) / per_band;
    const int64_t nb_max = (a.rows + 7) / 8;
    nb = nb < 1 ? 1 : (nb > nb_max ? nb_max : nb);
    const int32_t band = (int32_t)((a.rows + nb - 1) / nb);
    nb = (a.rows + band - 1) / band;
    const int64_t nm_items = nb * nm_kc * nm_sg;
    bool sweep_nm = !blocked && R >= 1 && R <= 8;
    if (sweep_nm) {
        const char *env = std::getenv("VS_SOM_SMOOTH");
        if (env && std::strcmp(env, "passes") == 0) sweep_nm = false;
        else if (!(env && std::strcmp(env, "sweep") == 0))
            sweep_nm = nm_items * 4 >= kSmoothMinWaves;
    }
    if (blocked && R >= 1 && R <= 8) {
        const int32_t ntx = (a.cols + 63) / 64;
        const int64_t items = (int64_t)((a.d + kSF - 1) / kSF) * ntx;
        const dim3 gw((unsigned)((items + 3) / 4));
#define VS_SMOOTH(RR)                                                                          \
    case RR:                                                                                   \
        if (a.cols % 64 == 0)                                                                  \
            hipLaunchKernelGGL((k_som_smooth_blk<RR, true>), gw, dim3(kThreads), 0, st, a.S,    \
                               a.C, a.d, a.rows, a.cols, ntx, items, a.g, a.rden);              \
        else                                                                                   \
            hipLaunchKernelGGL((k_som_smooth_blk<RR, false>), gw, dim3(kThreads), 0, st, a.S,   \
                               a.C, a.d, a.rows, a.cols, ntx, items, a.g, a.rden);              \
        break;
        switch (R) {
            VS_SMOOTH(1) VS_SMOOTH(2) VS_SMOOTH(3) VS_SMOOTH(4)
            VS_SMOOTH(5) VS_SMOOTH(6) VS_SMOOTH(7) VS_SMOOTH(8)
        }
#undef VS_SMOOTH
    } else if (sweep_nm) {
        const dim3 gw((unsigned)((nm_items + 7) / 8 * 8));
#define VS_SMOOTH(RR)                                                                          \
    case RR:                                                                                   \
        hipLaunchKernelGGL((k_som_smooth_nm<RR>), gw, dim3(kThreads), 0, st, a.S, a.C, a.d,     \
                           a.rows, a.cols, nm_kc, nm_sg, band, nm_items, a.g, a.rden);          \
        break;
        switch (R) {
            VS_SMOOTH(1) VS_SMOOTH(2) VS_SMOOTH(3) VS_SMOOTH(4)
            VS_SMOOTH(5) VS_SMOOTH(6) VS_SMOOTH(7) VS_SMOOTH(8)
        }
#undef VS_SMOOTH
    } else if (blocked) {
        const int32_t nblk = (int32_t)((nc + 63) / 64);
        const int32_t per = (nblk + 7) / 8;
        const int64_t nkc = (a.d + 4 * kKV - 1) / (4 * kKV);
        const dim3 gb((unsigned)(8 * (int64_t)per * nkc));
        hipLaunchKernelGGL((k_som_pass_blk<true, false>), gb, dim3(kThreads), 0, st, a.S, a.T,
                           (int32_t)nc, a.d, a.rows, a.cols, R, per, a.g, nullptr);
        hipLaunchKernelGGL((k_som_pass_blk<false, true>), gb, dim3(kThreads), 0, st, a.T, a.C,
                           (int32_t)nc, a.d, a.rows, a.cols, R, per, a.g, a.rden);
    } else {
        int32_t sg = 1;
        while (sg < a.d && sg < kThreads) sg <<= 1;
        const int64_t per = kThreads / sg;
        const int32_t rpx = (a.rows + 7) / 8;
        const int64_t npos = (int64_t)rpx * ((a.cols + kStrip - 1) / kStrip) * kStrip;
        int64_t wpx = (npos + per - 1) / per;  // workgroups per XCD
        const int64_t cap = (int64_t)(n_cu > 0 ? n_cu : 256) * 4;
        wpx = wpx < 1 ? 1 : (wpx > cap ? cap : wpx);
        const dim3 gn((unsigned)(8 * wpx));
        hipLaunchKernelGGL((k_som_pass_nm<true, false>), gn, dim3(kThreads), 0, st, a.S, a.T,
                           a.d, sg, a.rows, a.cols, rpx, R, a.g, nullptr);
        hipLaunchKernelGGL((k_som_pass_nm<false, true>), gn, dim3(kThreads), 0, st, a.T, a.C,
                           a.d, sg, a.rows, a.cols, rpx, R, a.g, a.rden);
    }
    return hipGetLastError();
}

hipError_t launch_som_qe(const float *score, int64_t n, double *out, hipStream_t st) {
    hipLaunchKernelGGL(k_som_qe, dim3(1), dim3(1024), 0, st, score, n, out);
    return hipGetLastError();
}

}  // namespace vs
