// roofs.hip -- measurement kernels: the on-chip roof of the sparse scan, the
// fp32 MFMA issue rate the dense scans are measured against, and the
// row-gather rate of the diversity runs from the Gram matrix.
//
// Not part of the search ABI (built into libvs_roofs.so, used by bench.py's
// --roof mode).  The sparse scan reads codebook rows as 256-byte segments,
// one per 4-byte load instruction or four per 16-byte load instruction, out
// of a slice that lives in its XCD's L2; this kernel reads the same shapes
// from an L2-resident region so that the achieved L2 -> CU bandwidth of that
// access pattern can be quoted as the roof.
//
// Each XCD (workgroup group = blockIdx % 8, as the hardware deals workgroups
// to XCDs) reads its own region of `rows` rows, row stride `ld` floats;
// every wave walks the rows in a scattered order, 16 loads in flight,
// `passes` times.  One float per wave is written so the loads are not dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define VS_API extern "C" __attribute__((visibility("default")))

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int VW, int RPI>  // floats per lane per load; rows per load instruction
__global__ __launch_bounds__(256) void k_l2_roof(const float *__restrict__ buf, int64_t rows,
                                                int64_t ld, int32_t passes,
                                                float *__restrict__ out) {
    constexpr int LPR = 64 / RPI;  // lanes per row
    const int lane = threadIdx.x & 63;
    const int x = blockIdx.x & 7;
    const int64_t local = blockIdx.x >> 3;
    const int64_t wpx = (int64_t)(gridDim.x >> 3) * 4;  // waves per XCD
    const int64_t w = __builtin_amdgcn_readfirstlane((int)(local * 4 + (threadIdx.x >> 6)));
    // this lane's column; lane group lane / LPR reads its own row of each load
    const float *region = buf + (int64_t)x * rows * ld + (lane % LPR) * VW;
    const int64_t sub = lane / LPR;  // row offset of this lane group
    float acc = 0.0f;
    const int64_t steps = (int64_t)passes * rows / wpx;
    const int64_t mask = rows - 1;  // rows is a power of two
    int64_t r = (w * 9973) & mask;
    for (int64_t t = 0; t < steps; t += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int64_t row = (r + (int64_t)u * 4099 + sub * 1031) & mask;
            if constexpr (VW == 1) {
                v[u] = region[row * ld];
            } else {
                const f32x4 q = *reinterpret_cast<const f32x4 *>(region + row * ld);
                v[u] = q.x + q.y + q.z + q.w;
            }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += v[u];
        r = (r + 16 * 4099 + 1) & mask;
    }
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}


// fp32 MFMA issue rate: every wave runs `iters` x 8 MFMAs over two
// independent accumulator chains with operands in registers (no memory in the
// loop), the dependence pattern of the dense scans.  SHAPE 32: 32x32x2
// (4,096 FLOP each), SHAPE 16: 16x16x4 (2,048 FLOP each).  One float per
// thread is written so the chains are not dead.
template <int SHAPE>
__global__ __launch_bounds__(1024) void k_mfma_roof(int32_t iters, float a, float b,
                                                    float *__restrict__ out) {
    const float x = a + (float)threadIdx.x * 1e-7f, y = b;
    float s = 0.0f;
    if constexpr (SHAPE == 32) {
        f32x16 c0 = {}, c1 = {};
        for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, c1, 0, 0, 0);
            }
        }
        s = c0[0] + c1[15];
    } else {
        f32x4 c0 = {}, c1 = {};
        for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c1, 0, 0, 0);
            }
        }
        s = c0[0] + c1[3];
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Row gather: one workgroup of 4 waves per sequence (grid-stride over
// sequences) reads, for each step t, the whole row rows[t * nseq + s] of a
// table (n floats, row stride ld with ld % 4 == 0), 16 bytes per lane and two
// loads in flight, the way the whole-run Gram kernel reads its reference
// rows, with nothing else in the loop.  Row indices outside [0, nrows) are
// skipped.  Every thread writes one float so the loads are not dead.
__global__ __launch_bounds__(256) void k_gather_roof(const float *__restrict__ G, int64_t nrows,
                                                     int64_t n, int64_t ld,
                                                     const int32_t *__restrict__ rows,
                                                     int64_t nseq, int32_t steps,
                                                     float *__restrict__ out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t nn = (int32_t)n;
    float acc = 0.0f;
    for (int64_t s = blockIdx.x; s < nseq; s += gridDim.x) {
        for (int32_t t = 0; t < steps; ++t) {
            const int32_t r = rows[(int64_t)t * nseq + s];
            if (r < 0 || r >= nrows) continue;
            const float *row = G + (int64_t)r * ld;
            for (int32_t j0 = 256 * wave + 4 * lane; j0 < nn; j0 += 2048) {
                const int32_t j1 = j0 + 1024;
                // j < n <= ld, j % 4 == 0 and ld % 4 == 0: j + 3 < ld
                const f32x4 va = *reinterpret_cast<const f32x4 *>(row + j0);
                f32x4 vb = {0.0f, 0.0f, 0.0f, 0.0f};
                if (j1 < nn) vb = *reinterpret_cast<const f32x4 *>(row + j1);
                acc += (va.x + va.y) + (va.z + va.w) + (vb.x + vb.y) + (vb.z + vb.w);
            }
        }
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// Reads, per XCD region (8 regions, rows a power of two, row stride ld),
// `passes` times over: with rpi = 1 one row segment of 64 * vw floats per
// load instruction, with rpi = 4 (vw = 4) four row segments of 64 floats
// (256 bytes) per instruction, one per 16-lane group.  Returns the bytes the
// kernel read; the caller times the launch on `stream`.  out needs grid * 4
// floats, grid = 8 * wg_per_xcd.
VS_API int64_t vs_roof_l2_read(const float *buf, int64_t rows, int64_t ld, int32_t passes,
                               int32_t vw, int32_t rpi, int32_t wg_per_xcd, float *out,
                               void *stream) {
    if (!buf || !out || rows < 16 || (rows & (rows - 1)) != 0 || passes < 1 || wg_per_xcd < 1 ||
        (vw != 1 && vw != 4) || (rpi != 1 && rpi != 4) || (rpi == 4 && vw != 4) ||
        ld < 64 * vw / rpi)
        return -1;
    const dim3 grid((unsigned)(8 * wg_per_xcd)), block(256);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (vw == 1)
        hipLaunchKernelGGL((k_l2_roof<1, 1>), grid, block, 0, st, buf, rows, ld, passes, out);
    else if (rpi == 1)
        hipLaunchKernelGGL((k_l2_roof<4, 1>), grid, block, 0, st, buf, rows, ld, passes, out);
    else
        hipLaunchKernelGGL((k_l2_roof<4, 4>), grid, block, 0, st, buf, rows, ld, passes, out);
    if (hipGetLastError() != hipSuccess) return -1;
    const int64_t waves = (int64_t)8 * wg_per_xcd * 4;
    const int64_t steps = (int64_t)passes * rows / (waves / 8);
    const int64_t loads_per_wave = (steps + 15) / 16 * 16;
    return waves * loads_per_wave * 64 * 4 * vw;
}

// Launches k_mfma_roof with `cus` workgroups of 4 x waves_per_simd waves
// (one workgroup per CU) and returns its FLOPs; the caller times the launch
// on `stream`.  out needs cus * 256 * waves_per_simd floats.
VS_API int64_t vs_roof_mfma(int32_t shape, int32_t waves_per_simd, int32_t iters, int32_t cus,
                            float *out, void *stream) {
    if (!out || (shape != 16 && shape != 32) || waves_per_simd < 1 || waves_per_simd > 4 ||
        iters < 1 || cus < 1)
        return -1;
    const dim3 grid((unsigned)cus), block((unsigned)(256 * waves_per_simd));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (shape == 32)
        hipLaunchKernelGGL((k_mfma_roof<32>), grid, block, 0, st, iters, 1.0f, 1.0f, out);
    else
        hipLaunchKernelGGL((k_mfma_roof<16>), grid, block, 0, st, iters, 1.0f, 1.0f, out);
    if (hipGetLastError() != hipSuccess) return -1;
    const int64_t waves = (int64_t)cus * 4 * waves_per_simd;
    return waves * (int64_t)iters * 8 * (shape == 32 ? 4096 : 2048);
}

// Launches k_gather_roof over `grid` workgroups (out needs grid * 256
// floats); the caller times the launch on `stream` and counts the bytes
// (n * 4 per row index in [0, nrows)).  Returns 0, or -1 on bad arguments.
VS_API int32_t vs_roof_gather(const float *G, int64_t nrows, int64_t n, int64_t ld,
                              const int32_t *rows, int64_t nseq, int32_t steps, int32_t grid,
                              float *out, void *stream) {
    if (!G || !rows || !out || nrows < 1 || n < 1 || n > 2147483647 || ld < n || ld % 4 != 0 ||
        (reinterpret_cast<uintptr_t>(G) & 15) != 0 || nseq < 1 || steps < 1 || grid < 1)
        return -1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_gather_roof, dim3((unsigned)grid), dim3(256), 0, st, G, nrows, n, ld,
                       rows, nseq, steps, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The launch floor: a kernel with no work, one workgroup of one wave.
__global__ __launch_bounds__(64) void k_empty() {}

// Launches k_empty `count` times on `stream` (one launch per call of the
// caller's own loop when count = 1).  Returns 0, or -1 on a launch error.
VS_API int32_t vs_roof_empty(int32_t count, void *stream) {
    if (count < 1) return -1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < count; ++i) hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, st);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
