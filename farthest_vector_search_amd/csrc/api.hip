// api.hip -- the C ABI of libvs (declared in include/vs.h).
//
// Host side only: argument checks (before anything is enqueued), workspace
// layout, the per-device architecture check and the kernel sequence of each
// entry point on the caller's stream.  The library allocates no device
// memory: every buffer is the caller's.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "vs.h"
#include "vs_internal.h"

#define VS_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip = 0;  // the HIP error of this thread's last failed call

struct DevInfo {
    bool probed = false, ok = false;
    int n_cu = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

int device_ready(int *n_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip = (int)e;
        return VS_ERR_HIP;
    }
    if (dev < 0 || dev >= 64) return VS_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DevInfo &di = g_dev[dev];
    if (!di.probed) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        if (e != hipSuccess) {
            g_last_hip = (int)e;
            return VS_ERR_HIP;
        }
        di.ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
        di.n_cu = p.multiProcessorCount;
        di.probed = true;
    }
    if (!di.ok) return VS_ERR_UNSUPPORTED;
    *n_cu = di.n_cu;
    return VS_OK;
}

inline size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool al4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
inline bool al256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

constexpr int64_t kMaxIndex = 2147483647;  // indices are int32
constexpr int32_t kMaxDim = 1 << 20;

// Workspace of the dense and CSR searches: keys[nq] u64 | qn[nq] f32 | cn[nc] f32.
struct Layout {
    size_t keys = 0, qn = 0, cn = 0, total = 0;
};
Layout search_layout(int64_t nq, int64_t nc, int32_t metric) {
    Layout L;
    L.keys = 0;
    L.total = up256((size_t)nq * 8);
    if (vs::metric_is_l2(metric)) {
        L.qn = L.total;
        L.total += up256((size_t)nq * 4);
        L.cn = L.total;
        L.total += up256((size_t)nc * 4);
    }
    return L;
}

// The dense search's workspace: search_layout, or for a problem the small
// search may take, at least its partial keys and query norms (from offset 0;
// the small search uses nothing else).
Layout dense_layout(int64_t nq, int64_t nc, int32_t d, int32_t metric) {
    Layout L = search_layout(nq, nc, metric);
    if (vs::small_shape(nq, nc, d)) {
        const size_t small = vs::small_workspace(nq, nc);
        L.total = L.total > small ? L.total : small;
    }
    return L;
}

// Dense kernel choice: the two-launch small search for problems far too
// small to fill the chip (nq <= 1,024, nc <= 2,048, d <= 256, d % 4 == 0,
// 16-byte aligned rows); otherwise 32 queries per wave in registers for
// d <= 256, 16 per wave for d <= 768 (d % 4 == 0, 16-byte aligned rows), the
// LDS-tiled kernel otherwise.  VS_DENSE_KERNEL=small|qreg|q16|tiled forces
// one where it applies (all give results within the same bound; small, qreg
// and tiled are bit-identical).
enum class DenseKernel { SMALL, QREG, Q16, TILED };
DenseKernel dense_kernel(int64_t nq, int64_t nc, int32_t d, const float *C, const float *Q) {
    const char *env = std::getenv("VS_DENSE_KERNEL");
    const bool forced = env && env[0] != '\0';
    const bool q32 = vs::qreg_supports(d), q16 = vs::q16_supports(d, C, Q);
    const bool small = vs::small_supports(nq, nc, d, Q, C);
    if (small && (!forced || std::strcmp(env, "small") == 0)) return DenseKernel::SMALL;
    if (forced && std::strcmp(env, "tiled") == 0) return DenseKernel::TILED;
    if (forced && std::strcmp(env, "q16") == 0 && q16) return DenseKernel::Q16;
    if (q32) return DenseKernel::QREG;
    return q16 ? DenseKernel::Q16 : DenseKernel::TILED;
}

// Diversity step: the 16-query kernel where it applies, the tiled kernel
// otherwise or when VS_DIV_KERNEL=tiled.
bool div_use_q16(int32_t d, const float *C) {
    const char *env = std::getenv("VS_DIV_KERNEL");
    if (env && std::strcmp(env, "tiled") == 0) return false;
    return vs::q16_supports(d, C, nullptr);
}

#define VS_TRY_HIP(expr)                   \
    do {                                   \
        const hipError_t e_ = (expr);      \
        if (e_ != hipSuccess) {            \
            g_last_hip = (int)e_;          \
            return VS_ERR_HIP;             \
        }                                  \
    } while (0)

// ---- timing hook -------------------------------------------------------
struct Timing {
    std::mutex mu;
    bool on = false;
    int max = 0, count = 0;
    std::vector<hipEvent_t> start, stop;
    const char *name = "";
} g_timing;

}  // namespace

namespace vs {

void timing_before(hipStream_t st, const char *name) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.on || g_timing.count >= g_timing.max) return;
    g_timing.name = name;
    (void)hipEventRecord(g_timing.start[g_timing.count], st);
}

void timing_after(hipStream_t st) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.on || g_timing.count >= g_timing.max) return;
    (void)hipEventRecord(g_timing.stop[g_timing.count], st);
    ++g_timing.count;
}

}  // namespace vs

VS_API int vs_timing_enable(int32_t max_launches) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.on = false;
    g_timing.count = 0;
    if (max_launches <= 0) return VS_OK;
    while ((int)g_timing.start.size() < max_launches) {
        hipEvent_t a, b;
        VS_TRY_HIP(hipEventCreate(&a));
        VS_TRY_HIP(hipEventCreate(&b));
        g_timing.start.push_back(a);
        g_timing.stop.push_back(b);
    }
    g_timing.max = max_launches;
    g_timing.on = true;
    return VS_OK;
}

VS_API int vs_timing_read(double *total_ms, int64_t *launches) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    double sum = 0.0;
    for (int i = 0; i < g_timing.count; ++i) {
        VS_TRY_HIP(hipEventSynchronize(g_timing.stop[i]));
        float ms = 0.0f;
        VS_TRY_HIP(hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i]));
        sum += ms;
    }
    if (total_ms) *total_ms = sum;
    if (launches) *launches = g_timing.count;
    g_timing.on = false;
    g_timing.count = 0;
    return VS_OK;
}

VS_API const char *vs_timing_kernel_name(void) { return g_timing.name; }

// ---- dense search --------------------------------------------------------

VS_API size_t vs_bmu_search_workspace(int64_t nq, int64_t nc, int32_t d, int32_t metric) {
    if (nq < 0 || nc < 0 || metric < 0 || metric > 3) return 0;
    return dense_layout(nq, nc, d, metric).total;
}

// The dense search's kernel sequence over a workspace already checked to hold
// dense_layout(nq, nc, d, metric).total bytes (256-byte aligned).
static int dense_search(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                        int32_t metric, int32_t *idx_out, float *score_out, char *ws,
                        hipStream_t st, int n_cu) {
    const DenseKernel kernel = dense_kernel(nq, nc, d, C, Q);
    if (kernel == DenseKernel::SMALL) {
        VS_TRY_HIP(vs::launch_dense_small(Q, C, nq, nc, d, metric, reinterpret_cast<uint64_t *>(ws),
                                          idx_out, score_out, st));
        return VS_OK;
    }
    const Layout L = search_layout(nq, nc, metric);
    uint64_t *keys = reinterpret_cast<uint64_t *>(ws + L.keys);
    float *qn = vs::metric_is_l2(metric) ? reinterpret_cast<float *>(ws + L.qn) : nullptr;
    float *cn = vs::metric_is_l2(metric) ? reinterpret_cast<float *>(ws + L.cn) : nullptr;

    // every buffer of the workspace is written before it is read, in one
    // prologue launch: keys reset by a kernel (no memset node), the norms
    VS_TRY_HIP(vs::launch_dense_prep(C, nc, cn, Q, nq, score_out ? qn : nullptr, d, keys, st));

    vs::DenseArgs a{};
    a.Q = Q;
    a.C = C;
    a.cn = cn;
    a.keys = keys;
    a.nq = nq;
    a.nc = nc;
    a.d = d;
    switch (kernel) {
    case DenseKernel::QREG: VS_TRY_HIP(vs::launch_dense_qreg(a, metric, st, n_cu)); break;
    case DenseKernel::Q16: VS_TRY_HIP(vs::launch_dense_q16(a, metric, vs::kQRows, st, n_cu)); break;
    default: VS_TRY_HIP(vs::launch_dense(a, metric, vs::kQRows, st, n_cu)); break;
    }
    VS_TRY_HIP(vs::launch_finalize(keys, qn, nq, metric, idx_out, score_out, st));
    return VS_OK;
}

// Checks shared by the dense search and its no-allocation variant.
static int dense_check(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                       int32_t metric, const int32_t *idx_out, const float *score_out) {
    if (metric < 0 || metric > 3) return VS_ERR_METRIC;
    if (nq < 0 || nq > kMaxIndex || nc < 1 || nc > kMaxIndex || d < 1 || d > kMaxDim)
        return VS_ERR_SHAPE;
    if (nq == 0) return VS_OK;
    if (!Q || !C || !idx_out) return VS_ERR_NULL;
    if (!al4(Q) || !al4(C) || !al4(idx_out) || !al4(score_out)) return VS_ERR_ALIGN;
    return VS_OK;
}

VS_API int vs_bmu_search(const float *Q, const float *C, int64_t nq, int64_t nc, int32_t d,
                         int32_t metric, int32_t *idx_out, float *score_out, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (const int s = dense_check(Q, C, nq, nc, d, metric, idx_out, score_out)) return s;
    if (nq == 0) return VS_OK;
    if (!workspace) return VS_ERR_NULL;
    if (!al256(workspace)) return VS_ERR_ALIGN;
    if (workspace_bytes < dense_layout(nq, nc, d, metric).total) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    return dense_search(Q, C, nq, nc, d, metric, idx_out, score_out,
                        static_cast<char *>(workspace), reinterpret_cast<hipStream_t>(stream),
                        n_cu);
}

// ---- dense search with no allocation ---------------------------------------
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): the workspace of vs_bmu_search lives in this
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes `scratch` itself to a kernel (its name on the host is
// a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and is
// kept per device.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;  // 8 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch[64];  // device address of `scratch` per device (null until taken)
}  // namespace

static int scratch_ptr(char **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip = (int)e;
        return VS_ERR_HIP;
    }
    if (dev < 0 || dev >= 64) return VS_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            g_last_hip = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return VS_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = static_cast<char *>(g_scratch[dev]);
    return VS_OK;
}

VS_API int vs_bmu_search_noalloc(const float *Q, const float *C, int64_t nq, int64_t nc,
                                 int32_t d, int32_t metric, int32_t *idx_out, float *score_out,
                                 void *stream) {
    if (const int s = dense_check(Q, C, nq, nc, d, metric, idx_out, score_out)) return s;
    if (nq == 0) return VS_OK;
    if (dense_layout(nq, nc, d, metric).total > kNoAllocScratchBytes) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    char *ws = nullptr;
    if (const int s = scratch_ptr(&ws)) return s;
    return dense_search(Q, C, nq, nc, d, metric, idx_out, score_out, ws,
                        reinterpret_cast<hipStream_t>(stream), n_cu);
}

// ---- unfused comparator: score block, then a per-row pass -------------------

VS_API int vs_bmu_search_unfused(const float *Q, const float *C, int64_t nq, int64_t nc,
                                 int32_t d, int32_t metric, int32_t *idx_out, float *score_out,
                                 float *S, int64_t ld_s, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    if (metric < 0 || metric > 3) return VS_ERR_METRIC;
    if (nq < 0 || nq > kMaxIndex || nc < 1 || nc > kMaxIndex || d < 1 || d > kMaxDim ||
        ld_s < nc || ld_s % 4 != 0)
        return VS_ERR_SHAPE;
    if (nq == 0) return VS_OK;
    if (!Q || !C || !idx_out || !S || !workspace) return VS_ERR_NULL;
    if (!al4(Q) || !al4(C) || !al4(idx_out) || !al4(score_out) || !al256(workspace) ||
        (reinterpret_cast<uintptr_t>(S) & 15) != 0)
        return VS_ERR_ALIGN;
    const bool q32 = vs::qreg_supports(d);
    if (!q32 && !vs::q16_supports(d, C, Q)) return VS_ERR_UNSUPPORTED;
    const Layout L = search_layout(nq, nc, metric);
    if (workspace_bytes < L.total) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    uint64_t *keys = reinterpret_cast<uint64_t *>(ws + L.keys);
    float *qn = vs::metric_is_l2(metric) ? reinterpret_cast<float *>(ws + L.qn) : nullptr;
    float *cn = vs::metric_is_l2(metric) ? reinterpret_cast<float *>(ws + L.cn) : nullptr;
    if (cn) VS_TRY_HIP(vs::launch_row_sqnorms(C, nc, d, cn, st));
    if (qn && score_out) VS_TRY_HIP(vs::launch_row_sqnorms(Q, nq, d, qn, st));

    vs::DenseArgs a{};
    a.Q = Q;
    a.C = C;
    a.nq = nq;
    a.nc = nc;
    a.d = d;
    a.S = S;
    a.ld_s = ld_s;
    if (q32) VS_TRY_HIP(vs::launch_dense_qreg_store(a, st, n_cu));
    else VS_TRY_HIP(vs::launch_dense_q16_store(a, st, n_cu));
    VS_TRY_HIP(vs::launch_row_argbest(S, nq, nc, ld_s, cn, keys, metric, st));
    VS_TRY_HIP(vs::launch_finalize(keys, qn, nq, metric, idx_out, score_out, st));
    return VS_OK;
}

// ---- sparse-query search ---------------------------------------------------

// Workspace of the CSR search: keys[nq] | qn[nq] | cn[nc] | partial keys
// [csr_groups(nc)][nq].
struct CsrLayout {
    size_t keys = 0, qn = 0, cn = 0, part = 0, total = 0;
};
CsrLayout csr_layout(int64_t nq, int64_t nc) {
    CsrLayout L;
    L.qn = up256((size_t)nq * 8);
    L.cn = L.qn + up256((size_t)nq * 4);
    L.part = L.cn + up256((size_t)nc * 4);
    L.total = L.part + up256((size_t)vs::csr_groups(nc) * (size_t)nq * 8);
    return L;
}

VS_API size_t vs_bmu_search_csr_workspace(int64_t nq, int64_t nc, int32_t d, int32_t metric) {
    (void)d;
    if (nq < 0 || nc < 0 || metric < 0 || metric > 3) return 0;
    return csr_layout(nq, nc).total;
}

// Shared by both codebook layouts: feature k of neuron 64 b + j at
// CT + b * cstride bytes + (k * ld + j) floats (the column norms read the
// same layout).
static int csr_search(const int32_t *indptr, const int32_t *indices, const float *values,
                      int64_t nq, int64_t nnz, const float *CT, int64_t nc, int64_t ld,
                      int64_t cstride, int32_t d, int32_t metric, int32_t *idx_out,
                      float *score_out, void *workspace, size_t workspace_bytes, void *stream,
                      bool f16 = false) {
    if (nq == 0) return VS_OK;
    if (!indptr || !CT || !idx_out || !workspace || (nnz > 0 && (!indices || !values)))
        return VS_ERR_NULL;
    if (!al4(indptr) || !al4(indices) || !al4(values) || !al4(CT) || !al4(idx_out) ||
        !al4(score_out) || !al256(workspace))
        return VS_ERR_ALIGN;
    const CsrLayout L = csr_layout(nq, nc);
    if (workspace_bytes < L.total) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    uint64_t *keys = reinterpret_cast<uint64_t *>(ws + L.keys);
    float *qn = reinterpret_cast<float *>(ws + L.qn);
    float *cn = reinterpret_cast<float *>(ws + L.cn);
    uint64_t *part = reinterpret_cast<uint64_t *>(ws + L.part);

    if (vs::metric_is_l2(metric)) {
        if (f16)
            VS_TRY_HIP(vs::launch_col_sqnorms_f16(reinterpret_cast<const uint16_t *>(CT), nc, d,
                                                  cn, st));
        else
            VS_TRY_HIP(vs::launch_col_sqnorms(CT, nc, ld, cstride / 4, d, cn, st));
    }
    if (vs::metric_is_l2(metric) && score_out)
        VS_TRY_HIP(vs::launch_csr_row_sqnorms(indptr, values, nq, nnz, qn, st));

    vs::CsrArgs a{};
    a.indptr = indptr;
    a.indices = indices;
    a.values = values;
    a.CT = CT;
    a.cn = cn;
    a.keys = keys;
    a.nq = nq;
    a.nnz = nnz;
    a.nc = nc;
    a.ldct = ld;
    a.cstride = cstride;
    a.d = d;
    if (f16) VS_TRY_HIP(vs::launch_csr_f16(a, metric, st, n_cu, part));
    else VS_TRY_HIP(vs::launch_csr(a, metric, st, n_cu, part));
    VS_TRY_HIP(vs::launch_finalize(keys, qn, nq, metric, idx_out, score_out, st));
    return VS_OK;
}

static bool csr_shape_ok(int64_t nq, int64_t nnz, int64_t nc, int32_t d) {
    return !(nq < 0 || nq > kMaxIndex || nnz < 0 || nnz > kMaxIndex || nc < 1 ||
             nc > kMaxIndex || d < 1 || d > kMaxIndex);
}

VS_API int vs_bmu_search_csr(const int32_t *indptr, const int32_t *indices, const float *values,
                             int64_t nq, int64_t nnz, const float *CT, int64_t nc, int64_t ldct,
                             int32_t d, int32_t metric, int32_t *idx_out, float *score_out,
                             void *workspace, size_t workspace_bytes, void *stream) {
    if (metric < 0 || metric > 3) return VS_ERR_METRIC;
    if (!csr_shape_ok(nq, nnz, nc, d) || ldct < nc) return VS_ERR_SHAPE;
    return csr_search(indptr, indices, values, nq, nnz, CT, nc, ldct, 256, d, metric, idx_out,
                      score_out, workspace, workspace_bytes, stream);
}

VS_API size_t vs_csr_blocked_bytes(int64_t nc, int32_t d) {
    if (nc < 1 || nc > kMaxIndex || d < 1 || d > kMaxIndex) return 0;
    return (size_t)((nc + 63) / 64) * 64u * (size_t)d * 4u;
}

VS_API int vs_csr_block_codebook(const float *CT, int64_t nc, int64_t ldct, int32_t d, float *CB,
                                 void *stream) {
    if (nc < 1 || nc > kMaxIndex || ldct < nc || d < 1 || d > kMaxIndex) return VS_ERR_SHAPE;
    if (!CT || !CB) return VS_ERR_NULL;
    if (!al4(CT) || !al4(CB)) return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    VS_TRY_HIP(vs::launch_block_codebook(CT, nc, ldct, d, CB, reinterpret_cast<hipStream_t>(stream)));
    return VS_OK;
}

VS_API size_t vs_csr_blocked_f16_bytes(int64_t nc, int32_t d) {
    if (nc < 1 || nc > kMaxIndex || d < 1 || d > kMaxIndex) return 0;
    return (size_t)((nc + 127) / 128) * 128u * (size_t)d * 2u;
}

VS_API int vs_csr_block_codebook_f16(const float *CT, int64_t nc, int64_t ldct, int32_t d,
                                     uint16_t *CB16, void *stream) {
    if (nc < 1 || nc > kMaxIndex || ldct < nc || d < 1 || d > kMaxIndex) return VS_ERR_SHAPE;
    if (!CT || !CB16) return VS_ERR_NULL;
    if (!al4(CT) || (reinterpret_cast<uintptr_t>(CB16) & 15) != 0) return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    VS_TRY_HIP(vs::launch_block_codebook_f16(CT, nc, ldct, d, CB16,
                                             reinterpret_cast<hipStream_t>(stream)));
    return VS_OK;
}

VS_API int vs_csr_blocked_to_f16(const float *CB, int64_t nc, int32_t d, uint16_t *CB16,
                                 void *stream) {
    if (nc < 1 || nc > kMaxIndex || d < 1 || d > kMaxIndex) return VS_ERR_SHAPE;
    if (!CB || !CB16) return VS_ERR_NULL;
    if (!al4(CB) || (reinterpret_cast<uintptr_t>(CB16) & 15) != 0) return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    VS_TRY_HIP(vs::launch_block_codebook_f16(CB, nc, 64, d, CB16,
                                             reinterpret_cast<hipStream_t>(stream), true));
    return VS_OK;
}

VS_API int vs_bmu_search_csr_blocked_f16(const int32_t *indptr, const int32_t *indices,
                                         const float *values, int64_t nq, int64_t nnz,
                                         const uint16_t *CB16, int64_t nc, int32_t d,
                                         int32_t metric, int32_t *idx_out, float *score_out,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    if (metric < 0 || metric > 3) return VS_ERR_METRIC;
    if (!csr_shape_ok(nq, nnz, nc, d)) return VS_ERR_SHAPE;
    if (CB16 && (reinterpret_cast<uintptr_t>(CB16) & 15) != 0) return VS_ERR_ALIGN;
    return csr_search(indptr, indices, values, nq, nnz, reinterpret_cast<const float *>(CB16), nc,
                      128, (int64_t)d * 256, d, metric, idx_out, score_out, workspace,
                      workspace_bytes, stream, true);
}

VS_API int vs_bmu_search_csr_blocked(const int32_t *indptr, const int32_t *indices,
                                     const float *values, int64_t nq, int64_t nnz,
                                     const float *CB, int64_t nc, int32_t d, int32_t metric,
                                     int32_t *idx_out, float *score_out, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (metric < 0 || metric > 3) return VS_ERR_METRIC;
    if (!csr_shape_ok(nq, nnz, nc, d)) return VS_ERR_SHAPE;
    return csr_search(indptr, indices, values, nq, nnz, CB, nc, 64, (int64_t)d * 256, d, metric,
                      idx_out, score_out, workspace, workspace_bytes, stream);
}

// ---- diversity step ------------------------------------------------------

VS_API size_t vs_diversity_step_workspace(int64_t n, int32_t d, int64_t nseq) {
    (void)n;
    (void)d;
    if (nseq < 0) return 0;
    return up256((size_t)nseq * 8);
}

// The kernels of one diversity step (references gathered as C[last_pick[s]],
// or the rows of Q when Q is not null) on arguments already checked: the key
// reset (fill_keys; a run skips it after its first step, whose finalize
// left every key reset), the masked scan, the finalize (reset_keys: leave
// the keys reset for the run's next step).
static int diversity_step_enqueue(const float *C, int64_t n, int32_t d, const int32_t *last_pick,
                                  const float *Q, uint32_t *mask_bits, int64_t nseq,
                                  int32_t *idx_out, float *score_out, void *workspace,
                                  hipStream_t st, int n_cu, bool fill_keys, bool reset_keys) {
    uint64_t *keys = static_cast<uint64_t *>(workspace);
    const int64_t W = (n + 31) / 32;
    if (fill_keys) VS_TRY_HIP(vs::launch_fill_keys(keys, nseq, st));
    vs::DenseArgs a{};
    a.Q = Q;
    a.C = C;
    a.pick = last_pick;
    a.mask = mask_bits;
    a.keys = keys;
    a.nq = nseq;
    a.nc = n;
    a.d = d;
    a.mask_words = W;
    const int mode = Q ? vs::kQRowsMasked : vs::kQGatherMasked;
    const bool q16 = div_use_q16(d, C) && (!Q || vs::q16_supports(d, C, Q));
    if (q16) VS_TRY_HIP(vs::launch_dense_q16(a, VS_COS_MIN, mode, st, n_cu));
    else VS_TRY_HIP(vs::launch_dense(a, VS_COS_MIN, mode, st, n_cu));
    VS_TRY_HIP(vs::launch_finalize_div(keys, nseq, mask_bits, W, idx_out, score_out, st,
                                       reset_keys));
    return VS_OK;
}

VS_API int vs_diversity_step(const float *C, int64_t n, int32_t d, const int32_t *last_pick,
                             uint32_t *mask_bits, int64_t nseq, int32_t *idx_out,
                             float *score_out, void *workspace, size_t workspace_bytes,
                             void *stream) {
    if (n < 1 || n > kMaxIndex || d < 1 || d > kMaxDim || nseq < 0 || nseq > kMaxIndex)
        return VS_ERR_SHAPE;
    if (nseq == 0) return VS_OK;
    if (!C || !last_pick || !mask_bits || !idx_out || !workspace) return VS_ERR_NULL;
    if (!al4(C) || !al4(last_pick) || !al4(mask_bits) || !al4(idx_out) || !al4(score_out) ||
        !al256(workspace))
        return VS_ERR_ALIGN;
    if (workspace_bytes < vs_diversity_step_workspace(n, d, nseq)) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;

    return diversity_step_enqueue(C, n, d, last_pick, nullptr, mask_bits, nseq, idx_out,
                                  score_out, workspace, reinterpret_cast<hipStream_t>(stream),
                                  n_cu, true, false);
}

// A whole run: `steps` steps chained on the stream, step t's references being
// step t-1's picks (the seeds for t = 0).
VS_API int vs_diversity_run(const float *C, int64_t n, int32_t d, const int32_t *seeds,
                            uint32_t *mask_bits, int64_t nseq, int32_t steps,
                            int32_t *picks_out, float *scores_out, void *workspace,
                            size_t workspace_bytes, void *stream) {
    if (n < 1 || n > kMaxIndex || d < 1 || d > kMaxDim || nseq < 0 || nseq > kMaxIndex ||
        steps < 0)
        return VS_ERR_SHAPE;
    if (nseq == 0 || steps == 0) return VS_OK;
    // every check of the steps below, before anything is enqueued
    if (!C || !seeds || !picks_out || !mask_bits || !workspace) return VS_ERR_NULL;
    if (!al4(C) || !al4(seeds) || !al4(mask_bits) || !al4(picks_out) || !al4(scores_out) ||
        !al256(workspace))
        return VS_ERR_ALIGN;
    if (workspace_bytes < vs_diversity_step_workspace(n, d, nseq)) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (int32_t t = 0; t < steps; ++t) {
        const int32_t *last = t == 0 ? seeds : picks_out + (int64_t)(t - 1) * nseq;
        float *sc = scores_out ? scores_out + (int64_t)t * nseq : nullptr;
        if (const int s = diversity_step_enqueue(C, n, d, last, nullptr, mask_bits, nseq,
                                                 picks_out + (int64_t)t * nseq, sc, workspace,
                                                 st, n_cu, t == 0, t + 1 < steps))
            return s;
    }
    return VS_OK;
}

// ---- diversity from a cached Gram matrix -------------------------------------

VS_API int vs_diversity_step_ref(const float *C, int64_t n, int32_t d, const float *Q,
                                 uint32_t *mask_bits, int64_t nseq, int32_t *idx_out,
                                 float *score_out, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    if (n < 1 || n > kMaxIndex || d < 1 || d > kMaxDim || nseq < 0 || nseq > kMaxIndex)
        return VS_ERR_SHAPE;
    if (nseq == 0) return VS_OK;
    if (!C || !Q || !mask_bits || !idx_out || !workspace) return VS_ERR_NULL;
    if (!al4(C) || !al4(Q) || !al4(mask_bits) || !al4(idx_out) || !al4(score_out) ||
        !al256(workspace))
        return VS_ERR_ALIGN;
    if (workspace_bytes < vs_diversity_step_workspace(n, d, nseq)) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;

    return diversity_step_enqueue(C, n, d, nullptr, Q, mask_bits, nseq, idx_out, score_out,
                                  workspace, reinterpret_cast<hipStream_t>(stream), n_cu, true,
                                  false);
}

VS_API int vs_diversity_accumulate(const float *C, int64_t n, int32_t d, const int32_t *pick,
                                   float *Q, int64_t nseq, void *stream) {
    if (n < 1 || n > kMaxIndex || d < 1 || d > kMaxDim || nseq < 0 || nseq > kMaxIndex)
        return VS_ERR_SHAPE;
    if (nseq == 0) return VS_OK;
    if (!C || !pick || !Q) return VS_ERR_NULL;
    if (!al4(C) || !al4(pick) || !al4(Q)) return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    VS_TRY_HIP(vs::launch_div_accumulate(C, n, d, pick, Q, nseq,
                                         reinterpret_cast<hipStream_t>(stream)));
    return VS_OK;
}

VS_API int vs_diversity_run_ref(const float *C, int64_t n, int32_t d, const int32_t *seeds,
                                float *Q, uint32_t *mask_bits, int64_t nseq, int32_t steps,
                                int32_t *picks_out, float *scores_out, void *workspace,
                                size_t workspace_bytes, void *stream) {
    if (n < 1 || n > kMaxIndex || d < 1 || d > kMaxDim || nseq < 0 || nseq > kMaxIndex ||
        steps < 0)
        return VS_ERR_SHAPE;
    if (nseq == 0 || steps == 0) return VS_OK;
    // every check of the steps below, before anything is enqueued
    if (!C || !seeds || !Q || !picks_out || !mask_bits || !workspace) return VS_ERR_NULL;
    if (!al4(C) || !al4(seeds) || !al4(Q) || !al4(mask_bits) || !al4(picks_out) ||
        !al4(scores_out) || !al256(workspace))
        return VS_ERR_ALIGN;
    if (workspace_bytes < vs_diversity_step_workspace(n, d, nseq)) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // Q[s] = the seed's row: cleared, then the seed added (0 + x is exact)
    VS_TRY_HIP(vs::launch_zero_rows(Q, nseq, d, d, st));
    VS_TRY_HIP(vs::launch_div_accumulate(C, n, d, seeds, Q, nseq, st));
    for (int32_t t = 0; t < steps; ++t) {
        int32_t *idx = picks_out + (int64_t)t * nseq;
        float *sc = scores_out ? scores_out + (int64_t)t * nseq : nullptr;
        if (const int s = diversity_step_enqueue(C, n, d, nullptr, Q, mask_bits, nseq, idx, sc,
                                                 workspace, st, n_cu, t == 0, t + 1 < steps))
            return s;
        VS_TRY_HIP(vs::launch_div_accumulate(C, n, d, idx, Q, nseq, st));
    }
    return VS_OK;
}

VS_API int vs_diversity_gram(const float *C, int64_t n, int32_t d, float *G, int64_t ldg,
                             void *stream) {
    if (n < 1 || n > kMaxIndex || d < 1 || ldg < n || ldg % 4 != 0) return VS_ERR_SHAPE;
    if (!C || !G) return VS_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(G) & 15) != 0) return VS_ERR_ALIGN;
    if (!vs::q16_supports(d, C, nullptr)) return VS_ERR_UNSUPPORTED;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    vs::DenseArgs a{};
    a.Q = C;
    a.C = C;
    a.nq = n;
    a.nc = n;
    a.d = d;
    a.S = G;
    a.ld_s = ldg;
    VS_TRY_HIP(vs::launch_dense_q16_store(a, reinterpret_cast<hipStream_t>(stream), n_cu,
                                          true));
    return VS_OK;
}

VS_API int vs_diversity_step_gram(const float *G, int64_t n, int64_t ldg,
                                  const int32_t *last_pick, uint32_t *mask_bits, int64_t nseq,
                                  int32_t *idx_out, float *score_out, void *stream) {
    if (n < 1 || n > kMaxIndex || ldg < n || ldg % 4 != 0 || nseq < 0 || nseq > kMaxIndex)
        return VS_ERR_SHAPE;
    if (nseq == 0) return VS_OK;
    if (!G || !last_pick || !mask_bits || !idx_out) return VS_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(G) & 15) != 0 || !al4(last_pick) || !al4(mask_bits) ||
        !al4(idx_out) || !al4(score_out))
        return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    VS_TRY_HIP(vs::launch_div_gram_step(G, n, ldg, last_pick, mask_bits, nseq, idx_out, score_out,
                                        reinterpret_cast<hipStream_t>(stream)));
    return VS_OK;
}

VS_API int vs_diversity_step_gram_sum(const float *G, int64_t n, int64_t ldg,
                                      const int32_t *last_pick, float *R, int64_t ldr,
                                      uint32_t *mask_bits, int64_t nseq, int32_t *idx_out,
                                      float *score_out, void *stream) {
    if (n < 1 || n > kMaxIndex || ldg < n || ldg % 4 != 0 || ldr < n || ldr % 4 != 0 ||
        nseq < 0 || nseq > kMaxIndex)
        return VS_ERR_SHAPE;
    if (nseq == 0) return VS_OK;
    if (!G || !last_pick || !R || !mask_bits || !idx_out) return VS_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(G) & 15) != 0 || (reinterpret_cast<uintptr_t>(R) & 15) != 0 ||
        !al4(last_pick) || !al4(mask_bits) || !al4(idx_out) || !al4(score_out))
        return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    VS_TRY_HIP(vs::launch_div_gram_step(G, n, ldg, last_pick, mask_bits, nseq, idx_out, score_out,
                                        reinterpret_cast<hipStream_t>(stream), R, ldr));
    return VS_OK;
}

VS_API int vs_diversity_run_gram(const float *G, int64_t n, int64_t ldg, const int32_t *seeds,
                                 float *R, int64_t ldr, uint32_t *mask_bits, int64_t nseq,
                                 int32_t steps, int32_t *picks_out, float *scores_out,
                                 void *stream) {
    if (n < 1 || n > kMaxIndex || ldg < n || nseq < 0 || nseq > kMaxIndex || steps < 0 ||
        (R && (ldr < n || ldr % 4 != 0)))
        return VS_ERR_SHAPE;
    if (nseq == 0 || steps == 0) return VS_OK;
    // every check of the steps below, before anything is enqueued
    if (ldg % 4 != 0) return VS_ERR_SHAPE;
    if (!G || !seeds || !picks_out || !mask_bits) return VS_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(G) & 15) != 0 || (reinterpret_cast<uintptr_t>(R) & 15) != 0 ||
        !al4(seeds) || !al4(mask_bits) || !al4(picks_out) || !al4(scores_out))
        return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    if (R) VS_TRY_HIP(vs::launch_zero_rows(R, nseq, ldr, n, reinterpret_cast<hipStream_t>(stream)));
    if (vs::div_gram_run_supports(n)) {
        // the whole run in one launch (same picks, scores, masks and R as the
        // per-step calls below, which serve wider masks)
        VS_TRY_HIP(vs::launch_div_gram_run(G, n, ldg, seeds, mask_bits, nseq, steps, picks_out,
                                           scores_out, reinterpret_cast<hipStream_t>(stream), R,
                                           ldr));
        return VS_OK;
    }
    for (int32_t t = 0; t < steps; ++t) {
        const int32_t *last = t == 0 ? seeds : picks_out + (int64_t)(t - 1) * nseq;
        int32_t *idx = picks_out + (int64_t)t * nseq;
        float *sc = scores_out ? scores_out + (int64_t)t * nseq : nullptr;
        const int s = R ? vs_diversity_step_gram_sum(G, n, ldg, last, R, ldr, mask_bits, nseq,
                                                     idx, sc, stream)
                        : vs_diversity_step_gram(G, n, ldg, last, mask_bits, nseq, idx, sc,
                                                 stream);
        if (s) return s;
    }
    return VS_OK;
}

// ---- norms, tile rule, status ---------------------------------------------

VS_API int vs_candidate_norms(const float *C, int64_t nc, int32_t d, int32_t feature_major,
                              float *norms_out, void *stream) {
    if (nc < 0 || nc > kMaxIndex || d < 1 || d > kMaxIndex) return VS_ERR_SHAPE;
    if (nc == 0) return VS_OK;
    if (!C || !norms_out) return VS_ERR_NULL;
    if (!al4(C) || !al4(norms_out)) return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (feature_major) VS_TRY_HIP(vs::launch_col_sqnorms(C, nc, nc, 64, d, norms_out, st));
    else VS_TRY_HIP(vs::launch_row_sqnorms(C, nc, d, norms_out, st));
    return VS_OK;
}

// ---- SOM batch update, quantisation error, epoch ----------------------------

struct SomLayout {
    size_t S = 0, T = 0, cnt = 0, den_t = 0, den = 0, g = 0, total = 0;
};

SomLayout som_layout(int64_t nc, int32_t d, int32_t gmax) {
    SomLayout L;
    const size_t elems = (size_t)((nc + 63) / 64) * 64u * (size_t)d;
    L.T = up256(elems * 4);
    L.cnt = L.T + up256(elems * 4);
    L.den_t = L.cnt + up256((size_t)nc * 4);
    L.den = L.den_t + up256((size_t)nc * 4);
    L.g = L.den + up256((size_t)nc * 4);
    L.total = L.g + up256((size_t)gmax * 4);
    return L;
}

// map, sigma and radius checks; *R_eff = radius clipped to the map
static int som_params(int32_t rows, int32_t cols, int32_t d, float sigma, int32_t radius,
                      int32_t *R_eff) {
    if (rows < 1 || cols < 1 || (int64_t)rows * cols > kMaxIndex || d < 1 || d > kMaxIndex)
        return VS_ERR_SHAPE;
    if (!(sigma > 0.0f) || !(sigma < 3.0e38f) || radius < 0) return VS_ERR_SHAPE;
    // every weight inside the window stays a normal fp32 number (>= e^-64)
    if (radius > 0 && (double)radius > 8.0 * (double)sigma) return VS_ERR_SHAPE;
    // one pass launch covers 64 neurons x 32 features per workgroup and stays
    // under 2^32 threads (each of the two buffers is then < 128 GiB)
    if (((int64_t)rows * cols + 63) / 64 * 64 * (int64_t)d > (int64_t(1) << 35)) return VS_ERR_SHAPE;
    const int32_t ext = rows > cols ? rows : cols;
    *R_eff = radius < ext - 1 ? radius : ext - 1;
    return VS_OK;
}

static int som_update(vs::SomArgs &a, void *workspace, size_t workspace_bytes, void *stream) {
    const int64_t nc = (int64_t)a.rows * a.cols;
    const SomLayout L = som_layout(nc, a.d, a.rows > a.cols ? a.rows : a.cols);
    if (workspace_bytes < L.total) return VS_ERR_WORKSPACE;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    char *ws = static_cast<char *>(workspace);
    a.S = reinterpret_cast<float *>(ws + L.S);
    a.T = reinterpret_cast<float *>(ws + L.T);
    a.cnt = reinterpret_cast<int32_t *>(ws + L.cnt);
    a.den_t = reinterpret_cast<float *>(ws + L.den_t);
    a.rden = reinterpret_cast<float *>(ws + L.den);
    a.g = reinterpret_cast<float *>(ws + L.g);
    VS_TRY_HIP(vs::launch_som_update(a, reinterpret_cast<hipStream_t>(stream), n_cu));
    return VS_OK;
}

VS_API size_t vs_som_update_workspace(int32_t map_rows, int32_t map_cols, int32_t d) {
    int32_t R = 0;
    if (som_params(map_rows, map_cols, d, 1.0f, 0, &R)) return 0;
    return som_layout((int64_t)map_rows * map_cols, d, map_rows > map_cols ? map_rows : map_cols)
        .total;
}

VS_API int vs_som_update(const float *X, int64_t n, int32_t d, const int32_t *bmu, float *C,
                         int32_t map_rows, int32_t map_cols, float sigma, int32_t radius,
                         void *workspace, size_t workspace_bytes, void *stream) {
    int32_t R = 0;
    if (const int s = som_params(map_rows, map_cols, d, sigma, radius, &R)) return s;
    if (n < 0 || n > kMaxIndex) return VS_ERR_SHAPE;
    if (n == 0) return VS_OK;
    if (!X || !bmu || !C || !workspace) return VS_ERR_NULL;
    if (!al4(X) || !al4(bmu) || !al4(C) || !al256(workspace)) return VS_ERR_ALIGN;
    vs::SomArgs a{};
    a.csr = false;
    a.X = X;
    a.n = n;
    a.d = d;
    a.bmu = bmu;
    a.C = C;
    a.rows = map_rows;
    a.cols = map_cols;
    a.R = R;
    a.sigma = sigma;
    return som_update(a, workspace, workspace_bytes, stream);
}

VS_API int vs_som_update_csr(const int32_t *indptr, const int32_t *indices, const float *values,
                             int64_t n, int64_t nnz, const int32_t *bmu, float *CB,
                             int32_t map_rows, int32_t map_cols, int32_t d, float sigma,
                             int32_t radius, void *workspace, size_t workspace_bytes,
                             void *stream) {
    int32_t R = 0;
    if (const int s = som_params(map_rows, map_cols, d, sigma, radius, &R)) return s;
    if (n < 0 || n > kMaxIndex || nnz < 0 || nnz > kMaxIndex) return VS_ERR_SHAPE;
    if (n == 0) return VS_OK;
    if (!indptr || !bmu || !CB || !workspace || (nnz > 0 && (!indices || !values)))
        return VS_ERR_NULL;
    if (!al4(indptr) || !al4(indices) || !al4(values) || !al4(bmu) || !al4(CB) ||
        !al256(workspace))
        return VS_ERR_ALIGN;
    vs::SomArgs a{};
    a.csr = true;
    a.indptr = indptr;
    a.indices = indices;
    a.values = values;
    a.nnz = nnz;
    a.n = n;
    a.d = d;
    a.bmu = bmu;
    a.C = CB;
    a.rows = map_rows;
    a.cols = map_cols;
    a.R = R;
    a.sigma = sigma;
    return som_update(a, workspace, workspace_bytes, stream);
}

VS_API int vs_som_qe(const float *score, int64_t n, double *qe_out, void *stream) {
    if (n < 0 || n > kMaxIndex) return VS_ERR_SHAPE;
    if (!qe_out || (n > 0 && !score)) return VS_ERR_NULL;
    if (!al4(score) || (reinterpret_cast<uintptr_t>(qe_out) & 7) != 0) return VS_ERR_ALIGN;
    int n_cu = 0;
    if (const int s = device_ready(&n_cu)) return s;
    VS_TRY_HIP(vs::launch_som_qe(score, n, qe_out, reinterpret_cast<hipStream_t>(stream)));
    return VS_OK;
}

VS_API size_t vs_som_epoch_workspace(int64_t n, int32_t map_rows, int32_t map_cols, int32_t d) {
    const size_t u = vs_som_update_workspace(map_rows, map_cols, d);
    if (!u || n < 0) return 0;
    return up256(dense_layout(n, (int64_t)map_rows * map_cols, d, vs::L2SQ_MIN).total) + u;
}

VS_API int vs_som_epoch(const float *X, int64_t n, int32_t d, float *C, int32_t map_rows,
                        int32_t map_cols, float sigma, int32_t radius, int32_t *bmu_out,
                        float *score_out, double *qe_out, void *workspace,
                        size_t workspace_bytes, void *stream) {
    int32_t R = 0;
    if (const int s = som_params(map_rows, map_cols, d, sigma, radius, &R)) return s;
    if (n < 0 || n > kMaxIndex || d > kMaxDim) return VS_ERR_SHAPE;
    if (!C || !workspace || (n > 0 && (!X || !bmu_out || !score_out))) return VS_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(qe_out) & 7) != 0) return VS_ERR_ALIGN;
    const size_t need = vs_som_epoch_workspace(n, map_rows, map_cols, d);
    if (workspace_bytes < need) return VS_ERR_WORKSPACE;
    const int64_t nc = (int64_t)map_rows * map_cols;
    const size_t ws1 = up256(dense_layout(n, nc, d, vs::L2SQ_MIN).total);
    char *ws = static_cast<char *>(workspace);
    if (const int s = vs_bmu_search(X, C, n, nc, d, vs::L2SQ_MIN, bmu_out, score_out, ws, ws1,
                                    stream))
        return s;
    if (qe_out)
        if (const int s = vs_som_qe(score_out, n, qe_out, stream)) return s;
    return vs_som_update(X, n, d, bmu_out, C, map_rows, map_cols, sigma, radius, ws + ws1,
                         workspace_bytes - ws1, stream);
}

VS_API size_t vs_som_epoch_csr_workspace(int64_t n, int32_t map_rows, int32_t map_cols,
                                         int32_t d) {
    const size_t u = vs_som_update_workspace(map_rows, map_cols, d);
    if (!u || n < 0) return 0;
    return up256(csr_layout(n, (int64_t)map_rows * map_cols).total) + u;
}

VS_API int vs_som_epoch_csr(const int32_t *indptr, const int32_t *indices, const float *values,
                            int64_t n, int64_t nnz, float *CB, int32_t map_rows,
                            int32_t map_cols, int32_t d, float sigma, int32_t radius,
                            int32_t *bmu_out, float *score_out, double *qe_out, void *workspace,
                            size_t workspace_bytes, void *stream) {
    int32_t R = 0;
    if (const int s = som_params(map_rows, map_cols, d, sigma, radius, &R)) return s;
    if (n < 0 || n > kMaxIndex || nnz < 0 || nnz > kMaxIndex) return VS_ERR_SHAPE;
    if (!CB || !workspace || (n > 0 && (!bmu_out || !score_out))) return VS_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(qe_out) & 7) != 0) return VS_ERR_ALIGN;
    const size_t need = vs_som_epoch_csr_workspace(n, map_rows, map_cols, d);
    if (workspace_bytes < need) return VS_ERR_WORKSPACE;
    const int64_t nc = (int64_t)map_rows * map_cols;
    const size_t ws1 = up256(csr_layout(n, nc).total);
    char *ws = static_cast<char *>(workspace);
    if (const int s = vs_bmu_search_csr_blocked(indptr, indices, values, n, nnz, CB, nc, d,
                                                vs::L2SQ_MIN, bmu_out, score_out, ws, ws1,
                                                stream))
        return s;
    if (qe_out)
        if (const int s = vs_som_qe(score_out, n, qe_out, stream)) return s;
    return vs_som_update_csr(indptr, indices, values, n, nnz, bmu_out, CB, map_rows, map_cols, d,
                             sigma, radius, ws + ws1, workspace_bytes - ws1, stream);
}

VS_API int vs_som_epoch_csr_f16(const int32_t *indptr, const int32_t *indices,
                                const float *values, int64_t n, int64_t nnz, float *CB,
                                uint16_t *CB16, int32_t map_rows, int32_t map_cols, int32_t d,
                                float sigma, int32_t radius, int32_t *bmu_out, float *score_out,
                                double *qe_out, void *workspace, size_t workspace_bytes,
                                void *stream) {
    int32_t R = 0;
    if (const int s = som_params(map_rows, map_cols, d, sigma, radius, &R)) return s;
    if (n < 0 || n > kMaxIndex || nnz < 0 || nnz > kMaxIndex) return VS_ERR_SHAPE;
    if (!CB || !CB16 || !workspace || (n > 0 && (!bmu_out || !score_out))) return VS_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(qe_out) & 7) != 0) return VS_ERR_ALIGN;
    const size_t need = vs_som_epoch_csr_workspace(n, map_rows, map_cols, d);
    if (workspace_bytes < need) return VS_ERR_WORKSPACE;
    const int64_t nc = (int64_t)map_rows * map_cols;
    const size_t ws1 = up256(csr_layout(n, nc).total);
    char *ws = static_cast<char *>(workspace);
    if (const int s = vs_csr_blocked_to_f16(CB, nc, d, CB16, stream)) return s;
    if (const int s = vs_bmu_search_csr_blocked_f16(indptr, indices, values, n, nnz, CB16, nc, d,
                                                    vs::L2SQ_MIN, bmu_out, score_out, ws, ws1,
                                                    stream))
        return s;
    if (qe_out)
        if (const int s = vs_som_qe(score_out, n, qe_out, stream)) return s;
    return vs_som_update_csr(indptr, indices, values, n, nnz, bmu_out, CB, map_rows, map_cols, d,
                             sigma, radius, ws + ws1, workspace_bytes - ws1, stream);
}

VS_API int64_t vs_tile_rows(int64_t cache_bytes, int32_t d, int32_t bytes_per_value) {
    if (cache_bytes <= 0 || d < 1 || bytes_per_value < 1) return 0;
    // floor(cache * 0.85 / (d * b)) in exact integer arithmetic: 0.85 = 17/20
    const __int128 num = (__int128)cache_bytes * 17;
    const __int128 den = (__int128)20 * d * bytes_per_value;
    const int64_t rows = (int64_t)(num / den);
    return rows > 0 ? rows : 1;
}

VS_API const char *vs_status_str(int status) {
    switch (status) {
    case VS_OK: return "ok";
    case VS_ERR_NULL: return "required pointer is NULL";
    case VS_ERR_SHAPE: return "invalid size";
    case VS_ERR_METRIC: return "unknown metric";
    case VS_ERR_WORKSPACE: return "workspace too small";
    case VS_ERR_ALIGN: return "misaligned pointer";
    case VS_ERR_INDEX: return "index out of range";
    case VS_ERR_UNSUPPORTED: return "no supported (gfx950) GPU";
    case VS_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

VS_API int vs_last_hip_error(void) { return g_last_hip; }

VS_API const char *vs_version(void) { return "libvs 0.1 gfx950"; }
