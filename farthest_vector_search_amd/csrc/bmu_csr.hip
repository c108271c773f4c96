// bmu_csr.hip -- sparse (CSR) queries against a feature-major codebook,
// fused with the arg-reduction.
//
// Source: "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof ..."
// (summary), section 3 (codebook stored feature-major, weight columns
// reused, argmin fused so no score block is stored) and section 4 (levers:
// neuron-axis chunking to keep the codebook slice cache-resident, tile
// sizes, vectorised loads); section 6: the tuned kernel is bound by L2
// bandwidth.
//
// For a query with non-zeros (k, v) the dot product with neuron n is
// sum v * CT[k][n].  Feature-major storage makes the neurons of one feature
// contiguous, so a half-wave that owns 32 consecutive neurons (one per lane)
// reads the codebook row segment of each non-zero with one coalesced
// 128-byte load; the two halves of a wave serve two queries.  On this data a codebook value is needed by ~1.3 of the
// queries that share a tile, so reuse comes from the cache, not from LDS or
// registers: the kernel is bound by on-chip (L2) bandwidth at 4 bytes per
// multiply-add, and the design goal is that those bytes are L2 hits.
//
// Neuron-axis chunking, gfx950 style: the slice of the codebook for 32
// neurons is d x 128 bytes (2 MiB at d = 16,384), half of one XCD's L2; the
// CSR arrays, read once per round, are loaded non-temporally so that they do
// not evict it.  A codebook row stride that is a multiple of a large power of
// two maps every row's slice onto the same few L2 sets, so the row stride
// (ldct) is a parameter and callers can pad it.  Each launch
// is one "round": P <= 8 groups of workgroups, group x = blockIdx % P (the
// hardware deals consecutive workgroups to the eight XCDs in turn, so with
// P = 8 a group is one XCD) works on chunk round*P + x, its waves splitting
// all queries between them.  The kernel boundary between rounds keeps every
// XCD on a single chunk (a hard step, as the dispatch-per-tile variant of
// "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
// "Intended Behavior", proposes), instead of letting waves drift across
// chunks and thrash the L2.
//
// Merge: the wave that owns (group x, query q) is the only writer of
// partial[x][q] in its round, and rounds are ordered on the stream, so the
// running best per (group, query) is a plain read-min-write; a final pass
// takes the minimum over the P groups.  Packed (value, index) keys make both
// minima exact and order-independent (lowest index on ties).
// Rows with an out-of-range indptr span or column index are skipped whole
// (nothing outside the arrays is read) and keep the "no candidate" key.
#include <cstdlib>

#include "vs_internal.h"

namespace vs {

#ifndef VS_CSR_WG_PER_CU
#define VS_CSR_WG_PER_CU 7
#endif
constexpr int kCsrWgPerCu = VS_CSR_WG_PER_CU;  // x 4 waves resident per CU (VGPR-limited)
#ifndef VS_CSR_UNROLL
#define VS_CSR_UNROLL 8
#endif
constexpr int kCsrUnroll = VS_CSR_UNROLL;  // loads per group (two groups in flight)
// a batch holds 64 records and its walk is rounded up to whole groups, so a
// group size must divide 64 or the walk would read past the batch
static_assert(64 % kCsrUnroll == 0, "unroll must divide the 64-record batch");

template <typename T>
__device__ __forceinline__ T stream_load(const T *p) {
    return __builtin_nontemporal_load(p);
}

// HALVES = 1: a wave scans one query over a chunk of 64 neurons (one per
// lane); HALVES = 2: each half-wave scans its own query over a chunk of 32.
// A query's non-zeros are brought in 64 at a time with one coalesced,
// non-temporal load (lane j takes non-zero t+j); lane j turns its (k, v)
// into a record {address of codebook row k, v} in a wave-private LDS area.
// The walk over the batch then costs, per non-zero, one broadcast LDS read
// of the record, one 64-bit address add, one load of this lane's neuron and
// one FMA.
template <int M, int HALVES>
__global__ __launch_bounds__(256) void k_bmu_csr(const CsrArgs a, uint64_t *__restrict__ part,
                                                int64_t round, int32_t groups) {
    constexpr int NCW = 64 / HALVES;
    constexpr int U = kCsrUnroll;
    __shared__ uint64_t rec[4][HALVES][64];  // per wave, per query: row addresses
    __shared__ float wgt[4][HALVES][64];     // ... and weights
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = HALVES == 2 ? (lane >> 5) : 0;
    const int sub = lane % NCW;
    const int x = (int)(blockIdx.x % (unsigned)groups);
    const int64_t local = blockIdx.x / (unsigned)groups;
    const int64_t chunk = round * groups + x;
    if (chunk >= a.n_chunks) return;
    const int64_t waves_per_group = (int64_t)(gridDim.x / (unsigned)groups) * 4;
    const int64_t lw = __builtin_amdgcn_readfirstlane((int)(local * 4 + wave));
    const int64_t nq = a.nq, nc = a.nc, ld = a.ldct;
    const int32_t d = a.d;
    const int32_t n = (int32_t)(chunk * NCW + sub);
    const bool live = n < nc;
    const uint64_t off = (uint64_t)(live ? n : 0) * 4u;  // dead lanes read column 0
    const float cn = (metric_is_l2(M) && live) ? a.cn[n] : 0.0f;
    uint64_t *mine = part + (int64_t)x * nq;
    const uint64_t ct = reinterpret_cast<uint64_t>(a.CT);
    const int64_t qstep = HALVES * waves_per_group;

    // A "pair" is the HALVES queries a wave scans together.
    struct Pair {
        int64_t q0, b[HALVES], len[HALVES], L;
        bool ok[HALVES];
    };
    auto open_pair = [&](int64_t q0) {
        Pair P;
        P.q0 = q0;
        P.L = 0;
#pragma unroll
        for (int hh = 0; hh < HALVES; ++hh) {
            const int64_t q = q0 + hh;
            P.b[hh] = 0;
            P.len[hh] = 0;
            P.ok[hh] = q < nq;
            if (P.ok[hh]) {
                const int64_t bb = a.indptr[q], ee = a.indptr[q + 1];
                P.ok[hh] = bb >= 0 && ee >= bb && ee <= a.nnz;
                if (P.ok[hh]) {
                    P.b[hh] = bb;
                    P.len[hh] = ee - bb;
                }
            }
            P.L = P.len[hh] > P.L ? P.len[hh] : P.L;
        }
        return P;
    };
    // lane j fetches non-zero t+j of each query of the pair (0, 0 past its end)
    int32_t pk[HALVES];
    float pv[HALVES];
    auto prefetch = [&](const Pair &P, int64_t t) {
#pragma unroll
        for (int hh = 0; hh < HALVES; ++hh) {
            pk[hh] = 0;
            pv[hh] = 0.0f;
            if (t + lane < P.len[hh]) {
                pk[hh] = stream_load(a.indices + P.b[hh] + t + lane);
                pv[hh] = stream_load(a.values + P.b[hh] + t + lane);
            }
        }
    };
    auto issue = [&](int base, float (&c)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t addr = rec[wave][half][base + u] + off;
            c[u] = *reinterpret_cast<const __attribute__((address_space(1))) float *>(addr);
        }
    };
    // non-zero j of a batch (batches start at multiples of 64, groups at
    // multiples of U) goes to partial sum j % 4, the same split the
    // four-rows-per-load kernel uses, so every CSR path gives the same bits
    static_assert(U % 4 == 0, "groups must start at non-zero indices = 0 mod 4");
    auto consume = [&](int base, const float (&c)[U], float (&acc)[4]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc[u & 3] = __builtin_fmaf(wgt[wave][half][base + u], c[u], acc[u & 3]);
    };

    if (lw * HALVES >= nq) return;
    Pair cur = open_pair(HALVES * lw);
    prefetch(cur, 0);
    while (true) {
        float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        Pair nxt = cur;
        bool more = false;
        for (int64_t t = 0; t < cur.L; t += 64) {
            // this batch's (k, v) arrived with the previous prefetch
            int32_t kk[HALVES];
            float vv[HALVES];
#pragma unroll
            for (int hh = 0; hh < HALVES; ++hh) {
                kk[hh] = pk[hh];
                vv[hh] = pv[hh];
            }
            // start fetching the next batch (of this pair, or of the next pair)
            if (t + 64 < cur.L) {
                prefetch(cur, t + 64);
            } else if (cur.q0 + qstep < nq) {
                nxt = open_pair(cur.q0 + qstep);
                more = true;
                prefetch(nxt, 0);
            }
#pragma unroll
            for (int hh = 0; hh < HALVES; ++hh) {
                const bool bad = (uint32_t)kk[hh] >= (uint32_t)d;
                if (__any(bad)) cur.ok[hh] = false;
                if (bad) {
                    kk[hh] = 0;
                    vv[hh] = 0.0f;
                }
                rec[wave][hh][lane] = ct + (uint64_t)kk[hh] * (uint64_t)ld * 4u;
                wgt[wave][hh][lane] = vv[hh];
            }
            // walk the batch: U loads in flight while the previous U are used
            const int64_t rem = cur.L - t;
            const int cnt = (int)((rem < 64 ? rem : 64) + U - 1) / U * U;
            float c0[U], c1[U];
            issue(0, c0);
            for (int u0 = 0; u0 < cnt; u0 += 2 * U) {
                const bool two = u0 + U < cnt;
                if (two) issue(u0 + U, c1);
                consume(u0, c0, acc4);
                if (two) {
                    if (u0 + 2 * U < cnt) issue(u0 + 2 * U, c0);
                    consume(u0 + U, c1, acc4);
                }
            }
        }
        const float acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
        if (cur.L == 0 && cur.q0 + qstep < nq) {  // an all-empty pair prefetches nothing above
            nxt = open_pair(cur.q0 + qstep);
            more = true;
            prefetch(nxt, 0);
        }

        const bool row_ok = half ? cur.ok[HALVES - 1] : cur.ok[0];
        float be = (live && row_ok) ? rank_value<M>(acc, cn) : __builtin_inff();
        int32_t bi = (live && row_ok) ? n : -1;
#pragma unroll
        for (int s = NCW / 2; s >= 1; s >>= 1) {
            const float oe = __shfl_xor(be, s);
            const int32_t oi = __shfl_xor(bi, s);
            if (oi >= 0 && (bi < 0 || oe < be || (oe == be && oi < bi))) {
                be = oe;
                bi = oi;
            }
        }
        if (sub == 0 && row_ok && bi >= 0) {
            const int64_t q = cur.q0 + half;
            const uint64_t key = pack_key(be, (uint32_t)bi);
            if (key < mine[q]) mine[q] = key;
        }
        if (!more) break;
        cur = nxt;
    }
}

// Four-rows-per-load form (codebook rows 16-byte aligned, nc % 4 == 0).  A
// wave still owns 64 neurons, but one 16-byte-per-lane load now covers four
// non-zeros: lane group g = lane / 16 reads row k of non-zero 4i+g, lanes of
// a group four consecutive neurons each (16 x 16 B = one 256-byte row
// segment).  Wide loads reach about twice the L2 -> CU bandwidth of 4-byte
// loads on gfx950, and the codebook slice per XCD stays 4 MiB.  Each lane
// sums every fourth non-zero for its 4 neurons in order; the four partial
// sums are combined in one fixed order ((p0 + p1) + (p2 + p3)) at the end.
template <int M>
__global__ __launch_bounds__(256) void k_bmu_csr_q4(const CsrArgs a, uint64_t *__restrict__ part,
                                                   int64_t round, int32_t groups) {
    constexpr int U = 4;  // load instructions (16 non-zeros) per group, two groups in flight
    typedef float f4 __attribute__((ext_vector_type(4)));
    __shared__ uint64_t rec[4][64];  // per wave: row addresses of the batch
    __shared__ float wgt[4][64];     // ... and weights
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 4, col = lane & 15;
    const int x = (int)(blockIdx.x % (unsigned)groups);
    const int64_t local = blockIdx.x / (unsigned)groups;
    const int64_t chunk = round * groups + x;
    if (chunk >= a.n_chunks) return;
    const int64_t waves_per_group = (int64_t)(gridDim.x / (unsigned)groups) * 4;
    const int64_t lw = __builtin_amdgcn_readfirstlane((int)(local * 4 + wave));
    const int64_t nq = a.nq, nc = a.nc, ld = a.ldct;
    const int32_t d = a.d;
    const int32_t n0 = (int32_t)(chunk * 64 + 4 * col);  // this lane's 4 neurons
    const bool live = n0 < nc;                            // nc % 4 == 0: all 4 or none
    const uint64_t off = (uint64_t)(live ? n0 : 0) * 4u;
    f4 cn4 = {0.0f, 0.0f, 0.0f, 0.0f};
    if (metric_is_l2(M) && live) cn4 = *reinterpret_cast<const f4 *>(a.cn + n0);
    uint64_t *mine = part + (int64_t)x * nq;
    const uint64_t ct = reinterpret_cast<uint64_t>(a.CT);

    auto issue = [&](int base, f4 (&c)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t addr = rec[wave][base + 4 * u + grp] + off;
            c[u] = *reinterpret_cast<const __attribute__((address_space(1))) f4 *>(addr);
        }
    };
    auto consume = [&](int base, const f4 (&c)[U], f4 &acc) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = wgt[wave][base + 4 * u + grp];
            acc.x = __builtin_fmaf(w, c[u].x, acc.x);
            acc.y = __builtin_fmaf(w, c[u].y, acc.y);
            acc.z = __builtin_fmaf(w, c[u].z, acc.z);
            acc.w = __builtin_fmaf(w, c[u].w, acc.w);
        }
    };

    if (lw >= nq) return;
    // current query's span, and the next one's (prefetched one batch ahead)
    auto span = [&](int64_t q, int64_t &b, int64_t &len, bool &ok) {
        b = 0;
        len = 0;
        ok = q < nq;
        if (ok) {
            const int64_t bb = a.indptr[q], ee = a.indptr[q + 1];
            ok = bb >= 0 && ee >= bb && ee <= a.nnz;
            if (ok) {
                b = bb;
                len = ee - bb;
            }
        }
    };
    int32_t pk = 0;
    float pv = 0.0f;
    auto prefetch = [&](int64_t b, int64_t len, int64_t t) {
        pk = 0;
        pv = 0.0f;
        if (t + lane < len) {
            pk = stream_load(a.indices + b + t + lane);
            pv = stream_load(a.values + b + t + lane);
        }
    };

    int64_t q = lw, b, len;
    bool ok;
    span(q, b, len, ok);
    prefetch(b, len, 0);
    while (true) {
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        int64_t nb = 0, nlen = 0;
        bool nok = false, more = false;
        const int64_t qn = q + waves_per_group;
        for (int64_t t = 0; t < len; t += 64) {
            int32_t kk = pk;
            float vv = pv;
            if (t + 64 < len) {
                prefetch(b, len, t + 64);
            } else if (qn < nq) {
                span(qn, nb, nlen, nok);
                more = true;
                prefetch(nb, nlen, 0);
            }
            const bool bad = (uint32_t)kk >= (uint32_t)d;
            if (__any(bad)) ok = false;
            if (bad) {
                kk = 0;
                vv = 0.0f;
            }
            rec[wave][lane] = ct + (uint64_t)kk * (uint64_t)ld * 4u;  // past the end: row 0,
            wgt[wave][lane] = vv;                                    // weight 0
            const int64_t rem = len - t;
            const int cnt = (int)((rem < 64 ? rem : 64) + 4 * U - 1) / (4 * U) * (4 * U);
            f4 c0[U], c1[U];
            issue(0, c0);
            for (int u0 = 0; u0 < cnt; u0 += 8 * U) {
                const bool two = u0 + 4 * U < cnt;
                if (two) issue(u0 + 4 * U, c1);
                consume(u0, c0, acc);
                if (two) {
                    if (u0 + 8 * U < cnt) issue(u0 + 8 * U, c0);
                    consume(u0 + 4 * U, c1, acc);
                }
            }
        }
        if (len == 0 && qn < nq) {  // an empty row prefetches nothing above
            span(qn, nb, nlen, nok);
            more = true;
            prefetch(nb, nlen, 0);
        }
        // combine the four lane groups' partial sums: (p0 + p1) + (p2 + p3)
#pragma unroll
        for (int s2 = 16; s2 <= 32; s2 <<= 1) {
            acc.x += __shfl_xor(acc.x, s2);
            acc.y += __shfl_xor(acc.y, s2);
            acc.z += __shfl_xor(acc.z, s2);
            acc.w += __shfl_xor(acc.w, s2);
        }
        float be = __builtin_inff();
        int32_t bi = -1;
        if (live && ok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float r = rank_value<M>(acc[e], cn4[e]);
                if (r < be) {
                    be = r;
                    bi = n0 + e;
                }
            }
        }
#pragma unroll
        for (int s2 = 8; s2 >= 1; s2 >>= 1) {  // within a lane group (all groups agree)
            const float oe = __shfl_xor(be, s2);
            const int32_t oi = __shfl_xor(bi, s2);
            if (oi >= 0 && (bi < 0 || oe < be || (oe == be && oi < bi))) {
                be = oe;
                bi = oi;
            }
        }
        if (lane == 0 && ok && bi >= 0) {
            const uint64_t key = pack_key(be, (uint32_t)bi);
            if (key < mine[q]) mine[q] = key;
        }
        if (!more) break;
        q = qn;
        b = nb;
        len = nlen;
        ok = nok;
    }
}

__global__ __launch_bounds__(256) void k_min_partials(const uint64_t *__restrict__ part,
                                                     int32_t groups, int64_t nq,
                                                     uint64_t *__restrict__ keys) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= nq) return;
    uint64_t k = part[q];
    for (int x = 1; x < groups; ++x) {
        const uint64_t o = part[(int64_t)x * nq + q];
        k = o < k ? o : k;
    }
    keys[q] = k;
}

// Neurons per chunk: 64 (one query per wave) by default, 32 (two queries
// per wave, half the codebook slice per XCD) with VS_CSR_CHUNK=32.  Both give
// identical results; 64 halves the rounds and with them the re-reads of the
// CSR arrays, which measured faster on the 65,536-neuron codebook.
static int csr_chunk() {
    const char *env = getenv("VS_CSR_CHUNK");
    return (env && env[0] == '3') ? 32 : 64;
}

int32_t csr_groups(int64_t nc) {
    const int64_t chunks = (nc + 31) / 32;  // the larger count of the two chunk widths
    return (int32_t)(chunks < 8 ? chunks : 8);
}

hipError_t launch_csr(const CsrArgs &a0, int metric, hipStream_t st, int n_cu,
                      uint64_t *part) {
    CsrArgs a = a0;
    const int ncw = csr_chunk();
    a.n_chunks = (a.nc + ncw - 1) / ncw;
    const int32_t groups = (int32_t)(a.n_chunks < 8 ? a.n_chunks : 8);
    // workgroups per group: enough waves for the queries, at most a full chip
    const int64_t cu = n_cu > 0 ? n_cu : 256;
    int64_t per_group = (cu * kCsrWgPerCu) / groups;
    const int64_t need = (a.nq + 4 * (64 / ncw) - 1) / (4 * (64 / ncw));
    if (per_group > need) per_group = need;
    if (per_group < 1) per_group = 1;
    const dim3 grid((unsigned)(per_group * groups)), block(256);
    const int64_t rounds = (a.n_chunks + groups - 1) / groups;
    hipError_t err = launch_fill_keys(part, (int64_t)groups * a.nq, st);
    if (err != hipSuccess) return err;
    const bool q4 = ncw == 64 && a.nc % 4 == 0 && a.ldct % 4 == 0 &&
                    (reinterpret_cast<uintptr_t>(a.CT) & 15) == 0 && getenv("VS_CSR_DWORD") == nullptr;
    for (int64_t r = 0; r < rounds; ++r) {
        timing_before(st, "k_bmu_csr");
        if (q4) {
            switch (metric) {
            case L2SQ_MIN: hipLaunchKernelGGL(k_bmu_csr_q4<L2SQ_MIN>, grid, block, 0, st, a, part, r, groups); break;
            case L2SQ_MAX: hipLaunchKernelGGL(k_bmu_csr_q4<L2SQ_MAX>, grid, block, 0, st, a, part, r, groups); break;
            case COS_MAX: hipLaunchKernelGGL(k_bmu_csr_q4<COS_MAX>, grid, block, 0, st, a, part, r, groups); break;
            default: hipLaunchKernelGGL(k_bmu_csr_q4<COS_MIN>, grid, block, 0, st, a, part, r, groups); break;
            }
        } else if (ncw == 32) {
            switch (metric) {
            case L2SQ_MIN: hipLaunchKernelGGL((k_bmu_csr<L2SQ_MIN, 2>), grid, block, 0, st, a, part, r, groups); break;
            case L2SQ_MAX: hipLaunchKernelGGL((k_bmu_csr<L2SQ_MAX, 2>), grid, block, 0, st, a, part, r, groups); break;
            case COS_MAX: hipLaunchKernelGGL((k_bmu_csr<COS_MAX, 2>), grid, block, 0, st, a, part, r, groups); break;
            default: hipLaunchKernelGGL((k_bmu_csr<COS_MIN, 2>), grid, block, 0, st, a, part, r, groups); break;
            }
        } else {
            switch (metric) {
            case L2SQ_MIN: hipLaunchKernelGGL((k_bmu_csr<L2SQ_MIN, 1>), grid, block, 0, st, a, part, r, groups); break;
            case L2SQ_MAX: hipLaunchKernelGGL((k_bmu_csr<L2SQ_MAX, 1>), grid, block, 0, st, a, part, r, groups); break;
            case COS_MAX: hipLaunchKernelGGL((k_bmu_csr<COS_MAX, 1>), grid, block, 0, st, a, part, r, groups); break;
            default: hipLaunchKernelGGL((k_bmu_csr<COS_MIN, 1>), grid, block, 0, st, a, part, r, groups); break;
            }
        }
        err = hipGetLastError();
        timing_after(st);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(k_min_partials, dim3((unsigned)((a.nq + 255) / 256)), block, 0, st, part,
                       groups, a.nq, a.keys);
    return hipGetLastError();
}

}  // namespace vs
