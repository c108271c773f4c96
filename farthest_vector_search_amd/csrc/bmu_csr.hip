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
// contiguous, so the lanes that own consecutive neurons read the codebook
// row segment of each non-zero with one coalesced load.  On this data a
// codebook value is needed by ~1.3 of the queries that share a tile, so
// reuse comes from the cache, not from LDS or registers: the kernel is bound
// by on-chip (L2) bandwidth at 4 bytes per multiply-add, and the design goal
// is that those bytes are L2 hits that arrive with enough loads in flight.
//
// Neuron-axis chunking, gfx950 style: a wave owns a chunk of 64 neurons (32
// in the two-queries-per-wave variant); the codebook slice of a 64-neuron
// chunk is d x 256 bytes (4 MiB at d = 16,384), one XCD's L2.  Each launch
// is one "round": P <= 8 groups of workgroups, group x = blockIdx % P (the
// hardware deals consecutive workgroups to the eight XCDs in turn, so with
// P = 8 a group is one XCD) works on chunk round*P + x, its waves splitting
// all queries between them.  The kernel boundary between rounds keeps every
// XCD on a single chunk (a hard step, as the dispatch-per-tile variant of
// "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
// "Intended Behavior", proposes), instead of letting waves drift across
// chunks and thrash the L2.
//
// Codebook addressing: feature k of neuron 64 b + j is at CT + b * cstride
// bytes + (k * ldct + j) floats.  For the plain feature-major layout
// cstride = 256 and the row stride ldct is a parameter (a stride that is a
// multiple of a large power of two maps every row's slice onto the same few
// L2 sets, so callers can pad it); a slice is then d segments spread over the
// whole array, one address-translation entry each.  The 64-neuron blocked
// layout (ldct = 64, cstride = d * 256) makes each slice contiguous.
//
// Merge: the wave that owns (group x, query q) is the only writer of
// partial[x][q] in its round, and rounds are ordered on the stream, so the
// running best per (group, query) is a read-min-write (an atomicMin in the
// pipelined kernel); a final pass takes the minimum over the P groups.
// Packed (value, index) keys make both minima exact and order-independent
// (lowest index on ties).  Rows with an out-of-range indptr span or column
// index are skipped whole (nothing outside the arrays is read) and keep the
// "no candidate" key.
#include <cstdlib>

#include "vs_internal.h"

namespace vs {

#ifndef VS_CSR_WG_PER_CU
#define VS_CSR_WG_PER_CU 7
#endif
constexpr int kCsrWgPerCu = VS_CSR_WG_PER_CU;  // x 4 waves resident per CU (VGPR-limited)
// The pipelined kernel is launched with more workgroups than can be resident
// (4 waves per SIMD fit): its queries are dealt round-robin to waves, so more,
// shorter waves even out the end of a round (measured: 0.512 ms per round at
// 4 workgroups per CU, 0.491 at 8, 0.472 at 32)
#ifndef VS_CSR_RING_WG_PER_CU
#define VS_CSR_RING_WG_PER_CU 32
#endif
constexpr int kCsrRingWgPerCu = VS_CSR_RING_WG_PER_CU;
#ifndef VS_CSR_UNROLL
#define VS_CSR_UNROLL 8
#endif
constexpr int kCsrUnroll = VS_CSR_UNROLL;  // loads per group (two groups in flight)
#ifndef VS_CSR_RING
#define VS_CSR_RING 16
#endif

constexpr int kCsrRing = VS_CSR_RING;  // loads in flight per wave in the pipelined scan
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
    // the chunk's first neuron inside its 64-neuron block; dead lanes read
    // the chunk's first column
    const int64_t n_first = chunk * NCW;
    const uint64_t cbase = reinterpret_cast<uint64_t>(a.CT) + (uint64_t)(n_first >> 6) * a.cstride +
                           (uint64_t)(n_first & 63) * 4u;
    const uint64_t off = (uint64_t)(live ? sub : 0) * 4u;
    const float cn = (metric_is_l2(M) && live) ? a.cn[n] : 0.0f;
    uint64_t *mine = part + (int64_t)x * nq;
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
                rec[wave][hh][lane] = cbase + (uint64_t)kk[hh] * (uint64_t)ld * 4u;
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

// Four-rows-per-load, pipelined form (codebook rows 16-byte aligned,
// nc % 4 == 0).  A wave owns 64 neurons; one 16-byte-per-lane load covers
// four non-zeros: lane group g = lane / 16 reads row k of non-zero 4i+g, the
// 16 lanes of a group four consecutive neurons each (one 256-byte row
// segment).  Wide loads reach about twice the L2 -> CU bandwidth of 4-byte
// loads.  Each lane sums every fourth non-zero for its 4 neurons in order;
// the four partial sums are combined in one fixed order ((p0 + p1) +
// (p2 + p3)), the order the 4-byte-load kernel also uses, so both give the
// same bits.  The scan is latency-bound: what limits it is how many
// codebook loads each wave keeps in flight.  Here a wave's work is one stream of
// batches of 4N non-zeros (a query is cut into ceil(len / 4N) batches, at
// least one; the tail of its last batch is zero weights).  A batch is N
// load units (LU: four consecutive non-zeros, one 16-byte load per lane),
// and a ring of N register slots runs one batch behind the loads: rotation
// r consumes the LUs of batch r - 1 slot by slot and refills each slot with
// the matching LU of batch r, so N loads stay in flight across batch and
// query boundaries instead of draining at each batch.
//  - At the start of a rotation the batch's (k, v) (loaded into registers,
//    one non-zero per lane, at the start of the previous rotation, so N + 1
//    loads have been issued behind them) become row-address records in LDS;
//    then the (k, v) of the next batch are loaded.  Every step issues
//    exactly one codebook load, so the wait for a slot is vmcnt(N - 1).
//  - A query is finalised after the rotation that consumed its last batch;
//    the (group, query) result is merged with a 64-bit atomicMin (nothing
//    returned, nothing waited for).
template <int M, int N, bool HALF>
__global__ __launch_bounds__(256) void k_bmu_csr_ring(const CsrArgs a, uint64_t *__restrict__ part,
                                                     int64_t round, int32_t groups) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    constexpr int NPL = HALF ? 8 : 4;    // neurons per lane (one 16-byte load)
    constexpr int CW = 16 * NPL;         // neurons per chunk
    constexpr uint64_t ESZ = HALF ? 2 : 4;  // bytes per codebook value
    constexpr int B = 4 * N;  // non-zeros per batch
    static_assert(B <= 64, "a batch is staged by one wave, one non-zero per lane");
    __shared__ uint64_t rec[4][2][B]; // per wave, by rotation parity: row addresses of a batch
    __shared__ float wgt[4][2][B];    // ... and weights
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 4, col = lane & 15;
    const int x = (int)(blockIdx.x % (unsigned)groups);
    const int64_t local = blockIdx.x / (unsigned)groups;
    const int64_t chunk = round * groups + x;
    if (chunk >= a.n_chunks) return;
    const int64_t wpg = (int64_t)(gridDim.x / (unsigned)groups) * 4;  // waves per group
    const int64_t lw = __builtin_amdgcn_readfirstlane((int)(local * 4 + wave));
    const int64_t nq = a.nq, nc = a.nc, ld = a.ldct;
    const int32_t d = a.d;
    if (lw >= nq) return;
    const int32_t n0 = (int32_t)(chunk * CW + NPL * col);  // this lane's NPL neurons
    // a lane past nc reads the chunk's first columns (fp32: nc % 4 == 0, so a
    // lane's 4 neurons are all live or all dead; fp16: the blocked copy is
    // padded to whole chunks, and each neuron is checked at the end)
    const bool live = n0 < nc;
    const uint64_t off = (uint64_t)(HALF || live ? NPL * col : 0) * ESZ;
    float cnv[NPL];
#pragma unroll
    for (int e = 0; e < NPL; ++e)
        cnv[e] = (metric_is_l2(M) && n0 + e < nc) ? a.cn[n0 + e] : 0.0f;
    unsigned long long *mine = reinterpret_cast<unsigned long long *>(part + (int64_t)x * nq);
    const uint64_t cbase = reinterpret_cast<uint64_t>(a.CT) + (uint64_t)chunk * a.cstride;
    const __attribute__((address_space(4))) int32_t *indptr =
        (const __attribute__((address_space(4))) int32_t *)a.indptr;
    const int32_t n_my = (int32_t)((nq - lw + wpg - 1) / wpg);  // queries of this wave

    // ---- the batch stream (wave-uniform state).  "Staged": the batch whose
    // (k, v) are in (pk, pv) (or on their way).
    int32_t s_n = 0;      // its query (number within this wave's queries)
    int64_t s_b = 0;      // the query's CSR base
    int32_t s_len = 0;    // the query's length
    bool s_ok = true;     // the query's span is valid
    int32_t s_t = 0;      // the batch's first non-zero
    bool s_has = false;   // a staged batch exists
    // (readfirstlane keeps the stream state in scalar registers, so the
    // span is read with scalar loads, which never hold the vector-load
    // counter the ring relies on)
    auto open_query = [&](int32_t n) {
        n = __builtin_amdgcn_readfirstlane(n);
        const int64_t q = lw + (int64_t)n * wpg;
        const int32_t bb = __builtin_amdgcn_readfirstlane(indptr[q]);
        const int32_t ee = __builtin_amdgcn_readfirstlane(indptr[q + 1]);
        s_ok = bb >= 0 && ee >= bb && ee <= a.nnz;
        s_b = s_ok ? bb : 0;
        s_len = s_ok ? ee - bb : 0;
        s_n = n;
        s_t = 0;
        s_has = true;
    };
    // lane j < B fetches non-zero s_t + j of the staged batch into (pk, pv),
    // plain loads with the index clamped into the row (lanes past its end
    // are zeroed when the records are made); an empty row loads nothing
    int32_t pk = 0;
    float pv = 0.0f;
    auto stage = [&]() {
        if (s_len > 0) {
            const int32_t t = s_t + lane;
            const int64_t at = s_b + (t < s_len ? t : s_len - 1);
            pk = a.indices[at];  // plain loads: non-temporal ones measured slower here
            pv = a.values[at];
        }
    };

    // Turns the staged batch into the records of parity p and stages the
    // next one.  Returns, for the batch now in the records: its query,
    // whether it is the query's last batch, and whether the query is still
    // valid.
    bool i_ok = true;  // validity of the query being issued, over its batches so far
    auto make_records = [&](int p, int32_t &q_out, bool &last_out, bool &ok_out) {
        const bool in = lane < B && s_t + lane < s_len;
        int32_t kk = in ? pk : 0;
        float vv = in ? pv : 0.0f;
        const bool bad = (uint32_t)kk >= (uint32_t)d;
        if (bad) {
            kk = 0;
            vv = 0.0f;
        }
        if (lane < B) {
            rec[wave][p][lane] = cbase + (uint64_t)kk * (uint64_t)ld * ESZ;  // past the end: row 0,
            wgt[wave][p][lane] = vv;                                        // weight 0
        }
        if (s_t == 0) i_ok = s_ok;
        if (__any(bad)) i_ok = false;
        q_out = s_n;
        ok_out = i_ok;
        last_out = s_t + B >= s_len;
        // the next batch
        if (!last_out) {
            s_t += B;
        } else if (s_n + 1 < n_my) {
            open_query(s_n + 1);
        } else {
            s_has = false;
            return;
        }
        stage();
    };

    float acc[NPL];
#pragma unroll
    for (int e = 0; e < NPL; ++e) acc[e] = 0.0f;
    auto finalize = [&](int32_t n, bool ok) {
        const int64_t q = lw + (int64_t)__builtin_amdgcn_readfirstlane(n) * wpg;
        float sv[NPL];
        // combine the four lane groups' partial sums: (p0 + p1) + (p2 + p3)
#pragma unroll
        for (int e = 0; e < NPL; ++e) {
            sv[e] = acc[e];
            sv[e] += __shfl_xor(sv[e], 16);
            sv[e] += __shfl_xor(sv[e], 32);
        }
        float be = __builtin_inff();
        int32_t bi = -1;
        if (ok) {
#pragma unroll
            for (int e = 0; e < NPL; ++e) {
                const float r = rank_value<M>(sv[e], cnv[e]);
                if (n0 + e < nc && r < be) {
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
        if (lane == 0 && ok && bi >= 0)
            atomicMin(mine + q, (unsigned long long)pack_key(be, (uint32_t)bi));
#pragma unroll
        for (int e = 0; e < NPL; ++e) acc[e] = 0.0f;
    };
    // one load unit into the running sums: NPL products of weight w and the
    // slot's values (fp16 values are widened exactly to fp32 first)
    auto fma_slot = [&](float w, const f4 &v) {
        if constexpr (HALF) {
            const h8 hv = __builtin_bit_cast(h8, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w, (float)hv[e], acc[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, v[e], acc[e]);
        }
    };

    // ---- prologue: batch 0 staged, made current, and issued into the ring
    open_query(0);
    stage();
    int32_t q_cur = 0;
    bool last_cur = false, ok_cur = true;
    int par = 0;
    make_records(par, q_cur, last_cur, ok_cur);
    f4 buf[N];
#pragma unroll
    for (int j = 0; j < N; ++j)
        buf[j] = *reinterpret_cast<const __attribute__((address_space(1))) f4 *>(
            rec[wave][par][4 * j + grp] + off);
    while (true) {
        // the ring holds the batch of parity par; the staged batch becomes
        // the next one
        const int32_t q_prev = q_cur;
        const bool last_prev = last_cur, ok_prev = ok_cur;
        const int pp = par;
        if (s_has) {
            par ^= 1;
            make_records(par, q_cur, last_cur, ok_cur);
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const int r = 4 * j + grp;
                fma_slot(wgt[wave][pp][r], buf[j]);
                buf[j] = *reinterpret_cast<const __attribute__((address_space(1))) f4 *>(
                    rec[wave][par][r] + off);
                // keep slot j's refill after its use (hoisting the loads would
                // need a second set of slot registers)
                __builtin_amdgcn_sched_barrier(0);
            }
            if (last_prev) finalize(q_prev, ok_prev);
        } else {  // last rotation: nothing left to issue
#pragma unroll
            for (int j = 0; j < N; ++j) {
                fma_slot(wgt[wave][pp][4 * j + grp], buf[j]);
            }
            finalize(q_prev, ok_prev);  // the stream's last batch ends its query
            break;
        }
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
    const bool wide_ok = a.nc % 4 == 0 && a.ldct % 4 == 0 && a.cstride % 16 == 0 &&
                         (reinterpret_cast<uintptr_t>(a.CT) & 15) == 0 &&
                         getenv("VS_CSR_DWORD") == nullptr;
    const int ncw = csr_chunk();
    a.n_chunks = (a.nc + ncw - 1) / ncw;
    const int32_t groups = (int32_t)(a.n_chunks < 8 ? a.n_chunks : 8);
    // workgroups per group: enough waves for the queries, at most a full chip
    const int64_t cu = n_cu > 0 ? n_cu : 256;
    const bool ring = ncw == 64 && wide_ok;
    int64_t per_group = (cu * (ring ? kCsrRingWgPerCu : kCsrWgPerCu)) / groups;
    const int qpw = ncw == 32 ? 2 : 1;  // queries per wave
    const int64_t need = (a.nq + 4 * qpw - 1) / (4 * qpw);
    if (per_group > need) per_group = need;
    if (per_group < 1) per_group = 1;
    const dim3 grid((unsigned)(per_group * groups)), block(256);
    const int64_t rounds = (a.n_chunks + groups - 1) / groups;
    hipError_t err = launch_fill_keys(part, (int64_t)groups * a.nq, st);
    if (err != hipSuccess) return err;
    for (int64_t r = 0; r < rounds; ++r) {
        timing_before(st, "k_bmu_csr");
        if (ring) {
            switch (metric) {
            case L2SQ_MIN: hipLaunchKernelGGL((k_bmu_csr_ring<L2SQ_MIN, kCsrRing, false>), grid, block, 0, st, a, part, r, groups); break;
            case L2SQ_MAX: hipLaunchKernelGGL((k_bmu_csr_ring<L2SQ_MAX, kCsrRing, false>), grid, block, 0, st, a, part, r, groups); break;
            case COS_MAX: hipLaunchKernelGGL((k_bmu_csr_ring<COS_MAX, kCsrRing, false>), grid, block, 0, st, a, part, r, groups); break;
            default: hipLaunchKernelGGL((k_bmu_csr_ring<COS_MIN, kCsrRing, false>), grid, block, 0, st, a, part, r, groups); break;
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

// fp16 codebook in the 128-neuron blocked layout (feature k of neuron
// 128 b + j at CT + b * cstride + (k * 128 + j) halves): the pipelined scan
// with eight neurons per lane, 128-neuron chunks (a 4 MiB slice at
// d = 16,384), every value widened exactly to fp32 before its FMA.
hipError_t launch_csr_f16(const CsrArgs &a0, int metric, hipStream_t st, int n_cu,
                          uint64_t *part) {
    CsrArgs a = a0;
    constexpr int CW = 128;
    a.n_chunks = (a.nc + CW - 1) / CW;
    const int32_t groups = (int32_t)(a.n_chunks < 8 ? a.n_chunks : 8);
    const int64_t cu = n_cu > 0 ? n_cu : 256;
    int64_t per_group = (cu * kCsrRingWgPerCu) / groups;
    const int64_t need = (a.nq + 3) / 4;
    if (per_group > need) per_group = need;
    if (per_group < 1) per_group = 1;
    const dim3 grid((unsigned)(per_group * groups)), block(256);
    const int64_t rounds = (a.n_chunks + groups - 1) / groups;
    hipError_t err = launch_fill_keys(part, (int64_t)groups * a.nq, st);
    if (err != hipSuccess) return err;
    for (int64_t r = 0; r < rounds; ++r) {
        timing_before(st, "k_bmu_csr");
        switch (metric) {
        case L2SQ_MIN: hipLaunchKernelGGL((k_bmu_csr_ring<L2SQ_MIN, kCsrRing, true>), grid, block, 0, st, a, part, r, groups); break;
        case L2SQ_MAX: hipLaunchKernelGGL((k_bmu_csr_ring<L2SQ_MAX, kCsrRing, true>), grid, block, 0, st, a, part, r, groups); break;
        case COS_MAX: hipLaunchKernelGGL((k_bmu_csr_ring<COS_MAX, kCsrRing, true>), grid, block, 0, st, a, part, r, groups); break;
        default: hipLaunchKernelGGL((k_bmu_csr_ring<COS_MIN, kCsrRing, true>), grid, block, 0, st, a, part, r, groups); break;
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
