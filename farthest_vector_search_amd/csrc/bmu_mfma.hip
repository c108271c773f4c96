// bmu_mfma.hip -- dense scan of queries against a candidate table on the
// gfx950 matrix cores, fused with the arg-reduction (no score ever reaches
// memory).
//
// What it computes: for every query q and candidate c the dot product q.c,
// turned into a ranking value (squared L2: |c|^2 - 2 q.c; cosine on unit
// rows: +-q.c), then per query the best candidate with the lowest index on
// ties.  Sources (web pages, by title and section):
//  - "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof ..."
//    (summary), section 3: the BMU search; the arg-min there is taken inside
//    the distance kernel, so no query x neuron distance is ever stored;
//  - "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
//    "Intended Behavior": walk the candidates in tiles, all workgroups on the
//    same tile, the running best carried across tiles (never reset); the
//    winner does not depend on the tiling because max is associative;
//  - "Tiling en memoria compartida: el factor 16", "El kernel": stage tiles
//    in workgroup memory with coalesced loads, pad out-of-range elements
//    with zero instead of leaving early, one barrier between loading and
//    computing and one before a buffer is overwritten;
//  - same page, "Tiling en registros": each thread owns a block of outputs
//    so every staged value feeds several products (here an MFMA tile).
//
// gfx950 design (not the pages' GPU designs):
//  - v_mfma_f32_32x32x2f32: candidates are the MFMA rows, queries the
//    columns.  A lane's accumulator holds 16 candidates of ONE query, so the
//    per-tile reduction is lane-local compares; the running best lives in
//    two registers per query for the workgroup's whole candidate sweep.
//  - Workgroup = 4 waves (2 along queries x 2 along candidates), 128 queries
//    x 128 candidates per work item, each wave a 2x2 grid of 32x32 MFMA
//    blocks.  K runs in slabs of 32 features through double-buffered LDS
//    (64 KiB), one barrier per slab.  Each LDS row is 8 pieces of 16 bytes
//    stored at slot (piece XOR (row/2)%8): loads stay 128-byte coalesced and
//    the 16-byte LDS reads of the MFMA operands hit distinct banks.
//  - Operand order inside K: lane half h feeds features {8c+4h .. 8c+4h+3}
//    of chunk c, one per MFMA, from one 16-byte LDS read; both operands use
//    the same map, so every pair's sum runs over the same fixed sequence of
//    features whatever tile, wave or workgroup computes it.  No split over K.
//  - Work items = (query tile, candidate tile), query-tile major; workgroup g
//    takes one contiguous run.  With a full grid every workgroup owns whole
//    query tiles and all of them sweep the candidate tiles in the same order.
//    Consecutive workgroup ids land on different XCDs, so ids are renumbered
//    to give each XCD one contiguous run of items.
//  - A workgroup flushes a query's best with a 64-bit atomicMin on the packed
//    (value, index) key whenever its run leaves a query tile; the minimum of
//    packed keys is exact and order-independent, so any split of the
//    candidate range gives the same bits.
#include "vs_internal.h"

namespace vs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 32;  // features per slab = 8 pieces of 4 floats

// LDS banks are 64 x 4 bytes, so a 128-byte row covers half of them and rows
// r and r+1 fall on opposite halves: the slot key uses row/2 so that the 16
// rows one 16-lane group reads at a time land on 16 distinct bank groups.
__device__ __forceinline__ int lds_at(int row, int piece) {
    return row * kBK + ((piece ^ ((row >> 1) & 7)) << 2);
}

template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float *p, int32_t k, int32_t d) {
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p != nullptr) {
        if constexpr (VEC) {
            if (k < d) v = *reinterpret_cast<const f32x4 *>(p + k);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < d) v[e] = p[k + e];
        }
    }
    return v;
}

template <int M, int QM, bool VEC, int WQ, int WC>
__global__ __launch_bounds__(64 * WQ * WC) __attribute__((amdgpu_waves_per_eu(2)))
void k_bmu_mfma(const DenseArgs a) {
    constexpr bool GATHER = QM == kQGatherMasked;
    constexpr int NT = 64 * WQ * WC;
    constexpr int BQ = 64 * WQ, BC = 64 * WC;
    constexpr int RPP = NT / 8;  // rows per loader pass
    constexpr int AP = BC / RPP, BP = BQ / RPP;
    static_assert(BC % RPP == 0 && BQ % RPP == 0, "tile/loader mismatch");
    constexpr bool MASKED = QM != kQRows;  // the diversity step, gathered or explicit

    __shared__ __attribute__((aligned(16))) float sA[2][BC * kBK];
    __shared__ __attribute__((aligned(16))) float sB[2][BQ * kBK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wave = tid >> 6, wc = wave % WC, wq = wave / WC;

    int g = blockIdx.x;
    const int G = a.grid;
    if ((G & 7) == 0) g = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
    const int64_t it0 = (int64_t)g * a.n_items / G;
    const int64_t it1 = (int64_t)(g + 1) * a.n_items / G;
    if (it0 >= it1) return;  // whole workgroup: no barrier is skipped by part of it

    const int32_t d = a.d;
    const int64_t nq = a.nq, nc = a.nc, nct = a.n_ctiles;
    const int nslab = (d + kBK - 1) / kBK;
    const int lrow = tid >> 3, lpiece = tid & 7;

    const float *aptr[AP];
    const float *bptr[BP];
    f32x4 ra[AP], rb[BP];

    auto set_rows = [&](int64_t item) {
        const int64_t qt = item / nct, ct = item - qt * nct;
#pragma unroll
        for (int i = 0; i < AP; ++i) {
            const int64_t c = ct * BC + lrow + i * RPP;
            aptr[i] = c < nc ? a.C + c * d : nullptr;
        }
#pragma unroll
        for (int i = 0; i < BP; ++i) {
            const int64_t q = qt * BQ + lrow + i * RPP;
            if constexpr (GATHER) {
                const int64_t p = q < nq ? (int64_t)a.pick[q] : -1;
                bptr[i] = (p >= 0 && p < nc) ? a.C + p * d : nullptr;
            } else {
                bptr[i] = q < nq ? a.Q + q * d : nullptr;
            }
        }
    };
    auto fetch = [&](int slab) {
        const int32_t k = slab * kBK + 4 * lpiece;
#pragma unroll
        for (int i = 0; i < AP; ++i) ra[i] = load4<VEC>(aptr[i], k, d);
#pragma unroll
        for (int i = 0; i < BP; ++i) rb[i] = load4<VEC>(bptr[i], k, d);
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AP; ++i)
            *reinterpret_cast<f32x4 *>(&sA[buf][lds_at(lrow + i * RPP, lpiece)]) = ra[i];
#pragma unroll
        for (int i = 0; i < BP; ++i)
            *reinterpret_cast<f32x4 *>(&sB[buf][lds_at(lrow + i * RPP, lpiece)]) = rb[i];
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) acc[cb][qb] = f32x16{};
    float best[2] = {__builtin_inff(), __builtin_inff()};
    int32_t bidx[2] = {-1, -1};

    auto compute = [&](int buf) {
        const float *A = sA[buf];
        const float *B = sB[buf];
#pragma unroll
        for (int c = 0; c < kBK / 8; ++c) {
            const int piece = 2 * c + h;
            f32x4 af[2], bf[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                af[cb] = *reinterpret_cast<const f32x4 *>(&A[lds_at(wc * 64 + cb * 32 + l32, piece)]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                bf[qb] = *reinterpret_cast<const f32x4 *>(&B[lds_at(wq * 64 + qb * 32 + l32, piece)]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        acc[cb][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[cb][e], bf[qb][e],
                                                                           acc[cb][qb], 0, 0, 0);
        }
    };

    // Fold the finished dot products of one item into the running bests.
    // Accumulator register r of a lane holds candidate row 8*(r/4)+4h+(r%4)
    // of the 32-row block and query column l32; rows rise with r, blocks and
    // tiles are visited in ascending order, so strict "<" keeps the lowest
    // index among a lane's ties.
    auto epilogue = [&](int64_t item) {
        const int64_t qt = item / nct, ct = item - qt * nct;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int64_t blk = ct * BC + wc * 64 + cb * 32;
            float cnv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t c = blk + 8 * (r >> 2) + 4 * h + (r & 3);
                cnv[r] = (metric_is_l2(M) && c < nc) ? a.cn[c] : 0.0f;
            }
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                uint32_t mw = 0;
                if constexpr (MASKED) {
                    const int64_t q = qt * BQ + wq * 64 + qb * 32 + l32;
                    if (q < nq && blk < nc) mw = a.mask[q * a.mask_words + (blk >> 5)];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 8 * (r >> 2) + 4 * h + (r & 3);
                    const int64_t c = blk + row;
                    const float e = rank_value<M>(acc[cb][qb][r], cnv[r]);
                    const bool live = c < nc && !((mw >> row) & 1u);
                    if (live && e < best[qb]) {
                        best[qb] = e;
                        bidx[qb] = (int32_t)c;
                    }
                }
                acc[cb][qb] = f32x16{};
            }
        }
    };

    // Merge the two lane halves (same query, interleaved candidate rows) and
    // publish each query's best with one packed atomicMin.
    auto flush = [&](int64_t item) {
        const int64_t qt = item / nct;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float oe = __shfl_xor(best[qb], 32);
            const int32_t oi = __shfl_xor(bidx[qb], 32);
            if (oi >= 0 && (bidx[qb] < 0 || oe < best[qb] || (oe == best[qb] && oi < bidx[qb]))) {
                best[qb] = oe;
                bidx[qb] = oi;
            }
            if (h == 0 && bidx[qb] >= 0) {
                const int64_t q = qt * BQ + wq * 64 + qb * 32 + l32;
                bool ok = q < nq;
                if constexpr (GATHER) {
                    if (ok) {
                        const int64_t p = a.pick[q];
                        ok = p >= 0 && p < nc;
                    }
                }
                if (ok)
                    atomicMin(reinterpret_cast<unsigned long long *>(a.keys + q),
                              (unsigned long long)pack_key(best[qb], (uint32_t)bidx[qb]));
            }
            best[qb] = __builtin_inff();
            bidx[qb] = -1;
        }
    };

    // Prologue: first slab into buffer 0.
    set_rows(it0);
    fetch(0);
    stash(0);
    __syncthreads();

    int64_t item = it0, litem = it0;
    int slab = 0, lslab = 0, buf = 0;
    while (true) {
        // issue the global loads of the next slab before computing this one
        if (++lslab == nslab) {
            lslab = 0;
            ++litem;
            if (litem < it1) set_rows(litem);
        }
        const bool has_next = litem < it1;
        if (has_next) fetch(lslab);

        compute(buf);

        if (slab == nslab - 1) {
            epilogue(item);
            if (item + 1 == it1 || (item + 1) / nct != item / nct) flush(item);
        }
        if (!has_next) break;
        stash(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        if (++slab == nslab) {
            slab = 0;
            ++item;
        }
    }
}

template <int M, int QM>
static void dispatch_vec(const DenseArgs &a, bool vec, dim3 grid, dim3 block, hipStream_t st) {
    if (vec)
        hipLaunchKernelGGL((k_bmu_mfma<M, QM, true, 2, 2>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((k_bmu_mfma<M, QM, false, 2, 2>), grid, block, 0, st, a);
}

hipError_t launch_dense(const DenseArgs &a0, int metric, int qmode, hipStream_t st, int n_cu) {
    const bool gather = qmode == kQGatherMasked;
    constexpr int BQ = 128, BC = 128, OCC = 2;
    DenseArgs a = a0;
    const int64_t nqt = (a.nq + BQ - 1) / BQ;
    a.n_ctiles = (a.nc + BC - 1) / BC;
    a.n_items = nqt * a.n_ctiles;
    const int64_t cap = (int64_t)(n_cu > 0 ? n_cu : 256) * OCC;
    a.grid = (int32_t)(a.n_items < cap ? a.n_items : cap);
    const bool vec = (a.d % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.C) & 15) == 0) &&
                     (gather || (reinterpret_cast<uintptr_t>(a.Q) & 15) == 0);
    const dim3 grid((unsigned)a.grid), block(256);
    timing_before(st, gather ? "k_bmu_mfma<COS_MIN,gather>"
                             : (qmode == kQRowsMasked ? "k_bmu_mfma<COS_MIN,ref>" : "k_bmu_mfma"));
    if (gather) {
        dispatch_vec<COS_MIN, kQGatherMasked>(a, vec, grid, block, st);
    } else if (qmode == kQRowsMasked) {
        dispatch_vec<COS_MIN, kQRowsMasked>(a, vec, grid, block, st);
    } else {
        switch (metric) {
        case L2SQ_MIN: dispatch_vec<L2SQ_MIN, kQRows>(a, vec, grid, block, st); break;
        case L2SQ_MAX: dispatch_vec<L2SQ_MAX, kQRows>(a, vec, grid, block, st); break;
        case COS_MAX: dispatch_vec<COS_MAX, kQRows>(a, vec, grid, block, st); break;
        default: dispatch_vec<COS_MIN, kQRows>(a, vec, grid, block, st); break;
        }
    }
    const hipError_t err = hipGetLastError();
    timing_after(st);
    return err;
}

}  // namespace vs
