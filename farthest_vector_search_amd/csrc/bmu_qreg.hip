// bmu_qreg.hip -- dense scan for d <= 256 with the queries held in registers.
//
// Same computation and result as bmu_mfma.hip (fp32 MFMA dot products,
// fused ranking and lowest-index arg-reduction, packed-key merge), arranged
// so that HBM/L2 traffic stays near the algorithmic bytes: every wave keeps
// its 32 query rows in VGPRs for its whole candidate sweep (d/2 registers per
// lane), so a query is read from memory once per kernel, and only candidate
// slabs move through LDS.  Sources, by page title and section:
//  - "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
//    "Intended Behavior": every workgroup walks the same candidate tiles in
//    the same order, so a tile is fetched into the cache once and served to
//    all of them; the running best persists across tiles;
//  - "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof ..."
//    (summary), section 3: the argmin fused into the product;
//  - "Tiling en memoria compartida: el factor 16", "Tiling en registros":
//    the reused operand lives in registers (here the query block).
//
// Layout: workgroup = 8 waves = 256 queries (32 per wave, one MFMA column
// block each); work item = (query tile of 256, candidate tile of 64 = two
// 32-row MFMA blocks).  Candidate slabs of 64 features are double-buffered
// in LDS (2 x 16 KiB); a row is 16 pieces of 16 bytes stored at slot
// (piece XOR row%16), which keeps both the 256-byte coalesced global loads
// and the 16-byte MFMA operand reads free of bank conflicts.  Lane half h
// feeds features 8c+4h..8c+4h+3 of chunk c to four consecutive MFMAs from
// one LDS read (candidates) and one register quad (queries); every pair's
// dot product therefore runs over one fixed feature order.
#include "vs_internal.h"

#include <type_traits>

namespace vs {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

#ifndef VS_QREG_BK
#define VS_QREG_BK 64
#endif
#ifndef VS_QREG_PRIO
#define VS_QREG_PRIO 0
#endif

constexpr int kQW = 8;          // waves per workgroup (4 for searches too small to fill the chip)
constexpr int kBC = 64;         // candidates per tile
constexpr int kBK = VS_QREG_BK; // features per LDS slab (64 or 128)
constexpr int kCPS = kBK / 8;   // 8-feature chunks per slab
constexpr int kPieces = kBK / 4;
constexpr int kMaxSlabs = 256 / kBK;
static_assert(kBK == 64 || kBK == 128, "slab width");

__device__ __forceinline__ int slab_at(int row, int piece) {
    return row * kBK + ((piece ^ (row & 15)) << 2);
}

template <bool VEC>
__device__ __forceinline__ f32x4 ld4(const float *p, int32_t k, int32_t d) {
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

}  // namespace

// M is a metric, or kStoreDots: write every dot product to a.S instead of
// ranking (the score block of the unfused comparator).
constexpr int kStoreDots = 4;

template <int M, bool VEC, int NSLAB, int QW>
__global__ __launch_bounds__(64 * QW) __attribute__((amdgpu_waves_per_eu(2)))
void k_bmu_qreg(const DenseArgs a) {
    constexpr int kBQ = 32 * QW;  // queries per tile
    constexpr int NT = 64 * QW;
    constexpr int NCH = NSLAB * kCPS;
    constexpr int RPP = NT / kPieces;  // loader rows per pass (register path)
    constexpr int AP = kBC / RPP;      // loader pieces per thread (register path)
    constexpr int RPW = kBC / QW;      // slab rows owned by each wave (DMA path)
    constexpr int RPI = 64 / kPieces;  // rows per DMA instruction (1 KiB)
    static_assert(kBC % RPP == 0 && RPW % RPI == 0, "loader shape");

    __shared__ __attribute__((aligned(16))) float sA[2][kBC * kBK];
    __shared__ __attribute__((aligned(16))) float sN[2][kBC];  // candidate norms, by item parity

    const int tid = threadIdx.x;
    const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wave = tid >> 6;

    int g = blockIdx.x;
    const int G = a.grid;
    if ((G & 7) == 0) g = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
    const int64_t it0 = (int64_t)g * a.n_items / G;
    const int64_t it1 = (int64_t)(g + 1) * a.n_items / G;
    if (it0 >= it1) return;

    const int32_t d = a.d;
    const int64_t nq = a.nq, nc = a.nc;
    const int32_t nct = (int32_t)a.n_ctiles;  // nc < 2^31 rows

    f32x4 qreg[NCH];
    auto load_queries = [&](int64_t qt) {
        const int64_t q = qt * kBQ + wave * 32 + l32;
        const float *p = q < nq ? a.Q + q * d : nullptr;
#pragma unroll
        for (int c = 0; c < NCH; ++c) qreg[c] = ld4<VEC>(p, 8 * c + 4 * h, d);
    };

    // ---- candidate slab loader ----------------------------------------
    // VEC: direct-to-LDS.  Wave w fills rows [RPW w, RPW w + RPW); one
    // instruction covers RPI rows x kPieces slots, lane l -> row +l/kPieces,
    // slot l%kPieces, which holds piece slot ^ (row % 16) of that row.  The
    // source of each lane is fixed per candidate tile (a 32-bit element
    // offset from the tile's first row, kept in voff); a slab only moves the
    // tile's base.  Rows past nc re-read row nc - 1 (their results are
    // discarded); features >= d are written as zeros with ds_write.
    // Scalar path: through registers, as in the tiled kernel.
    const int lrow = tid / kPieces, lpiece = tid % kPieces;
    const float *aptr[AP];
    f32x4 ra[AP];
    uint32_t voff[RPW / RPI];
    int32_t dpiece[RPW / RPI];  // 4 x the piece this lane loads
    int32_t row_base = 0;       // first candidate of the tile being loaded
    auto set_rows = [&](int32_t ctile) {
        row_base = ctile * kBC;
        if constexpr (VEC) {
            const int32_t last = (int32_t)(nc - row_base) - 1;  // last row of the tile inside C
#pragma unroll
            for (int i = 0; i < RPW / RPI; ++i) {
                const int row = wave * RPW + RPI * i + lane / kPieces;
                const int piece = (lane % kPieces) ^ (row & 15);
                dpiece[i] = 4 * piece;
                voff[i] = (uint32_t)((row < last ? row : last) * d + 4 * piece);
            }
        } else {
#pragma unroll
            for (int i = 0; i < AP; ++i) {
                const int64_t c = (int64_t)row_base + lrow + i * RPP;
                aptr[i] = c < nc ? a.C + c * d : nullptr;
            }
        }
    };
    auto load_slab = [&](int slab, int buf) {
        if constexpr (VEC) {
            const float *tile = a.C + (int64_t)row_base * d + slab * kBK;
            if ((slab + 1) * kBK <= d) {  // uniform: no feature past d
#pragma unroll
                for (int i = 0; i < RPW / RPI; ++i)
                    dma16(tile + voff[i], &sA[buf][(wave * RPW + RPI * i) * kBK]);
            } else {
#pragma unroll
                for (int i = 0; i < RPW / RPI; ++i) {
                    float *dst = &sA[buf][(wave * RPW + RPI * i) * kBK];
                    if (dpiece[i] < d - slab * kBK) dma16(tile + voff[i], dst);
                    else *reinterpret_cast<f32x4 *>(dst + 4 * lane) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
        } else {
            const int32_t k = slab * kBK + 4 * lpiece;
#pragma unroll
            for (int i = 0; i < AP; ++i) ra[i] = ld4<false>(aptr[i], k, d);
        }
    };
    auto finish_slab = [&](int buf) {  // register path: registers -> LDS
        if constexpr (!VEC) {
#pragma unroll
            for (int i = 0; i < AP; ++i)
                *reinterpret_cast<f32x4 *>(&sA[buf][slab_at(lrow + i * RPP, lpiece)]) = ra[i];
        }
    };
    auto load_norms = [&](int par) {  // wave 0: the tile's 64 candidate norms
        if constexpr (metric_is_l2(M)) {
            if (wave == 0) {
                const int64_t c = (int64_t)row_base + lane;
                if constexpr (VEC) {
                    if (c < nc) dma4(a.cn + c, &sN[par][0]);
                    else sN[par][lane] = 0.0f;
                } else {
                    sN[par][lane] = c < nc ? a.cn[c] : 0.0f;
                }
            }
        }
    };
    auto wait_loads = [&]() {
        if constexpr (VEC) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    f32x16 acc[2] = {f32x16{}, f32x16{}};
    float best = __builtin_inff();
    int32_t bidx = -1;

    // Accumulator register r of a lane = candidate row 8*(r/4)+4h+(r%4) of
    // its 32-row block, query column l32; rows rise with r and tiles are
    // visited in ascending order.  A tile first reduces to its own best
    // (strict "<" over rising rows keeps the lowest row among equal values),
    // which replaces the running best only when strictly lower, so the
    // lowest index wins ties across tiles too.
    // The norms of this lane's 32 rows of the tile (L2 metrics), read from
    // LDS ahead of the epilogue so that their latency is hidden.
    f32x4 cnr[8];
    auto read_norms = [&](int par) {
        if constexpr (metric_is_l2(M)) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                cnr[j] = *reinterpret_cast<const f32x4 *>(&sN[par][(j >> 2) * 32 + 8 * (j & 3) + 4 * h]);
        }
    };
    auto epilogue = [&](int64_t qtile, int32_t ctile) {
        const int32_t base = ctile * kBC;  // < nc < 2^31
        if constexpr (M == kStoreDots) {
            // S[q][c] for this lane's query column; register quad r4 holds
            // rows 8 r4 + 4h .. + 3 of each 32-row block
            const int64_t q = qtile * kBQ + wave * 32 + l32;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int64_t c = (int64_t)base + cb * 32 + 8 * r4 + 4 * h;
                    if (q < nq && c < nc) {
                        float *dst = a.S + q * a.ld_s + c;
                        const f32x4 v = {acc[cb][4 * r4], acc[cb][4 * r4 + 1],
                                         acc[cb][4 * r4 + 2], acc[cb][4 * r4 + 3]};
                        if (c + 4 <= nc) {
                            *reinterpret_cast<f32x4 *>(dst) = v;
                        } else {
                            for (int e = 0; e < 4 && c + e < nc; ++e) dst[e] = v[e];
                        }
                    }
                }
                acc[cb] = f32x16{};
            }
            return;
        }
        // rows r + 4h < live exist (all of them unless this is C's last tile)
        const int32_t live = (int32_t)(nc - base < kBC ? nc - base : kBC) - 4 * h;
        float tb = __builtin_inff();
        int32_t tr = 0;
        auto scan = [&](auto check_rows) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 cn4 = {0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (metric_is_l2(M)) cn4 = cnr[4 * cb + r4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = cb * 32 + 8 * r4 + e;  // row in the tile, less 4h
                        const float v = rank_value<M>(acc[cb][4 * r4 + e], cn4[e]);
                        bool lt = v < tb;
                        if constexpr (decltype(check_rows)::value) lt = lt && r < live;
                        tb = lt ? v : tb;
                        tr = lt ? r : tr;
                    }
                }
                acc[cb] = f32x16{};
            }
        };
        if ((int64_t)base + kBC <= nc) {  // uniform: a full tile
            // Rank in place, take the tile's minimum with a min tree, and look
            // for its lowest row only where it beats the running best (late in
            // a sweep a tile rarely improves any of a wave's queries).  Same
            // result as the scan: the lowest row holding the minimum, taken
            // only when strictly below the best.
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    f32x4 cn4 = {0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (metric_is_l2(M)) cn4 = cnr[4 * cb + (i >> 2)];
                    acc[cb][i] = rank_value<M>(acc[cb][i], cn4[i & 3]);
                }
            }
            float m[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m[j] = __builtin_fminf(__builtin_fminf(acc[j >> 2][4 * (j & 3)], acc[j >> 2][4 * (j & 3) + 1]),
                                       __builtin_fminf(acc[j >> 2][4 * (j & 3) + 2], acc[j >> 2][4 * (j & 3) + 3]));
            const float tmin = __builtin_fminf(
                __builtin_fminf(__builtin_fminf(m[0], m[1]), __builtin_fminf(m[2], m[3])),
                __builtin_fminf(__builtin_fminf(m[4], m[5]), __builtin_fminf(m[6], m[7])));
            if (tmin < best) {
                // rows r = cb * 32 + 8 * r4 + e hold acc[cb][4 * r4 + e]: the
                // lowest row with the minimum, found from the highest down
#pragma unroll
                for (int cb = 1; cb >= 0; --cb) {
#pragma unroll
                    for (int i = 15; i >= 0; --i) {
                        const int r = cb * 32 + 8 * (i >> 2) + (i & 3);
                        tr = acc[cb][i] == tmin ? r : tr;
                    }
                }
                best = tmin;
                bidx = base + 4 * h + tr;
            }
            acc[0] = f32x16{};
            acc[1] = f32x16{};
        } else {
            scan(std::true_type{});
            if (tb < best) {
                best = tb;
                bidx = base + 4 * h + tr;
            }
        }
    };
    auto flush = [&](int64_t qtile) {
        if constexpr (M == kStoreDots) return;
        const float oe = __shfl_xor(best, 32);
        const int32_t oi = __shfl_xor(bidx, 32);
        if (oi >= 0 && (bidx < 0 || oe < best || (oe == best && oi < bidx))) {
            best = oe;
            bidx = oi;
        }
        const int64_t q = qtile * kBQ + wave * 32 + l32;
        if (h == 0 && bidx >= 0 && q < nq)
            atomicMin(reinterpret_cast<unsigned long long *>(a.keys + q),
                      (unsigned long long)pack_key(best, (uint32_t)bidx));
        best = __builtin_inff();
        bidx = -1;
    };

    // (query tile, candidate tile) of the item being computed; items are
    // visited candidate-tile major inside a query tile
    int64_t qt = it0 / nct;
    int32_t ct = (int32_t)(it0 - qt * nct);
    load_queries(qt);
    set_rows(ct);
    load_slab(0, 0);
    load_norms(0);
    finish_slab(0);
    wait_loads();
    __syncthreads();
    int buf = 0, par = 0;
    // With two or more slabs per item, the last chunk of each slab is held
    // in registers across the slab's barrier: after the barrier a wave first
    // reads the next slab's first operands, then issues the held MFMAs (and
    // at an item's end its epilogue), so the pipe has work while the barrier
    // resolves and the reads land.  The held epilogue reads norms slot par
    // after the barrier; that slot is reloaded two items later, behind at
    // least one more barrier when NSLAB >= 2.
    constexpr bool HOLD = NSLAB >= 2;
    auto mfma_chunk = [&](const f32x4 &x0, const f32x4 &x1, const f32x4 &qv) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0[e], qv[e], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1[e], qv[e], acc[1], 0, 0, 0);
        }
    };
    f32x4 a0 = *reinterpret_cast<const f32x4 *>(&sA[0][slab_at(l32, h)]);
    f32x4 a1 = *reinterpret_cast<const f32x4 *>(&sA[0][slab_at(32 + l32, h)]);
    for (int64_t item = it0; item < it1; ++item) {
        int64_t nqt = qt;
        int32_t nctile = ct + 1;
        if (nctile == nct) {
            nctile = 0;
            ++nqt;
        }
#pragma unroll
        for (int s = 0; s < NSLAB; ++s) {
            bool has_next = true;
            if (s + 1 < NSLAB) {
                load_slab(s + 1, buf ^ 1);
            } else {
                has_next = item + 1 < it1;
                if (has_next) {
                    set_rows(nctile);
                    load_slab(0, buf ^ 1);
                    load_norms(par ^ 1);
                }
            }
            // 8 chunks of 8 features; the operands of chunk cc+1 are read
            // from LDS before the MFMAs of chunk cc are issued (the
            // scheduling barriers keep the compiler from sinking the reads
            // behind the MFMAs, where their latency would be exposed)
            if constexpr (VS_QREG_PRIO) __builtin_amdgcn_s_setprio(1);
            const float *A = sA[buf];
            if constexpr (!HOLD) {
                a0 = *reinterpret_cast<const f32x4 *>(&A[slab_at(l32, h)]);
                a1 = *reinterpret_cast<const f32x4 *>(&A[slab_at(32 + l32, h)]);
            }
#pragma unroll
            for (int cc = 0; cc < kCPS; ++cc) {
                // this chunk's operands have landed (LDS reads complete in order)
                asm volatile("" ::"v"(a0), "v"(a1));
                if (HOLD && cc == kCPS - 1) continue;  // held: issued after the barrier
                f32x4 n0 = a0, n1 = a1;
                if (cc + 1 < kCPS) {
                    const int piece = 2 * (cc + 1) + h;
                    n0 = *reinterpret_cast<const f32x4 *>(&A[slab_at(l32, piece)]);
                    n1 = *reinterpret_cast<const f32x4 *>(&A[slab_at(32 + l32, piece)]);
                }
                __builtin_amdgcn_sched_barrier(0);
                mfma_chunk(a0, a1, qreg[s * kCPS + cc]);
                __builtin_amdgcn_sched_barrier(0);
                a0 = n0;
                a1 = n1;
            }
            if constexpr (VS_QREG_PRIO) __builtin_amdgcn_s_setprio(0);
            if (!HOLD && s == NSLAB - 1) {
                read_norms(par);
                epilogue(qt, ct);
            }
            if (has_next) finish_slab(buf ^ 1);
            wait_loads();
            __syncthreads();
            buf ^= 1;
            if constexpr (HOLD) {
                const f32x4 h0 = a0, h1 = a1;
                if (s + 1 < NSLAB || has_next) {
                    a0 = *reinterpret_cast<const f32x4 *>(&sA[buf][slab_at(l32, h)]);
                    a1 = *reinterpret_cast<const f32x4 *>(&sA[buf][slab_at(32 + l32, h)]);
                }
                if (s == NSLAB - 1) read_norms(par);
                __builtin_amdgcn_sched_barrier(0);
                mfma_chunk(h0, h1, qreg[s * kCPS + kCPS - 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (s == NSLAB - 1) epilogue(qt, ct);
            }
        }
        par ^= 1;
        if (item + 1 == it1 || nqt != qt) {
            flush(qt);
            if (item + 1 < it1) load_queries(nqt);
        }
        qt = nqt;
        ct = nctile;
    }
}

template <int M, int NSLAB, int QW>
static void dispatch_q(const DenseArgs &a, bool vec, dim3 grid, hipStream_t st) {
    if (vec)
        hipLaunchKernelGGL((k_bmu_qreg<M, true, NSLAB, QW>), grid, dim3(64 * QW), 0, st, a);
    else
        hipLaunchKernelGGL((k_bmu_qreg<M, false, NSLAB, QW>), grid, dim3(64 * QW), 0, st, a);
}

template <int M, int QW>
static void dispatch_slabs(const DenseArgs &a, bool vec, dim3 grid, hipStream_t st) {
    const int nslab = (a.d + kBK - 1) / kBK;
    if constexpr (kMaxSlabs == 4) {
        switch (nslab) {
        case 1: dispatch_q<M, 1, QW>(a, vec, grid, st); break;
        case 2: dispatch_q<M, 2, QW>(a, vec, grid, st); break;
        case 3: dispatch_q<M, 3, QW>(a, vec, grid, st); break;
        default: dispatch_q<M, 4, QW>(a, vec, grid, st); break;
        }
    } else {
        if (nslab == 1) dispatch_q<M, 1, QW>(a, vec, grid, st);
        else dispatch_q<M, 2, QW>(a, vec, grid, st);
    }
}

// Items of (32 QW queries) x 64 candidates; at most 8 waves per CU of work
// split into contiguous runs, one per workgroup.
static DenseArgs qreg_split(const DenseArgs &a0, int qw, int n_cu) {
    DenseArgs a = a0;
    const int64_t nqt = (a.nq + 32 * qw - 1) / (32 * qw);
    a.n_ctiles = (a.nc + kBC - 1) / kBC;
    a.n_items = nqt * a.n_ctiles;
    const int64_t cap = (int64_t)(n_cu > 0 ? n_cu : 256) * (kQW / qw);
    a.grid = (int32_t)(a.n_items < cap ? a.n_items : cap);
    return a;
}

bool qreg_supports(int32_t d) { return d >= 1 && d <= 256; }

hipError_t launch_dense_qreg(const DenseArgs &a0, int metric, hipStream_t st, int n_cu) {
    // A search with fewer 8-wave items than CUs (e.g. 256 queries x 1,024
    // candidates: 16 items) runs 4-wave workgroups instead: twice the items,
    // one wave per SIMD, so each item's MFMA chain takes half as long.  The
    // per-pair arithmetic is the same, so are the results, bit for bit.
    DenseArgs a = qreg_split(a0, kQW, n_cu);
    const bool small = a.n_items < (int64_t)(n_cu > 0 ? n_cu : 256);
    if (small) a = qreg_split(a0, kQW / 2, n_cu);
    const bool vec = (a.d % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.C) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(a.Q) & 15) == 0);
    const dim3 grid((unsigned)a.grid);
    timing_before(st, "k_bmu_qreg");
    if (small) {
        switch (metric) {
        case L2SQ_MIN: dispatch_slabs<L2SQ_MIN, kQW / 2>(a, vec, grid, st); break;
        case L2SQ_MAX: dispatch_slabs<L2SQ_MAX, kQW / 2>(a, vec, grid, st); break;
        case COS_MAX: dispatch_slabs<COS_MAX, kQW / 2>(a, vec, grid, st); break;
        default: dispatch_slabs<COS_MIN, kQW / 2>(a, vec, grid, st); break;
        }
    } else {
        switch (metric) {
        case L2SQ_MIN: dispatch_slabs<L2SQ_MIN, kQW>(a, vec, grid, st); break;
        case L2SQ_MAX: dispatch_slabs<L2SQ_MAX, kQW>(a, vec, grid, st); break;
        case COS_MAX: dispatch_slabs<COS_MAX, kQW>(a, vec, grid, st); break;
        default: dispatch_slabs<COS_MIN, kQW>(a, vec, grid, st); break;
        }
    }
    const hipError_t err = hipGetLastError();
    timing_after(st);
    return err;
}

// Every dot product Q[q] . C[c] (d <= 256) written to S[q * ld_s + c]
// (ld_s % 4 == 0, S 16-byte aligned) by the arithmetic of the scan above, so
// each value equals, bit for bit, the dot product that scan ranks.
hipError_t launch_dense_qreg_store(const DenseArgs &a0, hipStream_t st, int n_cu) {
    const DenseArgs a = qreg_split(a0, kQW, n_cu);
    const bool vec = (a.d % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.C) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(a.Q) & 15) == 0);
    timing_before(st, "k_bmu_qreg<store>");
    dispatch_slabs<kStoreDots, kQW>(a, vec, dim3((unsigned)a.grid), st);
    const hipError_t err = hipGetLastError();
    timing_after(st);
    return err;
}

}  // namespace vs
