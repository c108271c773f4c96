// bmu_q16.hip -- dense scan for d <= 768 with 16 queries per wave held in
// registers; also the gathered, masked diversity step.
//
// Same result as bmu_mfma.hip and bmu_qreg.hip (fp32 MFMA dot products, fused
// ranking, lowest-index arg-reduction, packed-key merge).  The 32x32x2 MFMA
// of bmu_qreg.hip costs d/2 registers per lane for its 32 query columns,
// which caps it at d = 256; v_mfma_f32_16x16x4f32 has 16 query columns and
// four K rows, so a wave keeps its 16 queries in d/4 registers per lane and
// d = 768 (192 registers) still leaves room for two waves per SIMD.
// Sources, by page title and section:
//  - "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
//    "Intended Behavior": the diversity step's masked arg-extreme, and the
//    cache-tile idea: every workgroup on one XCD walks the same candidate
//    range, small enough to stay in that XCD's L2, with the running best
//    carried across tiles;
//  - "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof ..."
//    (summary), section 3: the argmin fused into the product;
//  - "Tiling en memoria compartida: el factor 16", "Tiling en registros":
//    the reused operand (here the query block) lives in registers.
//
// Layout: workgroup = 8 waves = 128 queries (16 per wave); work item =
// (query tile of 128, candidate tile of 32 = two 16-row MFMA blocks).
// Candidate slabs of kBK features go to LDS with global_load_lds (16 bytes
// per lane) into three buffers, each slab's loads issued two slabs before
// it is used; the item's candidate norms and the tile's mask words travel
// the same way.  A slab row is kBK/4 pieces of 16 bytes stored at slot
// (piece XOR row%16), conflict-free for both the 1 KiB loads and the 16-row
// operand reads.  MFMA operand map for chunk c (16 features):
// lane l = (g = l/16, i = l%16) holds features 16c+4g .. 16c+4g+3 of
// candidate row i (one 16-byte LDS read) and of query column i (a register
// quad); component t of both feeds MFMA t, so four MFMAs cover the chunk and
// every pair's dot product runs over one fixed feature order.
//
// Work split: when there are fewer queries than candidates the candidate
// tiles are cut into 8 ranges, range x handled by the workgroups that the
// hardware places on XCD x (blockIdx % 8), each of those taking a contiguous
// run of (query tile, candidate tile) items of that range; otherwise all
// items are split contiguously, query-tile major, as in bmu_qreg.hip.
#include "vs_internal.h"

namespace vs {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

#ifndef VS_Q16_BK
#define VS_Q16_BK 64
#endif
#ifndef VS_Q16_WAVES
#define VS_Q16_WAVES 8
#endif

constexpr int kW = VS_Q16_WAVES;  // waves per workgroup (4 or 8: 2 waves per SIMD either way)
constexpr int kBQ = 16 * kW;      // queries per tile
constexpr int kBC = 32;           // candidates per tile (= one mask word)
constexpr int kBK = VS_Q16_BK;    // features per LDS slab
constexpr int kCPS = kBK / 16;    // 16-feature chunks per slab
constexpr int kPPR = kBK / 4;     // 16-byte pieces per slab row
constexpr int kRPI = 64 / kPPR;   // slab rows per DMA instruction (1 KiB)
constexpr int kDPW = kBC / kRPI / kW;  // DMA instructions per wave per slab
constexpr int kMaxD = 768;
constexpr int kTPQ = kBQ / kBC;   // candidate tiles per query tile's rows
constexpr int32_t kSplitTriangle = 2;  // DenseArgs.split: the symmetric Gram walk
constexpr int kMaxSlabs = kMaxD / kBK;
static_assert(kBK == 64 || kBK == 128, "slab width");
static_assert(kW == 4 || kW == 8, "waves per workgroup");
static_assert(kDPW >= 1 && kDPW * kRPI * kW == kBC, "slab loader shape");

__device__ __forceinline__ int slab_at(int row, int piece) {
    return row * kBK + ((piece ^ (row & 15)) << 2);
}

}  // namespace

// MODE: kSearch (arg-reduce over Q's rows), kDiversity (queries gathered
// as C[pick], masked), kStore (write every dot product to S instead),
// kRef (Q's rows, masked: a diversity step against explicit references).
enum : int { kSearch = 0, kDiversity = 1, kStore = 2, kRef = 3 };

template <int M, int MODE, int NSLAB>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(2)))
void k_bmu_q16(const DenseArgs a) {
    constexpr int NCH = NSLAB * kCPS;
    constexpr bool GATHER = MODE == kDiversity;
    constexpr bool MASKED = MODE == kDiversity || MODE == kRef;
    constexpr bool STORE = MODE == kStore;

    __shared__ __attribute__((aligned(16))) float sA[3][kBC * kBK];
    __shared__ __attribute__((aligned(16))) float sN[3][kBC];  // candidate norms, by item mod 3
    __shared__ uint32_t sM[3][MASKED ? kBQ : 1];  // mask words of the tile's queries, by item mod 3

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, i16 = lane & 15;
    const int wave = tid >> 6;

    const int64_t nq = a.nq, nc = a.nc, nct = a.n_ctiles;
    const int32_t d = a.d;

    // ---- this workgroup's items: a run of n_my items over a range of nctx
    // candidate tiles starting at ct_lo, visited query-tile major: item
    // (qt, ct) is followed by (qt, ct + 1), or (qt + 1, ct_lo) at the range end.
    // Triangle walk (a.split == kSplitTriangle, the symmetric Gram build):
    // query tile q covers the candidate tiles from kTPQ q on, the first kTPQ
    // of them holding the tile's own rows.
    const bool tri = STORE && a.split == kSplitTriangle;
    int32_t ct_lo = 0, nctx = (int32_t)nct, qt, ctl, n_my;
    auto row_lo = [&](int32_t q) { return tri ? kTPQ * q : ct_lo; };
    auto row_n = [&](int32_t q) { return tri ? (int32_t)nct - kTPQ * q : nctx; };
    {
        const int G = a.grid;
        int64_t it0, it1;
        if (a.split == 8) {
            const int x = (int)(blockIdx.x & 7), gl = (int)(blockIdx.x >> 3), GX = G >> 3;
            ct_lo = (int32_t)((int64_t)x * nct / 8);
            nctx = (int32_t)((int64_t)(x + 1) * nct / 8) - ct_lo;
            const int64_t nx = (a.n_items / nct) * nctx;
            it0 = (int64_t)gl * nx / GX;
            it1 = (int64_t)(gl + 1) * nx / GX;
        } else {
            int gg = blockIdx.x;
            if ((G & 7) == 0) gg = (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
            it0 = (int64_t)gg * a.n_items / G;
            it1 = (int64_t)(gg + 1) * a.n_items / G;
        }
        if (it0 >= it1) return;  // whole workgroup: no barrier is skipped by part of it
        if (tri) {
            int64_t left = it0;
            qt = 0;
            while (left >= row_n(qt)) left -= row_n(qt++);
            ctl = (int32_t)left;
        } else {
            qt = (int32_t)(it0 / nctx);
            ctl = (int32_t)(it0 - (int64_t)qt * nctx);
        }
        n_my = (int32_t)(it1 - it0);
    }

    // ---- queries: 16 per wave, chunk c of query column i16 in qreg[c].
    // Loads always read inside the buffer (a missing query reads row 0, a
    // chunk past d reads the row's last 4 features) and are zeroed after.
    f32x4 qreg[NCH];
    bool q_ok = false;  // this lane's query exists (and, gathering, has a valid row)
    auto load_queries = [&](int32_t qtile) {
        const int64_t q = (int64_t)qtile * kBQ + wave * 16 + i16;
        int64_t row = 0;
        q_ok = q < nq;
        if constexpr (GATHER) {
            const int64_t pk = q_ok ? (int64_t)a.pick[q] : -1;
            q_ok = pk >= 0 && pk < nc;
            row = q_ok ? pk : 0;
        } else {
            row = q_ok ? q : 0;
        }
        const float *p = (GATHER ? a.C : a.Q) + row * d;
        // d and 4g pass through empty asm so that the per-chunk bounds below
        // are evaluated here, not hoisted out of the item loop (48 hoisted
        // compares would cost the registers the query block needs)
        int32_t dl = d, g4 = 4 * g;
        asm volatile("" : "+s"(dl));
        asm volatile("" : "+v"(g4));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int32_t k = 16 * c + g4;
            qreg[c] = (q_ok && k < dl) ? *reinterpret_cast<const f32x4 *>(p + k)
                                       : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        // wait for the block here: otherwise the wait lands at the first
        // MFMA of the item and also holds the slab loads issued just before
#pragma unroll
        for (int c = 0; c < NCH; ++c) asm volatile("" ::"v"(qreg[c]));
    };

    // ---- candidate slab loader (LDS-DMA).  Wave w fills rows
    // [kDPW kRPI w, kDPW kRPI (w + 1)); one instruction covers kRPI rows x
    // kPPR slots, lane l -> row + l / kPPR, slot l % kPPR, which holds piece
    // slot ^ (row % 16) of that row.  Rows past nc re-read row nc - 1 (their
    // results are discarded); features >= d are written as zeros with
    // ds_write, so a padded feature never meets a non-zero query value.
    const float *src[kDPW];  // this lane's piece of slab 0 of the item being loaded
    int32_t piece_k[kDPW];   // its feature offset inside a slab
    int64_t row_base = 0;    // first candidate of the item being loaded
    auto set_rows = [&](int32_t ct) {
        row_base = (int64_t)ct * kBC;
#pragma unroll
        for (int u = 0; u < kDPW; ++u) {
            const int row = (wave * kDPW + u) * kRPI + lane / kPPR;
            const int piece = (lane % kPPR) ^ (row & 15);
            int64_t c = row_base + row;
            c = c < nc ? c : nc - 1;
            piece_k[u] = 4 * piece;
            src[u] = a.C + c * d + 4 * piece;
        }
    };
    // Every slab holds at least one feature below d (the kernel is launched
    // with NSLAB = ceil(d / kBK)), so each wave issues exactly kDPW loads per
    // slab, each with at least the lanes of piece 0 active: the slab
    // pipeline's waits count on that.
    auto load_slab = [&](int slab, int buf) {
        int32_t dl = d;  // opaque, as in load_queries
        asm volatile("" : "+s"(dl));
        const bool full = (slab + 1) * kBK <= dl;  // uniform: no feature past d
#pragma unroll
        for (int u = 0; u < kDPW; ++u) {
            float *dst = &sA[buf][(wave * kDPW + u) * kRPI * kBK];
            if (full || piece_k[u] < dl - slab * kBK) dma16(src[u] + slab * kBK, dst);
            else *reinterpret_cast<f32x4 *>(dst + 4 * lane) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    auto load_norms = [&](int par) {  // wave 0: the item's 32 candidate norms
        if constexpr (metric_is_l2(M)) {
            if (wave == 0 && lane < kBC) {
                const int64_t c = row_base + lane;
                dma4(a.cn + (c < nc ? c : nc - 1), &sN[par][0]);
            }
        }
    };
    // waves 0 and 1: the mask words (query tile qtile, candidate tile ct) of
    // the tile's 128 queries.  Every lane loads (a query past nq reads query
    // nq - 1's word, which nothing uses: such a query's result is never
    // published), so each of these waves issues exactly one load.
    auto load_mask = [&](int32_t qtile, int32_t ct, int par) {
        if constexpr (MASKED) {
            if (wave < kBQ / 64) {
                int64_t q = (int64_t)qtile * kBQ + wave * 64 + lane;
                q = q < nq ? q : nq - 1;
                dma4(reinterpret_cast<const float *>(a.mask + q * a.mask_words + ct),
                     reinterpret_cast<float *>(&sM[par][wave * 64]));
            }
        }
    };

    f32x4 acc[2] = {f32x4{}, f32x4{}};
    float best = __builtin_inff();
    int32_t bidx = -1;
    uint32_t mw = 0;  // mask word of (this lane's query, current candidate tile)

    // Accumulator register r of block b = candidate row 16b+4g+r of the tile,
    // query column i16; rows rise with (b, r) and tiles are visited in
    // ascending order, so strict "<" keeps the lowest index among ties.
    auto epilogue = [&](int32_t ct, int par) {
        const int32_t base = ct * kBC;  // < nc < 2^31
        if constexpr (STORE) {
            // S[q][c] for this lane's query column and its rows 16b+4g..+3
            // (16-byte stores: ld_s % 4 == 0 and S 16-byte aligned)
            const int64_t q = (int64_t)qt * kBQ + wave * 16 + i16;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int64_t c = (int64_t)base + 16 * b + 4 * g;
                if (q < nq && c < nc) {
                    float *dst = a.S + q * a.ld_s + c;
                    if (c + 4 <= nc) {
                        *reinterpret_cast<f32x4 *>(dst) = acc[b];
                    } else {
                        for (int r = 0; r < 4 && c + r < nc; ++r) dst[r] = acc[b][r];
                    }
                    // triangle walk: a tile right of the query tile's own rows
                    // also writes its transpose, S[c][q] (the pairs below the
                    // diagonal blocks are computed nowhere else); S[c][q] is
                    // the same MFMA dot product with the operands' roles
                    // exchanged, and the products and their order over the
                    // features are the same, so it is bit-identical
                    if (tri && ct >= kTPQ * (qt + 1)) {
                        for (int r = 0; r < 4 && c + r < nc; ++r)
                            a.S[(c + r) * a.ld_s + q] = acc[b][r];
                    }
                }
                acc[b] = f32x4{};
            }
            return;
        }
        // rows 16b + r of this lane group are live while 16b + r < lim;
        // mask bits of the group shifted down to bit 0 (constant shifts below)
        const int64_t left = nc - base - 4 * g;
        const int32_t lim = left < 64 ? (int32_t)left : 64;
        uint32_t mg = 0;
        if constexpr (MASKED) mg = mw >> (4 * g);
        if (nc - base >= kBC) {  // uniform: a full tile
            // Rank in place (masked rows rank as +inf), take the minimum with
            // a min tree, and look for its lowest row only where it beats the
            // running best: the same (value, lowest row) as the scan below.
            float v[8];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x4 cn4 = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (metric_is_l2(M))
                    cn4 = *reinterpret_cast<const f32x4 *>(&sN[par][16 * b + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = rank_value<M>(acc[b][r], cn4[r]);
                    if constexpr (MASKED) x = ((mg >> (16 * b + r)) & 1u) ? __builtin_inff() : x;
                    v[4 * b + r] = x;
                }
                acc[b] = f32x4{};
            }
            const float tmin = __builtin_fminf(
                __builtin_fminf(__builtin_fminf(v[0], v[1]), __builtin_fminf(v[2], v[3])),
                __builtin_fminf(__builtin_fminf(v[4], v[5]), __builtin_fminf(v[6], v[7])));
            if (tmin < best) {
                int32_t tr = 0;
#pragma unroll
                for (int j = 7; j >= 0; --j) tr = v[j] == tmin ? 16 * (j >> 2) + (j & 3) : tr;
                best = tmin;
                bidx = base + 4 * g + tr;
            }
            return;
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            f32x4 cn4 = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (metric_is_l2(M))
                cn4 = *reinterpret_cast<const f32x4 *>(&sN[par][16 * b + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = rank_value<M>(acc[b][r], cn4[r]);
                bool live = 16 * b + r < lim;
                if constexpr (MASKED) live = live && !((mg >> (16 * b + r)) & 1u);
                if (live && v < best) {
                    best = v;
                    bidx = base + 4 * g + 16 * b + r;
                }
            }
            acc[b] = f32x4{};
        }
    };
    // Merge the four lane groups (same query, interleaved candidate rows)
    // and publish each query's best with one packed atomicMin.
    auto flush = [&](int32_t qtile) {
        if constexpr (STORE) return;
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float oe = __shfl_xor(best, off);
            const int32_t oi = __shfl_xor(bidx, off);
            if (oi >= 0 && (bidx < 0 || oe < best || (oe == best && oi < bidx))) {
                best = oe;
                bidx = oi;
            }
        }
        const int64_t q = (int64_t)qtile * kBQ + wave * 16 + i16;
        if (g == 0 && bidx >= 0 && q_ok)
            atomicMin(reinterpret_cast<unsigned long long *>(a.keys + q),
                      (unsigned long long)pack_key(best, (uint32_t)bidx));
        best = __builtin_inff();
        bidx = -1;
    };

    // ---- slab pipeline.  The run is a sequence of n_my * NSLAB slabs; slab
    // f lives in LDS buffer f % 3 and its loads are issued while slab f - 2
    // is computed, so a load has two slabs of MFMA work to land.
    // Issues slab ts of item n + io (io items after the current one) into
    // buffer bufi, with the item's norms and mask words along with its first
    // slab; returns the number of vector-memory instructions this wave issued.
    auto issue = [&](int32_t n, int io, int ts, int bufi) -> int {
        if (n + io >= n_my) return 0;
        int ops = kDPW;
        if (ts == 0) {
            int32_t c = ctl + io, q = qt;
            while (c >= row_n(q)) {
                c -= row_n(q);
                ++q;
            }
            set_rows(row_lo(q) + c);
            if constexpr (metric_is_l2(M)) {
                load_norms((n + io) % 3);
                if (wave == 0) ++ops;
            }
            if constexpr (MASKED) {
                load_mask(q, row_lo(q) + c, (n + io) % 3);
                if (wave < kBQ / 64) ++ops;
            }
        }
        load_slab(ts, bufi);
        return ops;
    };

    load_queries(qt);
    issue(0, 0, 0, 0);
    wait_vmcnt(issue(0, 1 / NSLAB, 1 % NSLAB, 1));
    lds_barrier();
    int buf = 0;
    for (int32_t n = 0; n < n_my; ++n) {
        const int32_t ct = row_lo(qt) + ctl;
        // the item that follows this one
        int32_t nqt = qt, nctl = ctl + 1;
        if (nctl == row_n(qt)) {
            nctl = 0;
            ++nqt;
        }
        const bool has_next_item = n + 1 < n_my;
#pragma unroll
        for (int s = 0; s < NSLAB; ++s) {
            const int b2 = buf >= 1 ? buf - 1 : 2;  // (buf + 2) % 3
            const int issued = issue(n, (s + 2) / NSLAB, (s + 2) % NSLAB, b2);
            // kCPS chunks of 16 features; the operands of chunk cc+1 are
            // read from LDS before the MFMAs of chunk cc are issued (the
            // scheduling barriers keep the compiler from sinking the reads)
            const float *A = sA[buf];
            f32x4 a0 = *reinterpret_cast<const f32x4 *>(&A[slab_at(i16, g)]);
            f32x4 a1 = *reinterpret_cast<const f32x4 *>(&A[slab_at(16 + i16, g)]);
#pragma unroll
            for (int cc = 0; cc < kCPS; ++cc) {
                // wait for this chunk's operands here, before the next reads
                // are issued (LDS reads complete in order)
                asm volatile("" ::"v"(a0), "v"(a1));
                f32x4 n0 = a0, n1 = a1;
                if (cc + 1 < kCPS) {
                    const int piece = 4 * (cc + 1) + g;
                    n0 = *reinterpret_cast<const f32x4 *>(&A[slab_at(i16, piece)]);
                    n1 = *reinterpret_cast<const f32x4 *>(&A[slab_at(16 + i16, piece)]);
                }
                __builtin_amdgcn_sched_barrier(0);
                const f32x4 qv = qreg[s * kCPS + cc];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[t], qv[t], acc[0], 0, 0, 0);
                    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[t], qv[t], acc[1], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                a0 = n0;
                a1 = n1;
            }
            if (s == NSLAB - 1) {
                if constexpr (MASKED) mw = sM[n % 3][wave * 16 + i16];
                epilogue(ct, n % 3);
            }
            // slab f + 1 must have landed in every wave before anyone reads
            // it; slab f + 2 (issued above) may stay in flight.  The barrier
            // also frees buffer f % 3 for the loads issued at the next slab.
            wait_vmcnt(issued);
            lds_barrier();
            buf = buf == 2 ? 0 : buf + 1;
        }
        if (!has_next_item || nqt != qt) {
            flush(qt);
            if (has_next_item) load_queries(nqt);
        }
        qt = nqt;
        ctl = nctl;
    }
}

template <int M, int MODE>
static void dispatch_slabs(const DenseArgs &a, dim3 grid, hipStream_t st) {
    const int nslab = (a.d + kBK - 1) / kBK;
    static_assert(kMaxSlabs == 6 || kMaxSlabs == 12, "slab count table");
    if constexpr (kMaxSlabs == 6) {
        switch (nslab) {
        case 1: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 1>), grid, dim3(64 * kW), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 2>), grid, dim3(64 * kW), 0, st, a); break;
        case 3: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 3>), grid, dim3(64 * kW), 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 4>), grid, dim3(64 * kW), 0, st, a); break;
        case 5: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 5>), grid, dim3(64 * kW), 0, st, a); break;
        default: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 6>), grid, dim3(64 * kW), 0, st, a); break;
        }
    } else {
        // 64-feature slabs, the exact count: no slab lies wholly past d (the
        // slab pipeline counts kDPW loads per slab)
        switch (nslab) {
        case 1: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 1>), grid, dim3(64 * kW), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 2>), grid, dim3(64 * kW), 0, st, a); break;
        case 3: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 3>), grid, dim3(64 * kW), 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 4>), grid, dim3(64 * kW), 0, st, a); break;
        case 5: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 5>), grid, dim3(64 * kW), 0, st, a); break;
        case 6: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 6>), grid, dim3(64 * kW), 0, st, a); break;
        case 7: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 7>), grid, dim3(64 * kW), 0, st, a); break;
        case 8: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 8>), grid, dim3(64 * kW), 0, st, a); break;
        case 9: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 9>), grid, dim3(64 * kW), 0, st, a); break;
        case 10: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 10>), grid, dim3(64 * kW), 0, st, a); break;
        case 11: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 11>), grid, dim3(64 * kW), 0, st, a); break;
        default: hipLaunchKernelGGL((k_bmu_q16<M, MODE, 12>), grid, dim3(64 * kW), 0, st, a); break;
        }
    }
}

bool q16_supports(int32_t d, const float *C, const float *Q) {
    const bool al = (reinterpret_cast<uintptr_t>(C) & 15) == 0 &&
                    (Q == nullptr || (reinterpret_cast<uintptr_t>(Q) & 15) == 0);
    return d >= 1 && d <= kMaxD && d % 4 == 0 && al;
}

hipError_t launch_dense_q16(const DenseArgs &a0, int metric, int qmode, hipStream_t st,
                            int n_cu) {
    const bool gather = qmode == kQGatherMasked;
    DenseArgs a = a0;
    const int64_t nqt = (a.nq + kBQ - 1) / kBQ;
    a.n_ctiles = (a.nc + kBC - 1) / kBC;
    a.n_items = nqt * a.n_ctiles;
    // 8 waves per CU: one 8-wave or two 4-wave workgroups
    const int64_t cap = (int64_t)(n_cu > 0 ? n_cu : 256) * (8 / kW);
    a.grid = (int32_t)(a.n_items < cap ? a.n_items : cap);
    // Candidate ranges per XCD pay when the queries are the smaller operand:
    // each XCD then reads its slice of the candidates once and the (smaller)
    // query set eight times, instead of the whole candidate set eight times.
    a.split = (a.grid % 8 == 0 && a.n_ctiles >= 8 && a.nq < a.nc) ? 8 : 1;
    const dim3 grid((unsigned)a.grid);
    timing_before(st, gather ? "k_bmu_q16<COS_MIN,gather>"
                             : (qmode == kQRowsMasked ? "k_bmu_q16<COS_MIN,ref>" : "k_bmu_q16"));
    if (gather) {
        dispatch_slabs<COS_MIN, kDiversity>(a, grid, st);
    } else if (qmode == kQRowsMasked) {
        dispatch_slabs<COS_MIN, kRef>(a, grid, st);
    } else {
        switch (metric) {
        case L2SQ_MIN: dispatch_slabs<L2SQ_MIN, kSearch>(a, grid, st); break;
        case L2SQ_MAX: dispatch_slabs<L2SQ_MAX, kSearch>(a, grid, st); break;
        case COS_MAX: dispatch_slabs<COS_MAX, kSearch>(a, grid, st); break;
        default: dispatch_slabs<COS_MIN, kSearch>(a, grid, st); break;
        }
    }
    const hipError_t err = hipGetLastError();
    timing_after(st);
    return err;
}

// Every dot product Q[q] . C[c] written to S[q * ld_s + c] (ld_s >= nc,
// ld_s % 4 == 0, S 16-byte aligned) by the same MFMA arithmetic, in the
// same per-pair order, as the scans above: each stored value equals,
// bit for bit, the dot product those scans rank.
hipError_t launch_dense_q16_store(const DenseArgs &a0, hipStream_t st, int n_cu,
                                  bool symmetric) {
    DenseArgs a = a0;
    const int64_t nqt = (a.nq + kBQ - 1) / kBQ;
    a.n_ctiles = (a.nc + kBC - 1) / kBC;
    a.n_items = nqt * a.n_ctiles;
    if (symmetric) {
        // query tile q takes candidate tiles kTPQ q .. n_ctiles - 1 (at least
        // one: 128 (nqt - 1) < n, so kTPQ (nqt - 1) < n_ctiles)
        a.n_items -= (int64_t)kTPQ * nqt * (nqt - 1) / 2;
    }
    const int64_t cap = (int64_t)(n_cu > 0 ? n_cu : 256) * (8 / kW);
    a.grid = (int32_t)(a.n_items < cap ? a.n_items : cap);
    a.split = (a.grid % 8 == 0 && a.n_ctiles >= 8 && a.nq < a.nc) ? 8 : 1;
    if (symmetric) a.split = kSplitTriangle;
    const dim3 grid((unsigned)a.grid);
    dispatch_slabs<COS_MIN, kStore>(a, grid, st);  // not a dominant kernel: no timing events
    return hipGetLastError();
}

}  // namespace vs
