// Code scan and top-R: for each query, the integer sum of its int8 table
// entries at every scanned row's 4-bit codes, and the R best rows by
// (sum desc, original id asc).
//
// Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
// Product Search", section "Three stages of a search" (a row's approximate
// score is the sum of its table entries), "Using the library"
// (pre_reorder_num_neighbors candidates go on to reorder) and "Worked example:
// cost of one query" (the scan dominates; batching queries improves reuse of
// leaf data).
//
// gfx950 design
//  * The sum over blocks of T8[q][b][code(i,b)] is the contraction
//      sums[i][q] = sum_{b,c} onehot[i][(b,c)] * T8[q][(b,c)]
//    with K = 16*B.  The scan runs it on the int8 matrix cores
//    (v_mfma_i32_16x16x64_i8: exact int32 accumulation): the A operand is the
//    one-hot expansion of 16 rows' codes, read from a 16-entry LDS table (one
//    block per lane per k-step, 16 bytes with a single 1), the B operand is 16
//    queries' table rows, resident in LDS.  Each lane of a 16-lane group feeds
//    its own block, and A and B use the same (lane group, byte) -> (block,
//    center) map, so the hardware's internal k order does not matter.
//  * A workgroup (8 waves) owns up to 64 queries and a run of rows (a leaf, or a
//    chunk of the database); each wave takes 64 rows x 64 queries per step
//    (4 x 4 MFMA tiles), so every code byte fetched from HBM is used by all the
//    workgroup's queries and every one-hot operand by 4 query tiles.  The
//    tables stay in LDS (64 blocks x 64 queries = 64 KB per pass; more blocks
//    are processed in 64-block chunks).  With one chunk, the waves claim 64-row
//    slabs from an LDS counter and need no barrier until the item ends; each
//    wave streams its slab's codes into its own LDS buffer with 16-byte loads
//    issued a step ahead.
//  * Top-R without materialising sums: every query has a monotone threshold tau
//    (a lower bound on its R-th best sum).  A warm-up kernel sets it from the
//    query's first rows; a step's sums are tested against it per query tile,
//    then per row tile, then per element, and rows at or above it are logged
//    per wave in LDS and appended to the query's candidate list (one slot
//    reservation per query and flush); a histogram of the appended sums lets
//    each workgroup raise tau after every item (count(sum >= edge) >= R makes
//    the edge a valid bound).  A final kernel selects each query's exact top-R
//    from its list; a query whose list overflows is recomputed by a slow exact
//    fallback, so the result never depends on timing.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

#include <limits.h>
#include <type_traits>

namespace ah {

constexpr int kScanWaves = 8;
constexpr int kScanThreads = kScanWaves * kWave;  // 512
constexpr int kTilePts = 64 * kScanWaves;         // rows per tile
constexpr int kQG = 64;                           // queries per item
constexpr int kKC = 16;                           // k-steps (x4 blocks) of a resident table (B <= 64)
constexpr int kKCS = 8;                           // k-steps of one staged chunk (B > 64): half of lut_s
// The one-hot contraction runs on the sparse int8 matrix instruction (2:4
// structured sparsity, twice the k of the dense one per instruction); false
// selects the dense instruction with one-hot operands from an LDS table.
constexpr int kCodeStride = 9;                    // LDS row stride (dwords) for a chunk's 8 code dwords
constexpr int kNB = 1024;                         // histogram bins per query
constexpr int kLB = 64;                           // an item's LDS histogram bins per query
constexpr int kLogCap = 384;                      // logged hits per wave (one row tile of a query tile: 256 max)
constexpr int kItemPts = 16384;                   // rows per item (row offsets fit the log's 16 bits)
constexpr int kFbSlots = 4;                       // fallback workgroups
constexpr int kSelThreads = 256;
constexpr int kSelLds = 4096;                     // keys staged in LDS by the final select
constexpr int kStreamMaxQ = 4;                    // batches scanned by the streaming kernel (VALU lookups)
constexpr int kSpreadWG = 256;                    // spread warm-up: most workgroups (partial histograms) per query
constexpr int kSpreadThreads = 512;
constexpr int32_t kSpreadRows = 131072;           // spread warm-up: most rows per query
constexpr int64_t kSpreadLookups = 1LL << 25;     // spread warm-up: rows x blocks per query, at most

struct ScanLayout {
    size_t tau, cnt, hmax, hist, cand, ctrl, ovf, dfr, fb, lcnt, lqoff, lcur, qlist, qbias, itemoff, wpart, total;
    int64_t cap;
};

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

static ScanLayout scan_layout(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R) {
    (void)B;
    ScanLayout s{};
    int64_t cap = 16 * (int64_t)R;
    if (cap < 32768) cap = 32768;
    // a few queries scanned by every workgroup at once log many rows before
    // their thresholds meet: give them long lists (4M entries between them)
    if (nq > 0 && nq <= 4 && cap < (int64_t)(1 << 22) / nq) cap = (int64_t)(1 << 22) / nq;
    if (cap > n) cap = n > 0 ? n : 1;
    s.cap = cap;
    size_t o = 0;
    s.tau = o;     o = align_up(o + (size_t)nq * 4);
    s.cnt = o;     o = align_up(o + (size_t)nq * 4);
    s.hmax = o;    o = align_up(o + (size_t)nq * 4);
    s.hist = o;    o = align_up(o + (size_t)nq * kNB * 4);
    s.cand = o;    o = align_up(o + (size_t)nq * (size_t)cap * 8);
    s.ctrl = o;    o = align_up(o + 64);
    s.ovf = o;     o = align_up(o + (size_t)nq * 4);
    s.dfr = o;     o = align_up(o + (size_t)nq * 4);
    s.fb = o;      o = align_up(o + (size_t)kFbSlots * (size_t)(n > 0 ? n : 1) * 8);
    const bool part = L > 0 && nl > 0;
    s.lcnt = o;    o = align_up(o + (part ? (size_t)L * 4 : 0));
    s.lqoff = o;   o = align_up(o + (part ? (size_t)(L + 1) * 4 : 0));
    s.lcur = o;    o = align_up(o + (part ? (size_t)L * 4 : 0));
    s.qlist = o;   o = align_up(o + (part ? (size_t)nq * nl * 4 : 0));
    s.qbias = o;   o = align_up(o + (part ? (size_t)nq * nl * 4 : 0));
    s.itemoff = o; o = align_up(o + (part ? (size_t)(L + 1) * 8 : 0));
    // partial histograms of the spread warm-up (full scans by a few queries)
    s.wpart = o;   o = align_up(o + (!part && nq <= kStreamMaxQ ? (size_t)nq * kSpreadWG * kNB * 4 : 0));
    s.total = o;
    return s;
}

size_t scan_workspace_bytes(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R) {
    return scan_layout(nq, B, n, L, nl, R).total;
}

void scan_counter_offsets(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R, size_t* appended,
                          size_t* control) {
    const ScanLayout s = scan_layout(nq, B, n, L, nl, R);
    *appended = s.cnt;
    *control = s.ctrl;
}

struct ScanState {
    int32_t* tau;
    uint32_t* cnt;
    uint32_t* hmax;
    uint32_t* hist;
    uint64_t* cand;
    uint32_t* ctrl;  // [0] work counter, [1] overflow count, [2] fallback cursor
    int32_t* ovf;
    int32_t* dfr;  // queries whose final selection needs the workgroup path (ctrl[3] of them)
    uint64_t* fb;
    int64_t cap;
    int32_t hlo, hw, hsh;  // bin b covers sums [hlo + b*hw, hlo + (b+1)*hw), hw = 1 << hsh
};

struct Problem {
    const int8_t* lut;
    int64_t nq;
    int32_t B;
    const uint8_t* codes;
    int32_t stride;       // bytes per row (tiled: the row's 16-byte segments, padded)
    int64_t n;
    const int32_t* ids;
    const int64_t* leaf_offsets;
    int32_t L;
    const int32_t* leaves;
    int32_t nl;
    int32_t R;
    int32_t* out_ids;
    int32_t* out_scores;
    int64_t tile_bytes;   // tiled layout: bytes per 64-row tile (0: row-major)
    const int32_t* leaf_bias;  // residual variant: [nq][nl], or null
    int32_t bias_bound;
};

// The residual variant's term for the query's j-th leaf (0 without one).
__device__ __forceinline__ int32_t leaf_bias_at(const Problem& p, int64_t q, int j) {
    if (!p.leaf_bias) return 0;
    const int32_t v = p.leaf_bias[q * p.nl + j];
    return v < -p.bias_bound ? -p.bias_bound : (v > p.bias_bound ? p.bias_bound : v);
}
// The threshold for a sum whose score is sum + off.  INT_MAX (disabled) and
// INT_MIN (open) stay as they are; every other threshold is a score in the
// histogram range, |tq| <= 255 B + bound, so tq - off cannot wrap.
__device__ __forceinline__ int32_t sat_sub(int32_t tq, int32_t off) {
    return (tq == INT_MAX || tq == INT_MIN) ? tq : tq - off;
}

// Row `row`'s first 16-byte segment and the distance between its segments:
// row-major rows are contiguous; in the tiled layout segment j of the 64 rows
// of a tile is one contiguous 1 KB run, so the same segment of consecutive rows
// is consecutive in memory.
__device__ __forceinline__ const uint8_t* code_row(const Problem& p, int64_t row) {
    return p.tile_bytes ? p.codes + (row >> 6) * p.tile_bytes + (row & 63) * 16 : p.codes + row * p.stride;
}
__device__ __forceinline__ int32_t seg_step(const Problem& p) { return p.tile_bytes ? 1024 : 16; }

__device__ __forceinline__ int hist_bin(int32_t s, int32_t hlo, int32_t hsh) {
    const int64_t d = (int64_t)s - hlo;
    const int64_t j = d < 0 ? 0 : d >> hsh;
    return (int)(j >= kNB ? kNB - 1 : j);
}
__device__ __forceinline__ int32_t ld_coherent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Orders this wave's LDS accesses across lanes (the hardware executes one
// wave's LDS operations in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int nibble(const uint8_t* row, int b) { return (row[b >> 1] >> (4 * (b & 1))) & 15; }

// Tables read by per-lane lookups (warm-up, fallback) are held in LDS center
// major: entry (b, c) at byte c * S + b with S = tstride(B), a multiple of 4 whose
// dword count is odd.  Lanes summing different rows read the same block at the
// same time, so their entries fall in 16 different banks (lanes on the same
// center share one address); block major, a block's 16 entries would share
// four banks.
__host__ __device__ constexpr int32_t tstride(int32_t B) { return 4 * (((B + 3) / 4) | 1); }

// Copies a query's int8 [B][16] table (src 16-byte aligned) into dst center
// major with stride tstride(Bp), Bp >= B, blocks B..Bp-1 zero: one 16-byte
// block per thread and pass, the loads of four passes issued before any is
// written.
__device__ __forceinline__ void stage_table_cm(int8_t* dst, const int8_t* src, int32_t B, int32_t Bp, int t0,
                                               int nt) {
    const int32_t S = tstride(Bp);
    for (int b0 = t0; b0 < Bp; b0 += 4 * nt) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = b0 + k * nt;
            v[k] = b < B ? *reinterpret_cast<const uint4*>(src + (int64_t)b * 16) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = b0 + k * nt;
            if (b >= Bp) break;
            const uint32_t wd[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int c = 0; c < 16; ++c) dst[c * S + b] = (int8_t)(wd[c >> 2] >> (8 * (c & 3)));
        }
    }
}

// Sum of one row's table entries; the table is int8, center major with stride
// S (at least tstride(B)), in LDS.
__device__ __forceinline__ int32_t row_sum(const int8_t* lut_s, int32_t B, int32_t S, const uint8_t* row,
                                           bool aligned4, int32_t ss = 16) {
    int32_t s = 0;
    if (aligned4) {  // dword k of the row: segment k / 4 (ss bytes apart), word k % 4
        for (int b0 = 0; b0 < B; b0 += 8) {
            const int k = b0 >> 3;
            const uint32_t wv = *reinterpret_cast<const uint32_t*>(row + (k >> 2) * ss + (k & 3) * 4);
            const int lim = B - b0 < 8 ? B - b0 : 8;
            for (int t = 0; t < lim; ++t) s += lut_s[((wv >> (4 * t)) & 15) * S + b0 + t];
        }
    } else {
        for (int b = 0; b < B; ++b) s += lut_s[nibble(row, b) * S + b];
    }
    return s;
}

// Sum of one row's table entries for rows of whole 16-byte segments (nseg of
// them, ss bytes apart): the segments of a batch of up to 8 are all loaded
// before any lookup, so a row costs one memory round trip per batch rather
// than one per word.  The table is center major in LDS with stride S, its
// blocks zero from B up to 32 nseg (nibbles past B, in padding bytes, add 0).
__device__ __forceinline__ int32_t row_sum_seg(const int8_t* lut_s, int32_t S, const uint8_t* src, int nseg,
                                               int32_t ss) {
    int32_t sv = 0;
    for (int j0 = 0; j0 < nseg; j0 += 8) {
        uint4 r[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (j0 + k < nseg) r[k] = *reinterpret_cast<const uint4*>(src + (j0 + k) * ss);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (j0 + k >= nseg) break;
            const uint32_t wd[4] = {r[k].x, r[k].y, r[k].z, r[k].w};
#pragma unroll
            for (int u = 0; u < 32; ++u)
                sv += lut_s[(int)((wd[u >> 3] >> (4 * (u & 7))) & 15u) * S + 32 * (j0 + k) + u];
        }
    }
    return sv;
}

// LDS bytes of a query's center-major table padded to whole 32-block segments.
__host__ __device__ inline size_t seg_lut_bytes(int32_t B) {
    return ((size_t)tstride(32 * (((B + 1) / 2 + 15) / 16)) * 16 + 15) & ~(size_t)15;
}

// ------------------------------------------------------------------ leaf -> query inversion
__global__ void zero_u32_kernel(uint32_t* p, int64_t count) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void leaf_count_kernel(const int32_t* __restrict__ leaves, int64_t pairs, int32_t L,
                                  uint32_t* __restrict__ lcnt) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < pairs; i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t l = leaves[i];
        if (l >= 0 && l < L) atomicAdd(&lcnt[l], 1u);
    }
}

// The same two steps with the pairs of a workgroup's chunk counted in LDS
// first (L <= kLeafLds): one device atomic per (workgroup, leaf) instead of one
// per pair.  Chunks of kLeafChunk pairs; dynamic LDS of L words.
constexpr int kLeafLds = 16384;
constexpr int kLeafThreads = 1024;
constexpr int64_t kLeafChunk = 32768;

__global__ __launch_bounds__(kLeafThreads) void leaf_count_lds_kernel(const int32_t* __restrict__ leaves, int64_t pairs,
                                                                     int32_t L, uint32_t* __restrict__ lcnt) {
    extern __shared__ uint32_t cnt_s[];
    const int tid = threadIdx.x;
    for (int l = tid; l < L; l += kLeafThreads) cnt_s[l] = 0;
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * kLeafChunk;
    const int64_t i1 = i0 + kLeafChunk < pairs ? i0 + kLeafChunk : pairs;
    for (int64_t i = i0 + tid; i < i1; i += kLeafThreads) {
        const int32_t l = leaves[i];
        if (l >= 0 && l < L) atomicAdd(&cnt_s[l], 1u);
    }
    __syncthreads();
    for (int l = tid; l < L; l += kLeafThreads)
        if (cnt_s[l]) atomicAdd(&lcnt[l], cnt_s[l]);
}

__global__ __launch_bounds__(kLeafThreads) void leaf_scatter_lds_kernel(const int32_t* __restrict__ leaves, int64_t nq,
                                                                       int32_t nl, int32_t L,
                                                                       const int32_t* __restrict__ lqoff,
                                                                       uint32_t* __restrict__ lcur,
                                                                       int32_t* __restrict__ qlist,
                                                                       const int32_t* __restrict__ bias, int32_t bound,
                                                                       int32_t* __restrict__ qbias) {
    extern __shared__ uint32_t pos_s[];
    const int tid = threadIdx.x;
    const int64_t pairs = nq * nl;
    for (int l = tid; l < L; l += kLeafThreads) pos_s[l] = 0;
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * kLeafChunk;
    const int64_t i1 = i0 + kLeafChunk < pairs ? i0 + kLeafChunk : pairs;
    for (int64_t i = i0 + tid; i < i1; i += kLeafThreads) {
        const int32_t l = leaves[i];
        if (l >= 0 && l < L) atomicAdd(&pos_s[l], 1u);
    }
    __syncthreads();
    // the chunk's slots of each leaf: one reservation per leaf
    for (int l = tid; l < L; l += kLeafThreads)
        if (pos_s[l]) pos_s[l] = (uint32_t)lqoff[l] + atomicAdd(&lcur[l], pos_s[l]);
    __syncthreads();
    for (int64_t i = i0 + tid; i < i1; i += kLeafThreads) {
        const int32_t l = leaves[i];
        if (l < 0 || l >= L) continue;
        const uint32_t at = atomicAdd(&pos_s[l], 1u);
        qlist[at] = (int32_t)(i / nl);
        int32_t v = bias ? bias[i] : 0;
        v = v < -bound ? -bound : (v > bound ? bound : v);
        qbias[at] = v;
    }
}

// Single workgroup: query offsets per leaf and item offsets per leaf.
__global__ __launch_bounds__(1024) void leaf_scan_kernel(const uint32_t* __restrict__ lcnt,
                                                         const int64_t* __restrict__ leaf_offsets, int32_t L,
                                                         int32_t qg, int32_t ipts, int32_t* __restrict__ lqoff,
                                                         int64_t* __restrict__ itemoff) {
    __shared__ int64_t part_q[1024], part_i[1024];
    const int tid = threadIdx.x;
    const int64_t per = (L + 1023) / 1024;
    const int64_t a = tid * per, b = (a + per < L) ? a + per : L;
    int64_t sq = 0, si = 0;
    for (int64_t l = a; l < b; ++l) {
        const int64_t nqL = lcnt[l];
        const int64_t rows = leaf_offsets[l + 1] - leaf_offsets[l];
        sq += nqL;
        si += (nqL > 0 && rows > 0) ? ((nqL + qg - 1) / qg) * ((rows + ipts - 1) / ipts) : 0;
    }
    part_q[tid] = sq;
    part_i[tid] = si;
    __syncthreads();
    if (tid == 0) {
        int64_t cq = 0, ci = 0;
        for (int t = 0; t < 1024; ++t) {
            const int64_t x = part_q[t], y = part_i[t];
            part_q[t] = cq;
            part_i[t] = ci;
            cq += x;
            ci += y;
        }
        lqoff[L] = (int32_t)cq;
        itemoff[L] = ci;
    }
    __syncthreads();
    int64_t cq = part_q[tid], ci = part_i[tid];
    for (int64_t l = a; l < b; ++l) {
        lqoff[l] = (int32_t)cq;
        itemoff[l] = ci;
        const int64_t nqL = lcnt[l];
        const int64_t rows = leaf_offsets[l + 1] - leaf_offsets[l];
        cq += nqL;
        ci += (nqL > 0 && rows > 0) ? ((nqL + qg - 1) / qg) * ((rows + ipts - 1) / ipts) : 0;
    }
}

// Also carries each (query, leaf) pair's clipped residual term next to the
// query in the leaf's list (qbias; 0 without the variant).
__global__ void leaf_scatter_kernel(const int32_t* __restrict__ leaves, int64_t nq, int32_t nl, int32_t L,
                                    const int32_t* __restrict__ lqoff, uint32_t* __restrict__ lcur,
                                    int32_t* __restrict__ qlist, const int32_t* __restrict__ bias, int32_t bound,
                                    int32_t* __restrict__ qbias) {
    const int64_t pairs = nq * nl;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < pairs; i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t l = leaves[i];
        if (l < 0 || l >= L) continue;
        const uint32_t pos = atomicAdd(&lcur[l], 1u);
        qlist[lqoff[l] + pos] = (int32_t)(i / nl);
        int32_t v = bias ? bias[i] : 0;
        v = v < -bound ? -bound : (v > bound ? bound : v);
        qbias[lqoff[l] + pos] = v;
    }
}

// ------------------------------------------------------------------ warm-up threshold
// One workgroup per query: sum the first W rows of the query's scan order (its
// leaves in probe order, or rows 0..W-1), set tau to the R-th best of them
// (a valid lower bound on the R-th best over all scanned rows), and clear the
// query's candidate count and histogram.
__global__ __launch_bounds__(kSelThreads) void warmup_kernel(Problem p, ScanState st, int32_t W) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ SelectShared sh;
    __shared__ int64_t got_s;
    const int64_t q = blockIdx.x;
    const int tid = threadIdx.x;
    int8_t* lut_s = reinterpret_cast<int8_t*>(smem);
    uint64_t* keys = reinterpret_cast<uint64_t*>(smem + seg_lut_bytes(p.B));
    // rows of whole 16-byte segments are summed a segment batch at a time on a
    // table padded to whole segments
    const bool al16 = (p.stride & 15) == 0 && (reinterpret_cast<uintptr_t>(p.codes) & 15) == 0;
    const int nseg = ((p.B + 1) / 2 + 15) / 16;
    const int32_t Bp = al16 ? 32 * nseg : p.B, S = tstride(Bp);
    stage_table_cm(lut_s, p.lut + q * p.B * 16, p.B, Bp, tid, kSelThreads);
    for (int j = tid; j < kNB; j += kSelThreads) st.hist[q * kNB + j] = 0;
    if (tid == 0) {
        st.cnt[q] = 0;
        st.hmax[q] = 0;
        got_s = 0;
    }
    for (int j = tid; j < W; j += kSelThreads) keys[j] = 0;
    __syncthreads();
    const bool al4 = (p.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(p.codes) & 3) == 0;
    const int nsrc = p.leaves ? p.nl : 1;
    for (int j = 0; j < nsrc; ++j) {
        const int64_t got = got_s;
        if (got >= W) break;
        int64_t a, b;
        if (p.leaves) {
            const int32_t l = p.leaves[q * p.nl + j];
            const bool okl = l >= 0 && l < p.L;
            a = okl ? p.leaf_offsets[l] : 0;
            b = okl ? p.leaf_offsets[l + 1] : 0;
        } else {
            a = 0;
            b = p.n;
        }
        int64_t take = b - a;
        if (take > W - got) take = W - got;
        const int32_t off = p.leaves ? leaf_bias_at(p, q, j) : 0;
        for (int64_t t = tid; t < take; t += kSelThreads) {
            const int64_t row = a + t;
            const uint8_t* src = code_row(p, row);
            const int32_t s = (al16 ? row_sum_seg(lut_s, S, src, nseg, seg_step(p))
                                    : row_sum(lut_s, p.B, S, src, al4, seg_step(p))) + off;
            keys[got + t] = int_key(s, p.ids ? p.ids[row] : (int32_t)row);
        }
        __syncthreads();
        if (tid == 0) got_s = got + take;
        __syncthreads();
    }
    int nvalid = 0;
    const uint64_t kth = wg_kth_largest<kSelThreads>(LdsKeys{keys}, W, p.R, sh, &nvalid);
    if (tid == 0) st.tau[q] = nvalid >= p.R ? key_int_score(kth) : INT_MIN;
    if (q == 0 && tid < 16) st.ctrl[tid] = 0;
}

// Warm-up of a full scan by a few queries, whose thresholds every workgroup of
// the scan starts from: W rows evenly spaced over the whole array (distinct, as
// W <= n), one per thread of nwg workgroups per query, each workgroup writing a
// histogram of its rows' sums; warmup_spread_finish_kernel adds them up.  Many
// more rows than the one-wave warm-up reads, in less time.  Rows of whole
// 16-byte segments load all their segments (up to 8) before any lookup, on a
// table padded with zero blocks to whole segments.
__global__ __launch_bounds__(kSpreadThreads) void warmup_spread_kernel(Problem p, ScanState st, int32_t W,
                                                                       uint32_t* part) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint32_t h_s[kNB];
    const int64_t q = blockIdx.y;
    const int tid = threadIdx.x;
    int8_t* lut_s = reinterpret_cast<int8_t*>(smem);
    const bool al4 = (p.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(p.codes) & 3) == 0;
    const bool al16 = (p.stride & 15) == 0 && (reinterpret_cast<uintptr_t>(p.codes) & 15) == 0;
    const int nseg = ((p.B + 1) / 2 + 15) / 16;
    const int32_t Bp = al16 ? 32 * nseg : p.B;
    stage_table_cm(lut_s, p.lut + q * p.B * 16, p.B, Bp, tid, kSpreadThreads);
    for (int j = tid; j < kNB; j += kSpreadThreads) h_s[j] = 0;
    __syncthreads();
    const int32_t S = tstride(Bp), ss = seg_step(p);
    const int64_t i = (int64_t)blockIdx.x * kSpreadThreads + tid;
    if (i < W) {
        const int64_t row = i * p.n / W;
        const uint8_t* src = code_row(p, row);
        const int32_t sv = al16 ? row_sum_seg(lut_s, S, src, nseg, ss) : row_sum(lut_s, p.B, S, src, al4, ss);
        atomicAdd(&h_s[hist_bin(sv, st.hlo, st.hsh)], 1u);
    }
    __syncthreads();
    uint32_t* dst = part + (q * gridDim.x + blockIdx.x) * kNB;
    for (int j = tid; j < kNB; j += kSpreadThreads) dst[j] = h_s[j];
}

// One workgroup per query: adds up the spread warm-up's partial histograms,
// sets tau to the lower edge of the bin holding the R-th best of the W sums (a
// valid bound, at most one bin below the exact R-th best) and clears the
// query's candidate count and histogram.
__global__ __launch_bounds__(kNB) void warmup_spread_finish_kernel(Problem p, ScanState st, int32_t W, int32_t nwg,
                                                                   const uint32_t* part) {
    __shared__ uint32_t h_s[kNB];
    __shared__ __align__(16) uint32_t h4_s[4][kNB];
    const int64_t q = blockIdx.x;
    const int j = threadIdx.x;
    if (q == 0 && j < 16) st.ctrl[j] = 0;
    {
        // thread j adds bins 4 (j % 256) .. +3 of every fourth partial
        // histogram from j / 256 (16-byte loads, 16 in flight), then the four
        // groups are added in LDS
        const int j4 = (j & 255) * 4, grp = j >> 8;
        const uint32_t* src = part + q * nwg * kNB + j4;
        uint4 c = make_uint4(0, 0, 0, 0);
#pragma unroll 16
        for (int g = grp; g < nwg; g += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)g * kNB);
            c.x += v.x;
            c.y += v.y;
            c.z += v.z;
            c.w += v.w;
        }
        *reinterpret_cast<uint4*>(&h4_s[grp][j4]) = c;
    }
    __syncthreads();
    h_s[j] = h4_s[0][j] + h4_s[1][j] + h4_s[2][j] + h4_s[3][j];
    st.hist[q * kNB + j] = 0;
    if (j == 0) {
        st.cnt[q] = 0;
        st.hmax[q] = 0;
    }
    __syncthreads();
    if (j >= kWave) return;
    const int lane = j;
    if (W < p.R) {
        if (lane == 0) st.tau[q] = INT_MIN;
        return;
    }
    // lane l owns the 16 bins from the top 16 l down
    int cb[16], tot = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        cb[k] = (int)h_s[kNB - 1 - 16 * lane - k];
        tot += cb[k];
    }
    const int incl = wave_inclusive_sum(tot);
    const uint64_t mk = __ballot(incl >= p.R);
    const int l = __ffsll((unsigned long long)mk) - 1;  // W >= R sums, so some lane reaches R
    if (lane == l) {
        int cum = incl - tot, bin = kNB - 1 - 16 * lane;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            cum += cb[k];
            if (cum >= p.R) {
                bin = kNB - 1 - 16 * lane - k;
                break;
            }
        }
        st.tau[q] = (int32_t)(st.hlo + ((int64_t)bin << st.hsh));
    }
}

// ------------------------------------------------------------------ main scan
// Source of the zero table entries a staged chunk holds for blocks past B.
__device__ __align__(16) int8_t g_zero16[16];

// One wave's direct global-to-LDS copy: lane l's 16 bytes at src land at
// lds_base + 16 l (lds_base is wave-uniform).  Completion is counted by vmcnt.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

template <int V>
__device__ __forceinline__ constexpr int buf_value(std::integral_constant<int, V>) { return V; }
__device__ __forceinline__ int buf_value(int b) { return b; }

struct MainArgs {
    Problem p;
    ScanState st;
    int32_t nkstep;   // k-steps of 4 blocks (blocks rounded up to 8)
    int32_t nchunk;   // 1: the table is resident (B <= 64); else staged chunks of 32 blocks
    int32_t qg;       // queries per item
    int32_t item_pts; // rows per item (MFMA kernel: kItemPts; streaming kernel: at most 65536)
    int32_t nqg;      // query groups (full scan)
    int64_t n_items;  // items (full scan); partitioned: itemoff[L]
    const int32_t* lqoff;
    const int32_t* qlist;
    const int32_t* qbias;  // residual terms beside qlist, or null
    const int64_t* itemoff;
    int fast_codes;   // rows 16-byte aligned (stride % 16 == 0)
};

// Item -> (rows [p0, p1), first entry qbase of its query list, qn queries).
// Full scan: item = chunk * nqg + group.  Partitioned: items are numbered leaf
// by leaf (itemoff), and within a leaf chunk-major over its query groups.
__device__ __forceinline__ void decode_item(const MainArgs& a, int64_t item, int64_t& p0, int64_t& p1,
                                            int64_t& qbase, int& qn) {
    const Problem& p = a.p;
    const int64_t G = a.qg;
    if (!p.leaves) {
        const int64_t chunk = item / a.nqg, grp = item % a.nqg;
        p0 = chunk * a.item_pts;
        p1 = p0 + a.item_pts < p.n ? p0 + a.item_pts : p.n;
        qbase = grp * G;
        qn = (int)(p.nq - qbase < G ? p.nq - qbase : G);
    } else {
        int lo = 0, hi = p.L;  // largest l with itemoff[l] <= item
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.itemoff[mid] <= item) lo = mid; else hi = mid;
        }
        const int l = lo;
        const int64_t nqL = a.lqoff[l + 1] - a.lqoff[l];
        const int64_t ng = (nqL + G - 1) / G;
        const int64_t loc = item - a.itemoff[l];
        const int64_t chunk = loc / ng, grp = loc % ng;
        const int64_t ra = p.leaf_offsets[l], rb = p.leaf_offsets[l + 1];
        p0 = ra + chunk * a.item_pts;
        p1 = p0 + a.item_pts < rb ? p0 + a.item_pts : rb;
        qbase = a.lqoff[l] + grp * G;
        qn = (int)(nqL - grp * G < G ? nqL - grp * G : G);
    }
}

// decode_item by one whole wave (every lane gets the result): a partitioned
// item's leaf is found in two rounds of 64 loads (every ceil(L/64)-th entry of
// itemoff, then the entries of the chosen stride) instead of a binary search's
// log2 L dependent loads, which every workgroup waited for at every item start.
__device__ __forceinline__ void decode_item_wave(const MainArgs& a, int64_t item, int64_t& p0, int64_t& p1,
                                                 int64_t& qbase, int& qn) {
    const Problem& p = a.p;
    if (!p.leaves || p.L > kWave * kWave) {
        decode_item(a, item, p0, p1, qbase, qn);
        return;
    }
    const int lane = lane_id();
    const int64_t G = a.qg;
    // largest l < L with itemoff[l] <= item (itemoff[0] = 0, non-decreasing)
    const int step = (p.L + kWave - 1) / kWave;
    const int i1 = lane * step;
    const uint64_t m1 = __ballot(i1 < p.L && a.itemoff[i1] <= item);
    const int l1 = (63 - __clzll((long long)m1)) * step;
    const int i2 = l1 + lane;
    const uint64_t m2 = __ballot(lane < step && i2 < p.L && a.itemoff[i2] <= item);
    const int l = l1 + (63 - __clzll((long long)m2));
    const int64_t nqL = a.lqoff[l + 1] - a.lqoff[l];
    const int64_t ng = (nqL + G - 1) / G;
    const int64_t loc = item - a.itemoff[l];
    const int64_t chunk = loc / ng, grp = loc % ng;
    const int64_t ra = p.leaf_offsets[l], rb = p.leaf_offsets[l + 1];
    p0 = ra + chunk * a.item_pts;
    p1 = p0 + a.item_pts < rb ? p0 + a.item_pts : rb;
    qbase = a.lqoff[l] + grp * G;
    qn = (int)(nqL - grp * G < G ? nqL - grp * G : G);
}

// The next item for a workgroup, by its wave 0 (lane 0 holds the claimed index
// and claims the one after): the item and its rows and queries go to LDS.
__device__ __forceinline__ void fetch_item(const MainArgs& a, int64_t& claimed, int64_t n_items, int64_t* item_s,
                                           int64_t* p0_s, int64_t* p1_s, int64_t* qbase_s, int* qn_s,
                                           uint32_t* slab_s) {
    const int lane = lane_id();
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)claimed);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)claimed >> 32));
    const int64_t item = (int64_t)(((uint64_t)hi << 32) | lo);
    if (lane == 0) *item_s = item;
    if (item >= n_items) return;
    int64_t p0, p1, qbase;
    int qn;
    decode_item_wave(a, item, p0, p1, qbase, qn);
    if (lane == 0) {
        *p0_s = p0;
        *p1_s = p1;
        *qbase_s = qbase;
        *qn_s = qn;
        if (slab_s) *slab_s = 0;
        claimed = (int64_t)atomicAdd(&a.st.ctrl[0], 1u);
    }
}

// Appends a wave's logged hits to the queries' candidate lists and counts them
// (kGlobalHist: also in the global histograms, hit by hit; fh: also in the
// wave's flush histogram, merged into the global ones after the flush) in the
// item's LDS histogram (lh: kLB bins per local query, starting at the
// query's global bin jb_s at item start; the top bin also takes everything
// above it).  Log entry: sum (high 32 bits) | local query (bits 16..21) |
// row - p0 (low 16).  Each lane takes four entries per pass.  The pass first
// counts its entries per local query in the wave's LDS scratch (wq), then
// reserves each query's list slots with one global atomic per query, so the
// per-query counters see one atomic per pass instead of one per hit and no
// two lanes of an atomic share an address.
template <bool kGlobalHist>
__device__ __forceinline__ void flush_log(const Problem& p, const ScanState& st, const uint64_t* log,
                                          int log_n, const int32_t* qid_s, uint32_t* qapp_s, int64_t p0,
                                          uint32_t* wq, uint32_t* wm, uint32_t* lh, const int32_t* jb_s,
                                          uint32_t* fh = nullptr) {
    const int lane = lane_id();
    for (int base = 0; base < log_n; base += 4 * kWave) {
        wq[lane] = 0;
        wm[lane] = 0;
        wave_fence();
        uint64_t ent[4];
        bool ok[4];
        int ql[4];
        uint32_t li[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = base + u * kWave + lane;
            ok[u] = e < log_n;
            ent[u] = log[ok[u] ? e : 0];
            ql[u] = (int)((ent[u] >> 16) & 63);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {  // lanes without an entry add 0 to their own counter
            li[u] = atomicAdd(&wq[ok[u] ? ql[u] : lane], ok[u] ? 1u : 0u);
            if (ok[u]) {
                // a logged sum is at or above the threshold the item started
                // with, so its bin is at least jb_s; anything lower would be
                // dropped (never counted where it could overstate a bound)
                const int gbin = hist_bin((int32_t)(uint32_t)(ent[u] >> 32), st.hlo, st.hsh);
                const int bl = gbin - jb_s[ql[u]];
                if (bl >= 0) {
                    atomicAdd(&lh[ql[u] * kLB + (bl < kLB ? bl : kLB - 1)], 1u);
                    if (fh) atomicAdd(&fh[ql[u] * kLB + (bl < kLB ? bl : kLB - 1)], 1u);
                }
                if (kGlobalHist) atomicMax(&wm[ql[u]], (uint32_t)gbin);
            }
        }
        wave_fence();
        const uint32_t c = wq[lane];
        const int q = qid_s[lane];
        uint32_t gb = 0;
        if (c) {
            gb = atomicAdd(&st.cnt[q], c);
            if (kGlobalHist) atomicMax(&st.hmax[q], wm[lane]);
            atomicAdd(&qapp_s[lane], c);
        }
        wq[lane] = gb;
        wave_fence();
        int32_t idv[4];
        if (p.ids) {
#pragma unroll
            for (int u = 0; u < 4; ++u) idv[u] = p.ids[ok[u] ? p0 + (int64_t)(ent[u] & 0xFFFF) : p0];
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) idv[u] = (int32_t)(p0 + (int64_t)(ent[u] & 0xFFFF));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (!ok[u]) continue;
            const int32_t sv = (int32_t)(uint32_t)(ent[u] >> 32);
            const uint32_t slot = wq[ql[u]] + li[u];
            const int qq = qid_s[ql[u]];
            if ((int64_t)slot < st.cap) st.cand[(int64_t)qq * st.cap + slot] = int_key(sv, idv[u]);
            if (kGlobalHist) atomicAdd(&st.hist[(int64_t)qq * kNB + hist_bin(sv, st.hlo, st.hsh)], 1u);
        }
        wave_fence();
    }
}

// Raises the item-local thresholds of one wave's queries (ql = w, w+8, ...) to
// the highest LDS-histogram edge with at least R of this item's appended sums
// at or above it: those are real rows, so the edge is a valid lower bound.
__device__ __forceinline__ void local_refresh(const uint32_t* lh, int32_t* tau_s, const int32_t* jb_s, int qn, int w,
                                              int R, int32_t hlo, int32_t hsh) {
    const int lane = lane_id();
    const int b = kLB - 1 - lane;  // lane 0 owns the highest bin
#pragma unroll 1
    for (int k = 0; k < kQG / kScanWaves; ++k) {
        const int ql = w + kScanWaves * k;
        if (ql >= qn) break;
        const int incl = wave_inclusive_sum((int)lh[ql * kLB + b]);
        const uint64_t mk = __ballot(incl >= R);
        if (mk && lane == __ffsll((unsigned long long)mk) - 1)
            atomicMax(&tau_s[ql], (int32_t)(hlo + ((int64_t)(jb_s[ql] + b) << hsh)));
    }
}

// Adds a wave's flush histogram (fh: kLB bins per local query from jb_s) to the
// global histograms and clears it (a bin past the global range is merged into
// the last one, which can only undercount higher bins); raises hmax to the
// highest bin added.
__device__ __forceinline__ void merge_flush(const ScanState& st, uint32_t* fh, const int32_t* jb_s,
                                            const int32_t* qid_s, int qn) {
    const int lane = lane_id();
#pragma unroll 1
    for (int ql = 0; ql < qn; ++ql) {
        const int q = qid_s[ql];
        const uint32_t c = fh[ql * kLB + lane];
        fh[ql * kLB + lane] = 0;
        int gb = jb_s[ql] + lane;
        gb = gb >= kNB ? kNB - 1 : gb;
        if (c) atomicAdd(&st.hist[(int64_t)q * kNB + gb], c);
        const uint64_t nz = __ballot(c != 0);
        if (lane == 0 && nz) {
            const int top = jb_s[ql] + 63 - __clzll((long long)nz);
            atomicMax(&st.hmax[q], (uint32_t)(top >= kNB ? kNB - 1 : top));
        }
    }
}

// Adds the item's LDS histograms (lh: kLB bins per local query from jb_s, the
// top bin holding everything above) of one wave's queries (ql = w, w+8, ...)
// to the global histograms, with a bin past the global range merged into the
// last one (both can only undercount higher bins, so every threshold drawn
// from the global histograms stays a valid bound), and raises hmax to the
// highest bin added.
__device__ __forceinline__ void merge_item_hist(const ScanState& st, const uint32_t* lh, const int32_t* jb_s,
                                                const int32_t* qid_s, int qn, int w) {
    const int lane = lane_id();
#pragma unroll 1
    for (int ql = w; ql < qn; ql += kScanWaves) {
        const int q = qid_s[ql];
        const uint32_t c = lh[ql * kLB + lane];
        int gb = jb_s[ql] + lane;
        gb = gb >= kNB ? kNB - 1 : gb;
        if (c) atomicAdd(&st.hist[(int64_t)q * kNB + gb], c);
        const uint64_t nz = __ballot(c != 0);
        if (lane == 0 && nz) {
            const int top = jb_s[ql] + 63 - __clzll((long long)nz);
            atomicMax(&st.hmax[q], (uint32_t)(top >= kNB ? kNB - 1 : top));
        }
    }
}

// Publishes one wave's queries' item-local thresholds (ql = w, w+8, ...).
__device__ __forceinline__ void publish_item(const ScanState& st, const int32_t* tau_s, const int32_t* qid_s, int qn,
                                             int w) {
    const int lane = lane_id();
    const int ql = w + kScanWaves * lane;
    if (lane < kQG / kScanWaves && ql < qn) atomicMax(st.tau + qid_s[ql], tau_s[ql]);
}

// Raises tau of query q to the highest histogram edge with at least R appended
// sums at or above it (one wave; general case, any window).
__device__ __forceinline__ void refresh_tau(const ScanState& st, int q, int R) {
    const int lane = lane_id();
    const int32_t tcur = ld_coherent(st.tau + q);
    const int jt = tcur == INT_MIN ? 0 : hist_bin(tcur, st.hlo, st.hsh);
    const int jm = (int)ld_coherent(st.hmax + q);
    int cum = 0;
    for (int top = jm; top >= jt; top -= kWave) {
        const int j = top - lane;
        const int v = j >= jt ? (int)ld_coherent(st.hist + (int64_t)q * kNB + j) : 0;
        const int incl = wave_inclusive_sum(v);
        const uint64_t mk = __ballot(cum + incl >= R);
        if (mk) {
            const int l = __ffsll((unsigned long long)mk) - 1;
            if (lane == 0) atomicMax(st.tau + q, (int32_t)(st.hlo + ((int64_t)(top - l) << st.hsh)));
            return;
        }
        cum += __shfl(incl, kWave - 1, kWave);
    }
}

// refresh_tau for the (up to 8) queries ql = w, w+8, ... of one wave that got
// appends in this item, with every load of all of them issued together (one
// round trip for thresholds and histogram tops, one for the 64-bin windows).
// Queries ql = first + stride * k (k < 8); with tau_s, each query's item-local
// threshold is also raised to the global one and to the new bound.
__device__ __forceinline__ void refresh_tau_wave(const ScanState& st, const int32_t* qid_s, const uint32_t* qapp_s,
                                                 int qn, int first, int stride, int R, int32_t* tau_s = nullptr) {
    const int lane = lane_id();
    int qk = -1;
    if (lane < 8) {
        const int ql = first + stride * lane;
        if (ql < qn && qapp_s[ql] > 0) qk = qid_s[ql];
    }
    if (__ballot(qk >= 0) == 0) return;
    int32_t tc = INT_MIN;
    int jm = 0;
    if (qk >= 0) {
        tc = ld_coherent(st.tau + qk);
        jm = (int)ld_coherent(st.hmax + qk);
    }
    if (tau_s && qk >= 0) atomicMax(&tau_s[first + stride * lane], tc);
    int qs[8], top[8], jt[8], v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        qs[k] = __shfl(qk, k, kWave);
        top[k] = __shfl(jm, k, kWave);
        const int32_t t = __shfl(tc, k, kWave);
        jt[k] = t == INT_MIN ? 0 : hist_bin(t, st.hlo, st.hsh);
        const int j = top[k] - lane;
        v[k] = (qs[k] >= 0 && j >= jt[k]) ? (int)ld_coherent(st.hist + (int64_t)qs[k] * kNB + j) : 0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (qs[k] < 0) continue;
        const int incl = wave_inclusive_sum(v[k]);
        const uint64_t mk = __ballot(incl >= R);
        if (mk) {
            const int l = __ffsll((unsigned long long)mk) - 1;
            const int32_t nt = (int32_t)(st.hlo + ((int64_t)(top[k] - l) << st.hsh));
            if (lane == 0) {
                atomicMax(st.tau + qs[k], nt);
                if (tau_s) atomicMax(&tau_s[first + stride * k], nt);
            }
        } else if (top[k] - kWave >= jt[k]) {
            refresh_tau(st, qs[k], R);  // the R-th best lies below the first window
        }
    }
}

// kBias: the residual variant (a.qbias set); the plain scan compiles without it.
// kStaged: tables of more than 64 blocks, staged 32 blocks at a time (a.nchunk
// chunks); else the table is resident for the item (a.nchunk == 1).  kFast
// (staged only): rows 16-byte aligned, one 16-byte code load per row and step
// (a separate instantiation, so the byte-wise loads of unaligned rows leave
// no pending loads in the aligned loop).
template <bool kBias, bool kStaged, bool kFast>
__global__ __launch_bounds__(kScanThreads, 1) void scan_main_kernel(MainArgs a) {
    // resident table: lut_s, 64 blocks [kstep][ntile][lane][16]; staged: lut_s
    // and lut_t hold alternate 32-block chunks.  Two objects, so that the
    // compiler sees a chunk's copy and the other chunk's reads as disjoint and
    // does not wait for the copy before those reads.
    __shared__ __align__(16) int8_t lut_s[(kStaged ? kKCS : kKC) * 4 * kWave * 16];
    __shared__ __align__(16) int8_t lut_t[kStaged ? kKCS * 4 * kWave * 16 : 16];
    __shared__ __align__(16) uint32_t code_s[2][kTilePts * kCodeStride];
    __shared__ uint64_t log_s[kScanWaves * kLogCap];
    __shared__ uint32_t spi_s[256];                   // sparse A index word by code byte
    __shared__ int32_t qid_s[kQG];
    __shared__ uint32_t qapp_s[kQG];
    __shared__ uint32_t lh[kQG * kLB];  // this item's appended sums per query, bins from jb_s
    __shared__ int32_t tau_s[kQG];     // item-local thresholds (raised from lh)
    __shared__ int32_t jb_s[kQG];      // global bin of the threshold at item start
    __shared__ int32_t off_s[kQG];     // residual variant: the item's leaf term per query (0 otherwise)
    __shared__ uint32_t fl_s[kScanWaves * 2 * kWave];  // per-wave flush scratch
    // the item's record (item, rows, queries, next 64-row slab with a resident
    // table), two of them: with a resident table wave 0 decodes the next item
    // into the other one while the rest of the workgroup starts on this one
    __shared__ int64_t item_r[2], p0_r[2], p1_r[2], qbase_r[2];
    __shared__ uint32_t slab_r[2];
    __shared__ int32_t qn_r[2];

    const Problem& p = a.p;
    const ScanState& st = a.st;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t n_items = p.leaves ? a.itemoff[p.L] : a.n_items;
    constexpr bool dyn = !kStaged;  // resident table; else staged 32-block chunks
    uint64_t* mylog = log_s + w * kLogCap;
    uint32_t* mywq = fl_s + w * 2 * kWave;
    // sparse one-hot index words: pair indices (c & 3, (c & 3) ^ 1) of both
    // blocks of a code byte in every pair of the block (nibble 4 ^ 5 (c & 3))
    if (tid < 256) {
        const uint32_t x = (uint32_t)tid;
        const uint32_t u = (x & 3u) | (((x >> 4) & 3u) << 16);
        spi_s[tid] = (u * 0x5555u) ^ 0x44444444u;
    }

    int64_t claimed = 0;  // thread 0: the next item, claimed while the current one computes
    if (tid == 0) claimed = (int64_t)atomicAdd(&st.ctrl[0], 1u);
    int par = 0;  // the record of the current item
    if (dyn && w == 0) fetch_item(a, claimed, n_items, &item_r[0], &p0_r[0], &p1_r[0], &qbase_r[0], &qn_r[0], &slab_r[0]);
    for (;;) {
        if (!dyn && w == 0)
            fetch_item(a, claimed, n_items, &item_r[par], &p0_r[par], &p1_r[par], &qbase_r[par], &qn_r[par], &slab_r[par]);
        __syncthreads();
        const int64_t item = item_r[par];
        if (item >= n_items) break;
        const int64_t p0 = p0_r[par], p1 = p1_r[par], qbase = qbase_r[par];
        const int qn = qn_r[par];
        if (tid < kQG) {
            int32_t qq = 0;
            if (tid < qn) qq = p.leaves ? a.qlist[qbase + tid] : (int32_t)(qbase + tid);
            qid_s[tid] = qq;
            qapp_s[tid] = 0;
            if (kBias) off_s[tid] = tid < qn ? a.qbias[qbase + tid] : 0;
            const int32_t t = tid < qn ? ld_coherent(st.tau + qq) : INT_MAX;
            tau_s[tid] = t;
            jb_s[tid] = (t == INT_MIN || t == INT_MAX) ? 0 : hist_bin(t, st.hlo, st.hsh);
        }
        for (int e = tid; e < kQG * kLB; e += kScanThreads) lh[e] = 0;
        __syncthreads();

        // staged tables (B > 64): chunk c (blocks 32c .. 32c+31) into dst (lut_s
        // or lut_t) by direct global-to-LDS copies, four 1 KB slices per wave,
        // in the B-operand layout [kstep][ntile][lane][16 bytes]; blocks past B
        // copy zeros, padded query slots copy query 0's (never passed by the filter)
        auto dma_lut = [&](int c, int8_t* dst) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = w * 4 + i, s = idx >> 2, nt = idx & 3;
                const int ql = 16 * nt + r16;
                const int blk = c * 32 + 4 * s + g;
                // an integer select keeps the copy a single unmasked instruction
                const uintptr_t tab = reinterpret_cast<uintptr_t>(p.lut + ((int64_t)qid_s[ql] * p.B + blk) * 16);
                const uintptr_t src = blk < p.B ? tab : reinterpret_cast<uintptr_t>(g_zero16);
                dma16(reinterpret_cast<const void*>(src), dst + idx * (kWave * 16));
            }
        };
        // resident table (B <= 64): B operand layout [kstep][ntile][lane][16 bytes]
        // (entries past the item's queries or past B read 16 zero bytes, so every
        // load is unconditional and a thread's eight are in flight together)
        auto stage_lut = [&](int c) {
            constexpr int kPer = kKC * 4 * kWave / kScanThreads;
            v4i v[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int e = tid + k * kScanThreads;
                const int s = e >> 8, nt = (e >> 6) & 3, ln = e & 63;
                const int ql = 16 * nt + (ln & 15);
                const int blk = c * 64 + 4 * s + (ln >> 4);
                const int8_t* src =
                    (ql < qn && blk < p.B) ? p.lut + ((int64_t)qid_s[ql] * p.B + blk) * 16 : g_zero16;
                v[k] = *reinterpret_cast<const v4i*>(src);
            }
#pragma unroll
            for (int k = 0; k < kPer; ++k) *reinterpret_cast<v4i*>(lut_s + (tid + k * kScanThreads) * 16) = v[k];
        };
        // code staging: lane l of a wave owns row rowbase + l, code bytes
        // [32c, 32c+32).  A staged pair of 16-byte words carries a keep mask
        // (bit 0: first word, bit 1: second); the words are zeroed by the mask
        // only when they are stored, so the loads stay in flight for a step.
        auto load_codes = [&](int64_t rowbase, int c, uint4& x0, uint4& x1, uint32_t& keep) {
            const int64_t row = rowbase + lane;
            const bool live = row < p1;
            if (!dyn) {
                // staged chunk c: code bytes [16c, 16c + 16), one 16-byte load
                x1 = make_uint4(0, 0, 0, 0);
                if (kFast) {
                    const int64_t r = live ? row : p1 - 1;
                    const int avail = p.stride - 16 * c;
                    x0 = *reinterpret_cast<const uint4*>(code_row(p, r) + (avail >= 16 ? c * seg_step(p) : 0));
                    keep = live && avail >= 16 ? 1u : 0u;
                } else {
                    keep = 1u;
                    x0 = make_uint4(0, 0, 0, 0);
                    if (!live) return;
                    const uint8_t* src = p.codes + row * p.stride + 16 * c;
                    const int cb = (p.B + 1) / 2 - 16 * c;
                    uint32_t wd[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        uint32_t v = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * k + e < cb) v |= (uint32_t)src[4 * k + e] << (8 * e);
                        wd[k] = v;
                    }
                    x0 = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                }
                return;
            }
            if (a.fast_codes) {
                // always exactly two 16-byte loads from an in-bounds address (the
                // row itself, or the item's last row), so the number of loads in
                // flight is static
                const int64_t r = live ? row : p1 - 1;
                const uint8_t* base = code_row(p, r);
                const int32_t ss = seg_step(p);
                const int avail = p.stride - 32 * c;
                x0 = *reinterpret_cast<const uint4*>(base + (avail >= 16 ? 2 * c * ss : 0));
                x1 = *reinterpret_cast<const uint4*>(base + (avail >= 32 ? (2 * c + 1) * ss : 0));
                keep = (live && avail >= 16 ? 1u : 0u) | (live && avail >= 32 ? 2u : 0u);
            } else {
                keep = 3u;
                x0 = make_uint4(0, 0, 0, 0);
                x1 = make_uint4(0, 0, 0, 0);
                if (!live) return;
                const uint8_t* src = p.codes + row * p.stride + 32 * c;
                const int cb = (p.B + 1) / 2 - 32 * c;  // code bytes of this row from the chunk start
                uint32_t wd[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    uint32_t v = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * k + e < cb) v |= (uint32_t)src[4 * k + e] << (8 * e);
                    wd[k] = v;
                }
                x0 = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                x1 = make_uint4(wd[4], wd[5], wd[6], wd[7]);
            }
        };
        auto store_codes = [&](int buf, const uint4& x0, const uint4& x1, uint32_t keep) {
            uint32_t* d = code_s[buf] + tid * kCodeStride;
            const uint32_t k0 = (keep & 1u) ? 0xFFFFFFFFu : 0u, k1 = (keep & 2u) ? 0xFFFFFFFFu : 0u;
            d[0] = x0.x & k0; d[1] = x0.y & k0; d[2] = x0.z & k0; d[3] = x0.w & k0;
            d[4] = x1.x & k1; d[5] = x1.y & k1; d[6] = x1.z & k1; d[7] = x1.w & k1;
        };

        // A wave's steps.  With a resident table (one chunk), each step is a
        // 64-row slab that the wave claims from the item's LDS counter, so the
        // waves of an item finish within one slab of each other.  With staged
        // chunks, the waves share each chunk's table and step through the
        // 512-row tiles in lockstep: step = tile * nchunk + c, rows tile * 512
        // + 64 w onwards; chunk c's table is copied into one half of lut_s
        // while the previous chunk is computed from the other half.
        const int64_t nslabs = (p1 - p0 + 63) / 64;
        const int64_t nsteps = ((p1 - p0 + kTilePts - 1) / kTilePts) * a.nchunk;
        auto claim = [&]() -> int64_t {
            uint32_t v = 0;
            if (lane == 0) v = atomicAdd(&slab_r[par], 1u);
            return (int64_t)__builtin_amdgcn_readfirstlane(v);
        };
        // (u, c): unit (slab, or tile) and chunk of a step; valid while u < nunits
        const int64_t nunits = dyn ? nslabs : nsteps / a.nchunk;
        auto rowbase_of = [&](int64_t u) { return dyn ? p0 + 64 * u : p0 + u * kTilePts + 64 * w; };
        int64_t cu = 0, nu = 0;  // current and next unit
        int cc = 0, nc = 0;      // their chunks
        auto step_after = [&](int64_t& u, int& c) {
            if (dyn) { u = claim(); return; }
            if (++c == a.nchunk) { c = 0; ++u; }
        };
        if (dyn) cu = claim();
        nu = cu; nc = cc;
        step_after(nu, nc);
        uint4 px0, px1;
        uint32_t pkeep;
        if (!dyn && cu < nunits) dma_lut(cc, lut_s);
        if (cu < nunits) {
            load_codes(rowbase_of(cu), cc, px0, px1, pkeep);
            store_codes(0, px0, px1, pkeep);
        }
        if (nu < nunits) load_codes(rowbase_of(nu), nc, px0, px1, pkeep);
        if (dyn) stage_lut(0);
        __syncthreads();  // lut_s (its first chunk), qid_s and the first codes for this item are complete
        // resident table (no workgroup barrier until the item ends): wave 0
        // decodes the next item now, its loads overlapping the other waves' slabs
        if (dyn && w == 0)
            fetch_item(a, claimed, n_items, &item_r[par ^ 1], &p0_r[par ^ 1], &p1_r[par ^ 1], &qbase_r[par ^ 1],
                       &qn_r[par ^ 1], &slab_r[par ^ 1]);

        v4i acc[4][4];
        int32_t tq[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
        // resident tables: the global thresholds for a slab's filter are loaded
        // one slab ahead (a threshold read earlier is still a valid bound), so a
        // short slab does not wait for them; the first slab uses tau_s alone
        // (1M x 100 workload: main kernel 0.78 -> 0.75 ms)
        int32_t tqn[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
        int log_n = 0;

        // one step; buf (0 or 1) selects the code buffer and, when staged, the
        // table half read by this step (a compile-time constant there)
        auto step = [&](auto buf_tag) {
            const int buf = buf_value(buf_tag);
            const int c = cc;
            if (c == 0) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) acc[m][nt] = v4i{0, 0, 0, 0};
            }
            // thresholds for the filter (padded query slots read query 0 and are
            // disabled in the filter).  Staged: this step's, issued before the
            // next chunk's table copies so that the filter's wait does not
            // include them.  Resident: the next slab's, while this slab's were
            // loaded one slab ago.
            if (dyn) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    tq[nt] = tqn[nt];
                    tqn[nt] = ld_coherent(st.tau + qid_s[16 * nt + r16]);
                }
            } else if (c == a.nchunk - 1) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) tq[nt] = ld_coherent(st.tau + qid_s[16 * nt + r16]);
            }
            // staged: every wave has passed the previous step's barrier, so the
            // half read one step ago is free for the next step's chunk
            if (!dyn) dma_lut(nu < nunits ? nc : cc, buf ? lut_s : lut_t);  // past the last step: an unused copy
            const int kc = dyn ? kKC : kKCS;
            const int ks = a.nkstep - c * kc < kc ? a.nkstep - c * kc : kc;  // even
            const uint32_t* crow = code_s[buf] + (w * 64 + r16) * kCodeStride;
            const int8_t* lutw = (dyn || buf == 0 ? lut_s : lut_t) + lane * 16;
            // a staged wave whose 64 rows all lie past the item's end computes
            // nothing (it still takes part in the copies and barriers).  (Skipping
            // 16-query tiles past the item's last query inside the loop measured
            // slower: the branch breaks the loop's schedule.)
            const bool wlive = dyn || rowbase_of(cu) < p1;
            if (wlive) {
                // Sparse steps of 8 blocks (a code dword per row tile).  Lane group
                // g's A operand is the one-hot of the code byte g of its row (blocks
                // 2g and 2g+1 of the step) in the 2:4 sparse form: value slots 0-7
                // hold the first block's four center groups as pairs, slots 8-15 the
                // second's, one pair per group with a 1 in its first slot where the
                // group holds the center, and each slot's 2-bit index selects the
                // center inside its group (every pair of a block carries the
                // center's indices; only the pair with the 1 contributes).  The
                // values of each block are the 64-bit word 1 << 16 (c >> 2), built
                // in registers (a 16-pattern LDS table read here was as fast or,
                // on the 20M-row scan, 0.7% slower); the index word comes from
                // spi_s (one per code byte; its closed form in registers measured
                // 1-3% slower).  The matching B fragment of lane group g is the table row
                // of block g (bytes 0-15) and of block 4 + g (bytes 16-31): the
                // dense fragments of k-steps 2S and 2S+1.  (Fetching the next
                // step's A operands a step ahead measured slower: the registers
                // cost more than the latency that the second wave per SIMD hides.)
                const int nss = ks >> 1;
                auto ldB = [&](int S, int nt) {
                    const v4i lo = *reinterpret_cast<const v4i*>(lutw + ((2 * S) * 4 + nt) * kWave * 16);
                    const v4i hi = *reinterpret_cast<const v4i*>(lutw + ((2 * S + 1) * 4 + nt) * kWave * 16);
                    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                };
                v8i bq[4];
                uint32_t cw[4], cwn[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) cw[m] = crow[m * 16 * kCodeStride];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) bq[nt] = ldB(0, nt);
                __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS reads only (see below)
                for (int S = 0; S < nss; ++S) {
                    // the next step's operands are fetched unconditionally (the last
                    // step re-reads its own), at most 12 LDS reads in flight
                    const int Sn = S + 1 < nss ? S + 1 : S;
#pragma unroll
                    for (int m = 0; m < 4; ++m) cwn[m] = crow[m * 16 * kCodeStride + Sn];
                    v4i av[4];
                    int iv[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const uint32_t x = __builtin_amdgcn_ubfe(cw[m], 8 * g, 8);
                        const uint64_t lo = 1ull << ((x << 2) & 0x30u), hi = 1ull << ((x >> 2) & 0x30u);
                        av[m] = v4i{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi, (int)(uint32_t)(hi >> 32)};
                        iv[m] = spi_s[x];
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            acc[m][nt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[m], bq[nt], acc[m][nt], iv[m], 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                        bq[nt] = ldB(Sn, nt);
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) cw[m] = cwn[m];
                }
            }
            if (wlive && c == a.nchunk - 1) {
                // filter: tile (m, nt) holds, in register i, the sum of row
                // 16m + 4g + i (of this wave's 64) for query 16nt + r16.  All
                // accumulator indices are compile-time constants, so the
                // accumulators stay in registers.  A query tile is tested by
                // its maximum, then each row tile by its own, and only row
                // tiles holding a sum at or above a threshold are tested
                // element by element; rows past the item's end (a partial
                // slab) are dropped there.  The log is flushed between row
                // tiles and always has room for one (4 x 64 hits).
                const int32_t lrow0 = (int32_t)(rowbase_of(cu) - p0) + 4 * g;  // item-local row of (m, i) = (0, 0)
                const int32_t nloc = (int32_t)(p1 - p0);
                const bool full = rowbase_of(cu) + 64 <= p1;
                // a row's score is its sum plus the query's leaf term (residual
                // variant), so the sums are tested against tau minus that term
                int32_t ofs[4] = {0, 0, 0, 0};
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    tq[nt] = max(tq[nt], tau_s[16 * nt + r16]);
                    if (16 * nt + r16 >= qn) tq[nt] = INT_MAX;
                    if (kBias) {
                        ofs[nt] = off_s[16 * nt + r16];
                        tq[nt] = sat_sub(tq[nt], ofs[nt]);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    int32_t mm[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        mm[m] = max(max(acc[m][nt][0], acc[m][nt][1]), max(acc[m][nt][2], acc[m][nt][3]));
                    const int32_t mx = max(max(mm[0], mm[1]), max(mm[2], mm[3]));
                    if (__ballot(mx >= tq[nt]) == 0) continue;
                    const uint64_t qbits = (uint64_t)(16 * nt + r16) << 16;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        if (__ballot(mm[m] >= tq[nt]) == 0) continue;
                        if (log_n > kLogCap - 4 * kWave) {
                            flush_log<false>(p, st, mylog, log_n, qid_s, qapp_s, p0, mywq, mywq + kWave, lh, jb_s);
                            log_n = 0;
                            local_refresh(lh, tau_s, jb_s, qn, w, p.R, st.hlo, st.hsh);
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int32_t lr = lrow0 + 16 * m + i;
                            const bool hit = acc[m][nt][i] >= tq[nt] && (full || lr < nloc);
                            const uint64_t mk = __ballot(hit);
                            if (mk) {
                                if (hit)
                                    mylog[log_n + __popcll(mk & lanemask_lt())] =
                                        ((uint64_t)(uint32_t)(kBias ? acc[m][nt][i] + ofs[nt] : acc[m][nt][i])
                                         << 32) |
                                        qbits | (uint64_t)(uint32_t)lr;
                                log_n += __popcll(mk);
                            }
                        }
                    }
                }
            }
            // Each wave stages and reads only its own 64 code rows, so with a
            // resident table the waves need no workgroup barrier inside an
            // item: a wave-scope fence orders this wave's reads of buf^1 (one
            // step ago) before its new writes.  Staged chunks are shared by
            // all waves (the barrier below).  The next step's loads are issued
            // after the filter, whose wait for the thresholds would otherwise
            // wait for them.
            wave_fence();
            if (nu < nunits) store_codes(buf ^ 1, px0, px1, pkeep);  // buf^1 was last read one step ago
            cu = nu;
            cc = nc;
            step_after(nu, nc);
            const bool more = nu < nunits;
            if (more) load_codes(rowbase_of(nu), nc, px0, px1, pkeep);
            if (!dyn) {
                // this wave's copies of the next chunk have landed (only the
                // code load just issued may still be in flight; with byte-wise
                // code loads, everything) and its LDS writes are done; after
                // the barrier every wave's copies are visible and every wave is
                // past this step's reads
                if (more && kFast) __builtin_amdgcn_s_waitcnt(0x0071);  // vmcnt(1) lgkmcnt(0)
                else __builtin_amdgcn_s_waitcnt(0x0070);                       // vmcnt(0) lgkmcnt(0)
                wave_fence();
                __builtin_amdgcn_s_barrier();
            }
            wave_fence();
        };
        if constexpr (kStaged) {
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            while (cu < nunits) {
                step(I0{});
                if (!(cu < nunits)) break;
                step(I1{});
            }
        } else {
            int buf = 0;
            while (cu < nunits) {
                step(buf);
                buf ^= 1;
            }
        }
        if (log_n > 0) flush_log<false>(p, st, mylog, log_n, qid_s, qapp_s, p0, mywq, mywq + kWave, lh, jb_s);
        __syncthreads();
        local_refresh(lh, tau_s, jb_s, qn, w, p.R, st.hlo, st.hsh);
        // the item's histograms go to the global ones once per item (one atomic
        // per touched bin), not hit by hit
        merge_item_hist(st, lh, jb_s, qid_s, qn, w);
        publish_item(st, tau_s, qid_s, qn, w);
        refresh_tau_wave(st, qid_s, qapp_s, qn, w, kScanWaves, p.R);
        __syncthreads();
        par ^= 1;
    }
}

// ------------------------------------------------------------------ small-batch streaming scan
// For a handful of queries (at most kStreamMaxQ) the one-hot contraction would
// leave most of every 16-query MFMA tile empty and the scan is bound by
// streaming the codes from HBM.  Each thread then sums one row's table entries
// itself, by LDS lookups, while its next 16 code bytes load.  Table layouts
// (G queries per item):
//  * pair tables (kPair), indexed by a whole code byte (two blocks): G = 1:
//    int16 T[2p][lo] + T[2p+1][hi]; G = 2: a dword of both queries' pair sums
//    + 256 as 16-bit fields, added as one 32-bit word (at most 128 pairs
//    between folds into int32, so no field overflows);
//  * nibble tables, for tables too large as pairs: G = 1: the int8 entries;
//    G = 4: a dword of the four queries' entries + 128, the even and odd bytes
//    accumulated as 16-bit fields (at most 256 blocks between folds).
// An odd last block leaves the high nibble of its byte out of the pair sums.
// Absent queries' entries are the bias (value 0).  The tables run on with zero
// entries up to whole 16-byte code segments, so every segment of a row is
// summed in full whatever its padding bytes hold.  Items, thresholds, hit logs
// and flushes are those of the main kernel, with G queries per item; every
// flush also merges into the global histograms and refreshes the global
// thresholds, because every workgroup scans rows of the same few queries.
constexpr size_t kStreamMaxTable = 120 * 1024;  // LDS bytes for the table
constexpr int kStreamWaves = 12;               // one workgroup (and one table copy) per CU, 3 waves per SIMD
constexpr int kStreamThreads = kStreamWaves * kWave;

// 16 code bytes of a row from src.  The streaming kernel runs only on aligned
// rows (stride a multiple of 16 bytes), so the whole 16 bytes stay inside the
// row's stride.  (Nontemporal loads measured no faster on the tiled layout and
// much slower on row-major rows, whose lines the row's other segments reuse.)
__device__ __forceinline__ uint4 load_code16(const uint8_t* src) {
    return *reinterpret_cast<const uint4*>(src);
}

// Raises the item-local thresholds of all of an item's qn queries (one wave).
__device__ __forceinline__ void local_refresh_all(const uint32_t* lh, int32_t* tau_s, const int32_t* jb_s, int qn,
                                                  int R, int32_t hlo, int32_t hsh) {
    const int lane = lane_id();
    const int b = kLB - 1 - lane;
#pragma unroll 1
    for (int ql = 0; ql < qn; ++ql) {
        const int incl = wave_inclusive_sum((int)lh[ql * kLB + b]);
        const uint64_t mk = __ballot(incl >= R);
        if (mk && lane == __ffsll((unsigned long long)mk) - 1)
            atomicMax(&tau_s[ql], (int32_t)(hlo + ((int64_t)(jb_s[ql] + b) << hsh)));
    }
}

template <int G, bool kPair>
struct StreamAcc {
    int32_t s[G == 1 ? 1 : 4] = {};
    uint32_t f0 = 0, f1 = 0;  // packed 16-bit fields

    // segment j of 16 code bytes (32 blocks, or 16 pairs).  Lookups are issued
    // sixteen at a time before any is added, so they overlap.
    __device__ __forceinline__ void add(const unsigned char* tbl, int j, uint4 v) {
        constexpr int N = kPair ? 16 : 32;  // entries per segment
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < N; h += 16) {
            uint32_t x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int u = h + i;
                const uint32_t w32 = wd[u / (N / 4)];
                const int e = u % (N / 4);
                if (kPair) {
                    const int c = (int)((w32 >> (8 * e)) & 255u);
                    x[i] = G == 1 ? (uint32_t)(int32_t)reinterpret_cast<const int16_t*>(tbl)[(16 * j + u) * 256 + c]
                                  : reinterpret_cast<const uint32_t*>(tbl)[(16 * j + u) * 256 + c];
                } else {
                    const int c = (int)((w32 >> (4 * e)) & 15u);
                    x[i] = G == 1 ? (uint32_t)(int32_t)reinterpret_cast<const int8_t*>(tbl)[(32 * j + u) * 16 + c]
                                  : reinterpret_cast<const uint32_t*>(tbl)[(32 * j + u) * 16 + c];
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (G == 1) {
                    s[0] += (int32_t)x[i];
                } else if (kPair) {
                    f0 += x[i];
                } else {
                    f0 += x[i] & 0x00FF00FFu;
                    f1 += __builtin_amdgcn_perm(x[i], x[i], 0x0c030c01u);  // bytes 1 and 3 -> 16-bit fields
                }
            }
            // sixteen lookups in flight at a time: the empty asm keeps the
            // compiler from regrouping the adds of a whole row into one tree
            // (which holds every lookup of the row live and spills them)
            if (G == 1) asm volatile("" : "+v"(s[0]));
            else asm volatile("" : "+v"(f0), "+v"(f1));
        }
    }
    __device__ __forceinline__ void fold() {
        if (G == 1) return;
        s[0] += (int32_t)(f0 & 0xFFFFu);
        s[G == 2 ? 1 : 2] += (int32_t)(f0 >> 16);
        if (G == 4) {
            s[1] += (int32_t)(f1 & 0xFFFFu);
            s[3] += (int32_t)(f1 >> 16);
        }
        f0 = f1 = 0;
    }
};

// kSegs > 0: rows of exactly kSegs 16-byte segments stay whole in registers;
// kSegs = 0: longer rows stream through a ring of four segments.
template <int G, bool kPair, int kSegs>
__global__ __launch_bounds__(kStreamThreads) void scan_stream_kernel(MainArgs a) {
    constexpr int kCap = G * kWave + 128;  // log entries per wave: room for one batch of hits
    extern __shared__ __align__(16) unsigned char tbl[];  // the table; nibble entries staged after it
    __shared__ uint64_t log_s[kStreamWaves * kCap];
    __shared__ int32_t qid_s[kQG];  // flushes read kQG entries
    __shared__ uint32_t qapp_s[kQG];
    __shared__ uint32_t fl_s[kStreamWaves * 2 * kWave];
    __shared__ uint32_t lh[G * kLB];
    __shared__ uint32_t fh_s[kStreamWaves * G * kLB];  // per-wave flush histograms
    __shared__ int32_t tau_s[kQG];
    __shared__ int32_t jb_s[kQG];
    __shared__ int32_t off_s[kQG];  // residual variant: the item's leaf term per query (0 otherwise)
    __shared__ int64_t item_s, p0_s, p1_s, qbase_s;
    __shared__ int32_t qn_s;

    const Problem& p = a.p;
    const ScanState& st = a.st;
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int64_t n_items = p.leaves ? a.itemoff[p.L] : a.n_items;
    uint64_t* mylog = log_s + w * kCap;
    uint32_t* mywq = fl_s + w * 2 * kWave;
    uint32_t* myfh = fh_s + w * G * kLB;
    for (int e = lane; e < G * kLB; e += kWave) myfh[e] = 0;
    const int cb = (p.B + 1) / 2;     // code bytes per row (= pairs)
    const int nseg = kSegs > 0 ? kSegs : (cb + 15) / 16;  // 16-byte segments per row (the last may be partial)
    const int nent = kPair ? 16 * nseg : 32 * nseg;  // table rows (pairs or blocks), zero past cb or B
    const size_t tbl_bytes = kPair ? (size_t)nent * 256 * (G == 1 ? 2 : 4) : (size_t)nent * 16 * (G == 1 ? 1 : 4);
    int8_t* nib_s = reinterpret_cast<int8_t*>(tbl + ((tbl_bytes + 15) & ~(size_t)15));  // pair tables: G x B x 16

    int64_t claimed = 0;
    int64_t staged_qbase = -1;  // the query group whose table is in LDS
    int staged_qn = 0;
    if (tid == 0) claimed = (int64_t)atomicAdd(&st.ctrl[0], 1u);
    for (;;) {
        if (w == 0) fetch_item(a, claimed, n_items, &item_s, &p0_s, &p1_s, &qbase_s, &qn_s, nullptr);
        __syncthreads();
        const int64_t item = item_s;
        if (item >= n_items) break;
        const int64_t p0 = p0_s, p1 = p1_s;
        const int qn = qn_s;
        const bool restage = qbase_s != staged_qbase || qn != staged_qn;
        if (tid < kQG) {
            int32_t qq = 0;
            if (tid < qn) qq = p.leaves ? a.qlist[qbase_s + tid] : (int32_t)(qbase_s + tid);
            qid_s[tid] = qq;
            qapp_s[tid] = 0;
            off_s[tid] = (a.qbias && tid < qn) ? a.qbias[qbase_s + tid] : 0;
            const int32_t t = tid < qn ? ld_coherent(st.tau + qq) : INT_MAX;
            tau_s[tid] = t;
            jb_s[tid] = (t == INT_MIN || t == INT_MAX) ? 0 : hist_bin(t, st.hlo, st.hsh);
        }
        for (int e = tid; e < G * kLB; e += kStreamThreads) lh[e] = 0;
        __syncthreads();
        if (restage) {  // table staging (items of one query group reuse it)
            staged_qbase = qbase_s;
            staged_qn = qn;
            if (kPair) {
                for (int e = tid; e < G * p.B * 16; e += kStreamThreads) {
                    const int g = e / (p.B * 16), r = e - g * (p.B * 16);
                    nib_s[e] = g < qn ? p.lut[(int64_t)qid_s[g] * p.B * 16 + r] : (int8_t)0;
                }
                __syncthreads();
                for (int e = tid; e < nent * 256; e += kStreamThreads) {
                    const int pr = e >> 8, c = e & 255;
                    const bool hi = 2 * pr + 1 < p.B;
                    if (pr >= cb) {
                        if (G == 1) reinterpret_cast<int16_t*>(tbl)[e] = 0;
                        else reinterpret_cast<uint32_t*>(tbl)[e] = 0u;
                    } else if (G == 1) {
                        const int v = nib_s[(2 * pr) * 16 + (c & 15)] + (hi ? nib_s[(2 * pr + 1) * 16 + (c >> 4)] : 0);
                        reinterpret_cast<int16_t*>(tbl)[e] = (int16_t)v;
                    } else {
                        uint32_t x = 0;
#pragma unroll
                        for (int g = 0; g < 2; ++g) {
                            const int8_t* t = nib_s + g * p.B * 16;
                            const int v = t[(2 * pr) * 16 + (c & 15)] + (hi ? t[(2 * pr + 1) * 16 + (c >> 4)] : 0);
                            x |= (uint32_t)(v + 256) << (16 * g);
                        }
                        reinterpret_cast<uint32_t*>(tbl)[e] = x;
                    }
                }
            } else if (G == 1) {
                const int8_t* src = p.lut + (int64_t)qid_s[0] * p.B * 16;
                for (int e = tid; e < nent * 16; e += kStreamThreads)
                    tbl[e] = e < p.B * 16 ? (unsigned char)src[e] : (unsigned char)0;
            } else {
                for (int e = tid; e < nent * 16; e += kStreamThreads) {
                    uint32_t x = 0;
#pragma unroll
                    for (int g = 0; g < G && e < p.B * 16; ++g) {
                        const int32_t t = g < qn ? (int32_t)p.lut[(int64_t)qid_s[g] * p.B * 16 + e] : 0;
                        x |= (uint32_t)(t + 128) << (8 * g);
                    }
                    reinterpret_cast<uint32_t*>(tbl)[e] = x;
                }
            }
            __syncthreads();
        }

        int log_n = 0;
        // appends a wave's log, raises the item's thresholds from its
        // histogram, merges the flush into the global histograms and refreshes
        // the global thresholds (every workgroup scans rows of the same few
        // queries, so they all profit at once)
        auto flush_publish = [&](int n) {
            flush_log<false>(p, st, mylog, n, qid_s, qapp_s, p0, mywq, mywq + kWave, lh, jb_s, myfh);
            local_refresh_all(lh, tau_s, jb_s, qn, p.R, st.hlo, st.hsh);
            merge_flush(st, myfh, jb_s, qid_s, qn);
            if (lane < qn) atomicMax(st.tau + qid_s[lane], tau_s[lane]);
            refresh_tau_wave(st, qid_s, qapp_s, qn, 0, 1, p.R, tau_s);
        };
        // thresholds, sums of the G queries for the lane's row, then the filter
        auto finish_row = [&](int64_t row, const StreamAcc<G, kPair>& acc) {
            const bool valid = row < p1;
            // residual variant: a row scores its sum plus the item's leaf term,
            // so the sum is tested against the threshold minus that term
            int32_t tq[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                tq[g] = g < qn ? tau_s[g] : INT_MAX;
                if (a.qbias) tq[g] = sat_sub(tq[g], off_s[g]);
            }
            int32_t sum[G];
#pragma unroll
            for (int g = 0; g < G; ++g)
                sum[g] = G == 1 ? acc.s[0] : acc.s[g] - (kPair ? 256 * cb : 128 * p.B);
            if (log_n > kCap - G * kWave) {
                flush_publish(log_n);
                log_n = 0;
            }
            const uint32_t lr = (uint32_t)(row - p0);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const bool hit = valid && sum[g] >= tq[g];
                const uint64_t mk = __ballot(hit);
                if (mk) {
                    if (hit)
                        mylog[log_n + __popcll(mk & lanemask_lt())] =
                            ((uint64_t)(uint32_t)(sum[g] + (a.qbias ? off_s[g] : 0)) << 32) |
                            ((uint64_t)g << 16) | (uint64_t)lr;
                    log_n += __popcll(mk);
                }
            }
        };
        const int64_t rb0 = p0 + w * kWave;
        const int32_t ss = seg_step(p);
        if (kSegs > 0) {
            // whole rows in registers; the next batch's rows load while this
            // batch's are summed.  Every load is unconditional (rows past the
            // item read the last valid one), so the compiler can wait for
            // exactly the loads it needs.
            auto load_row = [&](int64_t rb, uint4* r) {
                const int64_t row = rb + lane;
                const uint8_t* src = code_row(p, row < p1 ? row : p1 - 1);
#pragma unroll
                for (int j = 0; j < kSegs; ++j) r[j] = load_code16(src + j * ss);
            };
            auto batch = [&](int64_t rb, const uint4* r, uint4* nr) {
                load_row(rb + kStreamThreads, nr);
                StreamAcc<G, kPair> acc;
#pragma unroll
                for (int j = 0; j < kSegs; ++j) acc.add(tbl, j, r[j]);
                acc.fold();
                finish_row(rb + lane, acc);
            };
            uint4 ra[kSegs > 0 ? kSegs : 1], rbuf[kSegs > 0 ? kSegs : 1];
            load_row(rb0, ra);
            for (int64_t rb = rb0; rb < p1; rb += 2 * kStreamThreads) {
                batch(rb, ra, rbuf);
                if (rb + kStreamThreads >= p1) break;
                batch(rb + kStreamThreads, rbuf, ra);
            }
        } else {
            // long rows: a ring of four segments in flight within the row
            for (int64_t rb = rb0; rb < p1; rb += kStreamThreads) {
                const int64_t row = rb + lane;
                const uint8_t* src = code_row(p, row < p1 ? row : p1 - 1);
                uint4 ring[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (k < nseg) ring[k] = load_code16(src + k * ss);
                StreamAcc<G, kPair> acc;
                for (int j0 = 0; j0 < nseg; j0 += 4) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int j = j0 + k;
                        if (j >= nseg) break;
                        const uint4 v = ring[k];
                        if (j + 4 < nseg) ring[k] = load_code16(src + (j + 4) * ss);
                        acc.add(tbl, j, v);
                        if (j % 8 == 7) acc.fold();  // 128 pairs, or 256 blocks
                    }
                }
                acc.fold();
                finish_row(row, acc);
            }
        }
        if (log_n > 0) {
            flush_log<false>(p, st, mylog, log_n, qid_s, qapp_s, p0, mywq, mywq + kWave, lh, jb_s, myfh);
            merge_flush(st, myfh, jb_s, qid_s, qn);
        }
        __syncthreads();
        local_refresh(lh, tau_s, jb_s, qn, w, p.R, st.hlo, st.hsh);
        publish_item(st, tau_s, qid_s, qn, w);
        refresh_tau_wave(st, qid_s, qapp_s, qn, w, kScanWaves, p.R);
        __syncthreads();
    }
}

// LDS bytes of the streaming kernel's dynamic area (0: the variant does not fit).
static size_t stream_lds(int G, bool pair, int32_t B) {
    const size_t cb = (size_t)(B + 1) / 2, nseg = (cb + 15) / 16;  // tables padded to whole segments
    const size_t t = pair ? 16 * nseg * 256 * (G == 1 ? 2 : 4) : 32 * nseg * 16 * (G == 1 ? 1 : 4);
    const size_t extra = pair ? (size_t)G * B * 16 : 0;
    const size_t total = ((t + 15) & ~(size_t)15) + extra;
    return total <= kStreamMaxTable ? total : 0;
}

// ------------------------------------------------------------------ one-wave warm-up and selection
// Four queries per 256-thread workgroup, one wave each and no workgroup
// barrier, for the common sizes: the warm-up when the query's table fits in
// kWaveLut bytes; the final selection when at most kWaveKeys candidates reach
// the query's threshold (others are deferred to the workgroup kernel).
constexpr int kWaveKeys = 1024;
constexpr int kWaveLut = 4096;
constexpr int kFineShift = 8;                 // fine histogram of the final selection: 256 bins
constexpr int kFineBins = 1 << kFineShift;

// The warm-up threshold here is the lower edge of the histogram bin holding the
// R-th best of the W sums (a valid bound, at most one bin below the exact R-th
// best): one histogram instead of a sort.
__global__ __launch_bounds__(kSelThreads) void warmup_wave_kernel(Problem p, ScanState st, int32_t W) {
    __shared__ __align__(16) int8_t lut_all[4][kWaveLut];
    __shared__ uint32_t hist_all[4][kNB];
    const int w = threadIdx.x / kWave, lane = lane_id();
    const int64_t q = (int64_t)blockIdx.x * 4 + w;
    if (q == 0 && lane < 16) st.ctrl[lane] = 0;
    if (q >= p.nq) return;
    int8_t* lut_s = lut_all[w];
    uint32_t* hw_s = hist_all[w];
    // blocks padded with zeros to whole 16-byte code segments (32 blocks), so a
    // row's segments are summed without per-block tests
    const int nseg = ((p.B + 1) / 2 + 15) / 16;
    stage_table_cm(lut_s, p.lut + q * p.B * 16, p.B, 32 * nseg, lane, kWave);
    const int32_t S = tstride(32 * nseg);
    for (int j = lane; j < kNB; j += kWave) st.hist[q * kNB + j] = 0;
    if (lane == 0) {
        st.cnt[q] = 0;
        st.hmax[q] = 0;
    }
    const bool al4 = (p.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(p.codes) & 3) == 0;
    // 16-byte aligned rows (then the stride holds every 16-byte segment of the codes)
    const bool al16 = (p.stride & 15) == 0 && (reinterpret_cast<uintptr_t>(p.codes) & 15) == 0;
    for (int j = lane; j < kNB; j += kWave) hw_s[j] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int64_t got = 0;
    const int nsrc = p.leaves ? p.nl : 1;
    for (int j = 0; j < nsrc && got < W; ++j) {
        int64_t a, b;
        if (p.leaves) {
            const int32_t l = p.leaves[q * p.nl + j];
            const bool okl = l >= 0 && l < p.L;
            a = okl ? p.leaf_offsets[l] : 0;
            b = okl ? p.leaf_offsets[l + 1] : 0;
        } else {
            a = 0;
            b = p.n;
        }
        const int64_t take = b - a < W - got ? b - a : W - got;
        const int32_t off = p.leaves ? leaf_bias_at(p, q, j) : 0;
        const int32_t ss = seg_step(p);
        if (al16) {
            // the whole row's code bytes (at most 8 x 16) in registers, the
            // lane's next row loading while this one is summed (two buffers,
            // alternating; rows past the range read its last row, unused)
            constexpr int kS = kWaveLut / 512;
            auto load = [&](int64_t t, uint4* r) {
                const uint8_t* src = code_row(p, a + (t < take ? t : take - 1));
#pragma unroll
                for (int j = 0; j < kS; ++j)
                    if (j < nseg) r[j] = *reinterpret_cast<const uint4*>(src + j * ss);
            };
            auto sum = [&](int64_t t, const uint4* r, uint4* nr) {
                load(t + kWave, nr);
                if (t >= take) return;
                int32_t sv = off;
#pragma unroll
                for (int j = 0; j < kS; ++j) {
                    if (j >= nseg) break;
                    const uint32_t wd[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
                    for (int u = 0; u < 32; ++u)
                        sv += lut_s[(int)((wd[u >> 3] >> (4 * (u & 7))) & 15u) * S + 32 * j + u];
                }
                atomicAdd(&hw_s[hist_bin(sv, st.hlo, st.hsh)], 1u);
            };
            if (take > 0) {
                uint4 ra[kS], rb[kS];
                load(lane, ra);
                for (int64_t t0 = 0; t0 < take; t0 += 2 * kWave) {
                    sum(t0 + lane, ra, rb);
                    if (t0 + kWave >= take) break;
                    sum(t0 + kWave + lane, rb, ra);
                }
            }
        } else {
            for (int64_t t = lane; t < take; t += kWave) {
                const int32_t sv = off + row_sum(lut_s, p.B, S, code_row(p, a + t), al4, ss);
                atomicAdd(&hw_s[hist_bin(sv, st.hlo, st.hsh)], 1u);
            }
        }
        got += take;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // the highest bin edge with at least R sums at or above it: lane l owns
    // the 16 bins from the top 16 l down
    if (got < p.R) {
        if (lane == 0) st.tau[q] = INT_MIN;
        return;
    }
    int c[16], tot = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        c[k] = (int)hw_s[kNB - 1 - 16 * lane - k];
        tot += c[k];
    }
    const int incl = wave_inclusive_sum(tot);
    const uint64_t mk = __ballot(incl >= p.R);
    const int l = __ffsll((unsigned long long)mk) - 1;  // got >= R, so some lane reaches R
    if (lane == l) {
        int cum = incl - tot, bin = kNB - 1 - 16 * lane;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            cum += c[k];
            if (cum >= p.R) {
                bin = kNB - 1 - 16 * lane - k;
                break;
            }
        }
        st.tau[q] = (int32_t)(st.hlo + ((int64_t)bin << st.hsh));
    }
}

__global__ __launch_bounds__(kSelThreads) void final_select_wave_kernel(Problem p, ScanState st) {
    __shared__ uint64_t stage_all[4][kWaveKeys];
    __shared__ uint32_t fine_all[4][kFineBins];
    const int w = threadIdx.x / kWave, lane = lane_id();
    const int64_t q = (int64_t)blockIdx.x * 4 + w;
    if (q >= p.nq) return;
    const uint32_t total = st.cnt[q];
    if ((int64_t)total > st.cap) {
        if (lane == 0) st.ovf[atomicAdd(&st.ctrl[1], 1u)] = (int32_t)q;
        return;
    }
    // tau first raised to the highest edge of the query's histogram with at
    // least R appended sums at or above it (items publish only their own)
    refresh_tau(st, (int)q, p.R);
    const int32_t tau = ld_coherent(st.tau + q);
    const uint64_t* list = st.cand + q * st.cap;
    uint64_t* stage = stage_all[w];
    uint32_t* fine = fine_all[w];
    // The list's keys at or above tau are staged while they fit.  Alongside,
    // the scores in [tau, tau + kFineBins * fw) go into a fine histogram (fw:
    // the scan histogram's bin width / kFineBins, at least 1) and the keys
    // above that range are counted, so that when too many keys reach tau a
    // higher threshold t2 can be read off with at least R keys at or above it.
    const int32_t fsh = st.hsh > kFineShift ? st.hsh - kFineShift : 0;
    const int64_t ftop = (int64_t)tau + ((int64_t)kFineBins << fsh);
    for (int j = lane; j < kFineBins; j += kWave) fine[j] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // the list is read in rounds of 8 keys per lane, all loads of a round
    // issued before any key is used (every lane runs every call of f: f may
    // take ballots)
    auto for_keys = [&](auto f) {
        for (uint32_t b0 = 0; b0 < total; b0 += 8 * kWave) {
            uint64_t kk[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t i = b0 + r * kWave + lane;
                kk[r] = i < total ? list[i] : 0;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) f(kk[r]);
        }
    };
    int n = 0;        // keys at or above tau
    int n_high = 0;   // keys at or above ftop
    int32_t smax = INT_MIN;  // this lane's best score at or above tau
    for_keys([&](const uint64_t k) {
        const int32_t sc = key_int_score(k);
        const bool keep = k != 0 && sc >= tau;
        const uint64_t mk = __ballot(keep);
        const int pos = n + __popcll(mk & lanemask_lt());
        if (keep && pos < kWaveKeys) stage[pos] = k;
        n += __popcll(mk);
        const bool high = keep && (int64_t)sc >= ftop;
        n_high += __popcll(__ballot(high));
        if (keep && !high && tau != INT_MIN) atomicAdd(&fine[((int64_t)sc - tau) >> fsh], 1u);
        if (keep && sc > smax) smax = sc;
    });
    if (n > kWaveKeys) {
        // t2: the lower edge of the fine bin holding the R-th best key (n2
        // keys at or above it), read from the fine histogram of [lo, lo +
        // kFineBins << sh) with `above` keys above that range
        auto pick = [&](int64_t lo, int32_t sh, int above, int& n2, int32_t& t2) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            n2 = -1;
            int acc = above;
            for (int top = kFineBins - 1; top >= 0 && n2 < 0; top -= kWave) {
                const int j = top - lane;
                const int c = j >= 0 ? (int)fine[j] : 0;
                const int incl = acc + wave_inclusive_sum(c);
                const uint64_t mk = __ballot(j >= 0 && incl >= p.R);
                if (mk) {
                    const int l = __ffsll((unsigned long long)mk) - 1;
                    n2 = __shfl(incl, l);
                    t2 = (int32_t)(lo + ((int64_t)(top - l) << sh));
                }
                acc = __shfl(incl, kWave - 1);
            }
        };
        int n2 = -1;
        int32_t t2 = tau;
        if (tau != INT_MIN && n_high < p.R) {
            pick(tau, fsh, n_high, n2, t2);
        } else if (tau != INT_MIN) {
            // at least R keys lie above the first fine range (the histogram
            // that set tau counts some sums in lower bins than their own): a
            // second fine histogram over [ftop, the best score]
            for (int o = 1; o < kWave; o <<= 1) {
                const int32_t v = __shfl_xor(smax, o);
                smax = v > smax ? v : smax;
            }
            int32_t sh2 = 0;
            while (((int64_t)kFineBins << sh2) < (int64_t)smax - ftop + 1) ++sh2;
            for (int j = lane; j < kFineBins; j += kWave) fine[j] = 0;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            for_keys([&](const uint64_t k) {
                const int32_t sc = key_int_score(k);
                if (k != 0 && (int64_t)sc >= ftop) atomicAdd(&fine[((int64_t)sc - ftop) >> sh2], 1u);
            });
            pick(ftop, sh2, 0, n2, t2);
        }
        if (n2 < 0 || n2 > kWaveKeys) {
            if (lane == 0) st.dfr[atomicAdd(&st.ctrl[3], 1u)] = (int32_t)q;
            return;
        }
        // stage again: the n2 keys at or above t2
        n = 0;
        for_keys([&](const uint64_t k) {
            const bool keep = k != 0 && key_int_score(k) >= t2;
            const uint64_t mk = __ballot(keep);
            const int pos = n + __popcll(mk & lanemask_lt());
            if (keep && pos < kWaveKeys) stage[pos] = k;
            n += __popcll(mk);
        });
    }
    const int P = next_pow2(n > 0 ? n : 1);
    for (int j = n + lane; j < P; j += kWave) stage[j] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    wave_bitonic_sort_desc(stage, P);
    const int m = n < p.R ? n : p.R;
    for (int r = lane; r < p.R; r += kWave) {
        const uint64_t k = r < m ? stage[r] : 0;
        p.out_ids[q * p.R + r] = r < m ? key_id(k) : -1;
        p.out_scores[q * p.R + r] = r < m ? key_int_score(k) : INT_MIN;
    }
}

// The same selection by one 16-wave workgroup per query, for batches of a few
// queries: every workgroup of the scan appends to their lists, which grow long,
// and reading a long list one wave at a time is a chain of round trips.  Here
// the list is read by all 16 waves at once (8 keys per thread and round); the
// staged keys are sorted by the whole workgroup.
constexpr int kFewThreads = 1024;
constexpr int kFewMaxQ = 64;  // batches up to this many queries take this kernel

__global__ __launch_bounds__(kFewThreads) void final_select_few_kernel(Problem p, ScanState st) {
    __shared__ uint64_t stage[kWaveKeys];
    __shared__ uint32_t fine[kFineBins];
    __shared__ int32_t tau_s, t2_s, smax_s;
    __shared__ int n_s, nh_s, n2_s;
    const int tid = threadIdx.x, lane = lane_id();
    const int64_t q = blockIdx.x;
    const uint32_t total = st.cnt[q];
    if ((int64_t)total > st.cap) {
        if (tid == 0) st.ovf[atomicAdd(&st.ctrl[1], 1u)] = (int32_t)q;
        return;
    }
    if (tid < kWave) {
        refresh_tau(st, (int)q, p.R);
        const int32_t t = ld_coherent(st.tau + q);
        if (lane == 0) {
            tau_s = t;
            n_s = 0;
            nh_s = 0;
            smax_s = INT_MIN;
        }
    }
    for (int j = tid; j < kFineBins; j += kFewThreads) fine[j] = 0;
    __syncthreads();
    const int32_t tau = tau_s;
    const uint64_t* list = st.cand + q * st.cap;
    const int32_t fsh = st.hsh > kFineShift ? st.hsh - kFineShift : 0;
    const int64_t ftop = (int64_t)tau + ((int64_t)kFineBins << fsh);
    // rounds of 8 keys per thread, every load of a round issued before any key
    // is used; the keys of a round that pass `keep` go to consecutive stage
    // slots (one LDS atomic per wave and round)
    auto for_keys = [&](auto keep, auto f) {
        for (uint32_t b0 = 0; b0 < total; b0 += 8 * kFewThreads) {
            uint64_t kk[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t i = b0 + r * kFewThreads + tid;
                kk[r] = i < total ? list[i] : 0;
            }
            uint64_t mk[8];
            int cnt = 0;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                mk[r] = __ballot(keep(kk[r]));
                cnt += __popcll(mk[r]);
            }
            if (cnt == 0) continue;  // wave-uniform
            int base = 0;
            if (lane == 0) base = atomicAdd(&n_s, cnt);
            base = __shfl(base, 0, kWave);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const bool kp = (mk[r] >> lane) & 1;
                const int pos = base + __popcll(mk[r] & lanemask_lt());
                if (kp && pos < kWaveKeys) stage[pos] = kk[r];
                base += __popcll(mk[r]);
                if (kp) f(kk[r]);
            }
        }
    };
    int n_high = 0;
    int32_t smax = INT_MIN;
    for_keys([&](uint64_t k) { return k != 0 && key_int_score(k) >= tau; },
             [&](uint64_t k) {
                 const int32_t sc = key_int_score(k);
                 if ((int64_t)sc >= ftop) ++n_high;
                 else if (tau != INT_MIN) atomicAdd(&fine[((int64_t)sc - tau) >> fsh], 1u);
                 smax = sc > smax ? sc : smax;
             });
    if (n_high) atomicAdd(&nh_s, n_high);
    if (smax != INT_MIN) atomicMax(&smax_s, smax);
    __syncthreads();
    int n = n_s;
    if (n > kWaveKeys) {
        // t2: the lower edge of the fine bin holding the R-th best key (n2
        // keys at or above it), read by wave 0 from the fine histogram of
        // [lo, lo + kFineBins << sh) with `above` keys above that range
        auto pick = [&](int64_t lo, int32_t sh, int above) {
            if (tid >= kWave) return;
            int n2 = -1;
            int32_t t2 = tau;
            int acc = above;
            for (int top = kFineBins - 1; top >= 0 && n2 < 0; top -= kWave) {
                const int j = top - lane;
                const int c = j >= 0 ? (int)fine[j] : 0;
                const int incl = acc + wave_inclusive_sum(c);
                const uint64_t mk = __ballot(j >= 0 && incl >= p.R);
                if (mk) {
                    const int l = __ffsll((unsigned long long)mk) - 1;
                    n2 = __shfl(incl, l);
                    t2 = (int32_t)(lo + ((int64_t)(top - l) << sh));
                }
                acc = __shfl(incl, kWave - 1);
            }
            if (lane == 0) {
                n2_s = n2;
                t2_s = t2;
            }
        };
        const int nh = nh_s;
        if (tid == 0) n2_s = -1;
        __syncthreads();
        if (tau != INT_MIN && nh < p.R) {
            pick(tau, fsh, nh);
        } else if (tau != INT_MIN) {
            // at least R keys lie above the first fine range: a second fine
            // histogram over [ftop, the best score]
            const int32_t sm = smax_s;
            int32_t sh2 = 0;
            while (((int64_t)kFineBins << sh2) < (int64_t)sm - ftop + 1) ++sh2;
            for (int j = tid; j < kFineBins; j += kFewThreads) fine[j] = 0;
            __syncthreads();
            for (uint32_t b0 = 0; b0 < total; b0 += 8 * kFewThreads) {
                uint64_t kk[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const uint32_t i = b0 + r * kFewThreads + tid;
                    kk[r] = i < total ? list[i] : 0;
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int32_t sc = key_int_score(kk[r]);
                    if (kk[r] != 0 && (int64_t)sc >= ftop) atomicAdd(&fine[((int64_t)sc - ftop) >> sh2], 1u);
                }
            }
            __syncthreads();
            pick(ftop, sh2, 0);
        }
        __syncthreads();
        const int n2 = n2_s;
        const int32_t t2 = t2_s;
        if (n2 < 0 || n2 > kWaveKeys) {
            if (tid == 0) st.dfr[atomicAdd(&st.ctrl[3], 1u)] = (int32_t)q;
            return;
        }
        // stage again: the n2 keys at or above t2
        if (tid == 0) n_s = 0;
        __syncthreads();
        for_keys([&](uint64_t k) { return k != 0 && key_int_score(k) >= t2; }, [](uint64_t) {});
        __syncthreads();
        n = n_s;
        if (n > kWaveKeys) {  // (the count n2 says it cannot happen)
            if (tid == 0) st.dfr[atomicAdd(&st.ctrl[3], 1u)] = (int32_t)q;
            return;
        }
    }
    const int P = next_pow2(n > 0 ? n : 1);
    for (int j = n + tid; j < P; j += kFewThreads) stage[j] = 0;
    __syncthreads();
    // bitonic sort, descending, one compare-exchange per thread and step
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (P >> 1); i += kFewThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t x = stage[lo], y = stage[hi];
                if ((x < y) == desc) {
                    stage[lo] = y;
                    stage[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    const int m = n < p.R ? n : p.R;
    for (int r = tid; r < p.R; r += kFewThreads) {
        const uint64_t k = r < m ? stage[r] : 0;
        p.out_ids[q * p.R + r] = r < m ? key_id(k) : -1;
        p.out_scores[q * p.R + r] = r < m ? key_int_score(k) : INT_MIN;
    }
}

// ------------------------------------------------------------------ final selection
// The workgroup selection, for the queries the one-wave kernel deferred
// (workgroup i takes the i-th of them; the list has ctrl[3] entries).
__global__ __launch_bounds__(kSelThreads) void final_select_kernel(Problem p, ScanState st) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ SelectShared sh;
    __shared__ uint32_t nst;
    if (blockIdx.x >= st.ctrl[3]) return;
    const int64_t q = st.dfr[blockIdx.x];
    const int tid = threadIdx.x;
    const uint32_t total = st.cnt[q];
    const int32_t tau = st.tau[q];
    const uint64_t* list = st.cand + q * st.cap;
    uint64_t* stage = reinterpret_cast<uint64_t*>(smem);
    uint64_t* sel = stage + kSelLds;
    if (tid == 0) nst = 0;
    __syncthreads();
    uint32_t mine = 0;
    for (uint32_t i = tid; i < total; i += kSelThreads) mine += key_int_score(list[i]) >= tau;
    atomicAdd(&nst, mine);
    __syncthreads();
    const uint32_t above = nst;
    int m;
    if (above <= (uint32_t)kSelLds) {
        __syncthreads();
        if (tid == 0) nst = 0;
        __syncthreads();
        for (uint32_t i = tid; i < total; i += kSelThreads) {
            const uint64_t k = list[i];
            if (key_int_score(k) >= tau) stage[atomicAdd(&nst, 1u)] = k;
        }
        __syncthreads();
        m = wg_select_topk<kSelThreads>(LdsKeys{stage}, above, p.R, sh, sel);
    } else {
        m = wg_select_topk<kSelThreads>(GlobalKeysAbove{list, tau}, total, p.R, sh, sel);
    }
    for (int r = tid; r < p.R; r += kSelThreads) {
        p.out_ids[q * p.R + r] = r < m ? key_id(sel[r]) : -1;
        p.out_scores[q * p.R + r] = r < m ? key_int_score(sel[r]) : INT_MIN;
    }
}

// ------------------------------------------------------------------ overflow fallback
// A query whose candidate list overflowed is recomputed exactly: every scanned
// row's key into a private scratch slot, then the exact selection.  Persistent
// workgroups take overflowed queries from the list until it is exhausted.
__global__ __launch_bounds__(kSelThreads) void fallback_kernel(Problem p, ScanState st) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ SelectShared sh;
    __shared__ uint32_t item;
    const int tid = threadIdx.x;
    uint64_t* sel = reinterpret_cast<uint64_t*>(smem);
    int8_t* lut_s = reinterpret_cast<int8_t*>(sel + next_pow2(p.R));
    uint64_t* scratch = st.fb + (int64_t)blockIdx.x * (p.n > 0 ? p.n : 1);
    const bool al4 = (p.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(p.codes) & 3) == 0;
    for (;;) {
        if (tid == 0) item = atomicAdd(&st.ctrl[2], 1u);
        __syncthreads();
        const uint32_t it = item;
        if (it >= ld_coherent(&st.ctrl[1])) break;
        const int64_t q = st.ovf[it];
        stage_table_cm(lut_s, p.lut + q * p.B * 16, p.B, p.B, tid, kSelThreads);
        __syncthreads();
        int64_t m = 0;
        const int nsrc = p.leaves ? p.nl : 1;
        for (int j = 0; j < nsrc; ++j) {
            int64_t a, b;
            if (p.leaves) {
                const int32_t l = p.leaves[q * p.nl + j];
                const bool okl = l >= 0 && l < p.L;
                a = okl ? p.leaf_offsets[l] : 0;
                b = okl ? p.leaf_offsets[l + 1] : 0;
            } else {
                a = 0;
                b = p.n;
            }
            if (b - a > p.n - m) b = a + (p.n - m);
            const int32_t off = p.leaves ? leaf_bias_at(p, q, j) : 0;
            for (int64_t t = tid; t < b - a; t += kSelThreads) {
                const int64_t row = a + t;
                scratch[m + t] = int_key(row_sum(lut_s, p.B, tstride(p.B), code_row(p, row), al4, seg_step(p)) + off,
                                         p.ids ? p.ids[row] : (int32_t)row);
            }
            m += b - a;
        }
        __syncthreads();
        const int k = wg_select_topk<kSelThreads>(LdsKeys{scratch}, m, p.R, sh, sel);
        for (int r = tid; r < p.R; r += kSelThreads) {
            p.out_ids[q * p.R + r] = r < k ? key_id(sel[r]) : -1;
            p.out_scores[q * p.R + r] = r < k ? key_int_score(sel[r]) : INT_MIN;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ host side
template <typename K>
static void allow_lds(K kernel, size_t bytes) {
    if (bytes > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int G, bool kPair, int kSegs>
static void launch_stream1(int grid, size_t lds, hipStream_t stream, const MainArgs& ma) {
    allow_lds(scan_stream_kernel<G, kPair, kSegs>, lds);
    hipLaunchKernelGGL((scan_stream_kernel<G, kPair, kSegs>), dim3(grid), dim3(kStreamThreads), lds, stream, ma);
}

// Rows of 1 to 6 segments of 16 code bytes whole in registers (the count a
// compile-time constant, so the loads and their waits follow a fixed pattern),
// longer rows through the ring.
template <int G, bool kPair>
static void launch_stream(int nseg, int grid, size_t lds, hipStream_t stream, const MainArgs& ma) {
    switch (nseg) {
        case 1: launch_stream1<G, kPair, 1>(grid, lds, stream, ma); break;
        case 2: launch_stream1<G, kPair, 2>(grid, lds, stream, ma); break;
        case 3: launch_stream1<G, kPair, 3>(grid, lds, stream, ma); break;
        case 4: launch_stream1<G, kPair, 4>(grid, lds, stream, ma); break;
        case 5: launch_stream1<G, kPair, 5>(grid, lds, stream, ma); break;
        case 6: launch_stream1<G, kPair, 6>(grid, lds, stream, ma); break;
        default: launch_stream1<G, kPair, 0>(grid, lds, stream, ma); break;
    }
}

static int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    return cus;
}

hipError_t launch_scan(const ScanProblem& sp, void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t main_start,
                       hipEvent_t main_stop) {
    (void)ws_bytes;
    if (sp.nq == 0) return hipSuccess;
    const ScanLayout lay = scan_layout(sp.nq, sp.B, sp.n, sp.L, sp.nl, sp.R);
    char* base = reinterpret_cast<char*>(ws);
    const bool biased = sp.leaf_bias != nullptr && sp.leaves != nullptr;
    Problem p{sp.lut, sp.nq, sp.B, sp.codes, sp.stride, sp.n, sp.ids, sp.leaf_offsets, sp.L,
              sp.leaves, sp.nl, sp.R, sp.out_ids, sp.out_scores, sp.tile_bytes,
              biased ? sp.leaf_bias : nullptr, biased ? sp.bias_bound : 0};
    ScanState st{};
    st.tau = reinterpret_cast<int32_t*>(base + lay.tau);
    st.cnt = reinterpret_cast<uint32_t*>(base + lay.cnt);
    st.hmax = reinterpret_cast<uint32_t*>(base + lay.hmax);
    st.hist = reinterpret_cast<uint32_t*>(base + lay.hist);
    st.cand = reinterpret_cast<uint64_t*>(base + lay.cand);
    st.ctrl = reinterpret_cast<uint32_t*>(base + lay.ctrl);
    st.ovf = reinterpret_cast<int32_t*>(base + lay.ovf);
    st.dfr = reinterpret_cast<int32_t*>(base + lay.dfr);
    st.fb = reinterpret_cast<uint64_t*>(base + lay.fb);
    st.cap = lay.cap;
    // every sum lies in [-128 B, 127 B] (residual variant: widened by the bias
    // bound on both sides), so no score falls below bin 0's edge
    const int32_t bb = biased ? sp.bias_bound : 0;
    st.hlo = -128 * sp.B - bb;
    {
        const int64_t need = (255LL * sp.B + 2LL * bb + 1 + kNB - 1) / kNB;
        int32_t sh = 0;
        while ((1LL << sh) < need) ++sh;
        st.hsh = sh;
        st.hw = 1 << sh;
    }
    const bool part = sp.leaves != nullptr;
    hipError_t e;

    MainArgs ma{};
    ma.p = p;
    ma.st = st;
    const int32_t B8 = (sp.B + 7) & ~7;
    ma.nkstep = B8 / 4;
    // tables up to 64 blocks stay resident for an item; larger ones are staged
    // through LDS 32 blocks at a time
    ma.nchunk = ma.nkstep <= kKC ? 1 : (ma.nkstep + kKCS - 1) / kKCS;
    // small batches stream the codes through VALU lookups: one query, or two
    // per item, by byte-pair tables; else one or four per item by nibble
    // tables; larger batches use the MFMA kernel with 64 queries per item
    int sg = 0;
    bool spair = false;
    size_t stbl = 0;
    const bool aligned = (sp.stride % 16) == 0 && (reinterpret_cast<uintptr_t>(sp.codes) & 15) == 0;
    if (sp.nq >= 1 && sp.nq <= kStreamMaxQ && aligned) {
        const int gp = sp.nq == 1 ? 1 : 2, gn = sp.nq == 1 ? 1 : 4;
        if ((stbl = stream_lds(gp, true, sp.B)) != 0) {
            sg = gp;
            spair = true;
        } else if ((stbl = stream_lds(gn, false, sp.B)) != 0) {
            sg = gn;
        }
    }
    const bool streaming = sg != 0;
    ma.qg = streaming ? sg : kQG;
    ma.nqg = (int32_t)((sp.nq + ma.qg - 1) / ma.qg);
    // the MFMA kernel's items are kItemPts rows.  A full streaming scan is cut
    // into about three items per CU (fewer item ends, at which a workgroup's
    // loads stop while its waves flush; still some balancing); a partitioned
    // one into items small enough that every CU gets at least two.
    ma.item_pts = kItemPts;
    if (streaming && !part) {
        const int64_t want = 3LL * device_cus();
        const int64_t chunks = (want + ma.nqg - 1) / ma.nqg;
        int64_t pts = (sp.n + chunks - 1) / chunks;
        pts = (pts + 63) & ~(int64_t)63;  // whole 64-row tiles
        if (pts < 1024) pts = 1024;
        if (pts > 65536) pts = 65536;     // row offsets within an item fit the log's 16 bits
        ma.item_pts = (int32_t)pts;
    } else if (streaming) {
        const int64_t rows = (sp.n * sp.nl + sp.L - 1) / (sp.L > 0 ? sp.L : 1);  // rows per query group, roughly
        while (ma.item_pts > 1024 && (int64_t)ma.nqg * ((rows + ma.item_pts - 1) / ma.item_pts) < 2LL * device_cus())
            ma.item_pts >>= 1;
    }
    ma.n_items = (int64_t)ma.nqg * ((sp.n + ma.item_pts - 1) / ma.item_pts);
    ma.fast_codes = (sp.stride % 16) == 0 && (reinterpret_cast<uintptr_t>(sp.codes) & 15) == 0;
    if (part) {
        uint32_t* lcnt = reinterpret_cast<uint32_t*>(base + lay.lcnt);
        uint32_t* lcur = reinterpret_cast<uint32_t*>(base + lay.lcur);
        int32_t* lqoff = reinterpret_cast<int32_t*>(base + lay.lqoff);
        int32_t* qlist = reinterpret_cast<int32_t*>(base + lay.qlist);
        int32_t* qbias = reinterpret_cast<int32_t*>(base + lay.qbias);
        int64_t* itemoff = reinterpret_cast<int64_t*>(base + lay.itemoff);
        hipLaunchKernelGGL(zero_u32_kernel, dim3(64), dim3(256), 0, stream, lcnt, (int64_t)sp.L);
        hipLaunchKernelGGL(zero_u32_kernel, dim3(64), dim3(256), 0, stream, lcur, (int64_t)sp.L);
        const int64_t pairs = sp.nq * sp.nl;
        const unsigned gb = (unsigned)((pairs + 255) / 256 < 4096 ? (pairs + 255) / 256 : 4096);
        const bool lds = sp.L <= kLeafLds;
        const unsigned gc = (unsigned)((pairs + kLeafChunk - 1) / kLeafChunk);
        const size_t lbytes = (size_t)sp.L * 4;
        if (lds) {
            allow_lds(leaf_count_lds_kernel, lbytes);
            allow_lds(leaf_scatter_lds_kernel, lbytes);
            hipLaunchKernelGGL(leaf_count_lds_kernel, dim3(gc), dim3(kLeafThreads), lbytes, stream, sp.leaves, pairs,
                               sp.L, lcnt);
        } else {
            hipLaunchKernelGGL(leaf_count_kernel, dim3(gb), dim3(256), 0, stream, sp.leaves, pairs, sp.L, lcnt);
        }
        hipLaunchKernelGGL(leaf_scan_kernel, dim3(1), dim3(1024), 0, stream, lcnt, sp.leaf_offsets, sp.L, ma.qg,
                           ma.item_pts, lqoff, itemoff);
        if (lds)
            hipLaunchKernelGGL(leaf_scatter_lds_kernel, dim3(gc), dim3(kLeafThreads), lbytes, stream, sp.leaves, sp.nq,
                               sp.nl, sp.L, lqoff, lcur, qlist, p.leaf_bias, p.bias_bound, qbias);
        else
            hipLaunchKernelGGL(leaf_scatter_kernel, dim3(gb), dim3(256), 0, stream, sp.leaves, sp.nq, sp.nl, sp.L, lqoff,
                               lcur, qlist, p.leaf_bias, p.bias_bound, qbias);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        ma.lqoff = lqoff;
        ma.qlist = qlist;
        ma.qbias = biased ? qbias : nullptr;
        ma.itemoff = itemoff;
    }
    // warm-up rows per query: enough for a first bound; the item-local
    // thresholds tighten it within the first items.  Queries that scan about
    // 2^19 rows or more take at least 2,048: their first bound holds for the
    // whole first round of items (one per CU), which at 20M x 384 (1M rows per
    // query) otherwise appended 2.4x the candidates; with fewer rows per query
    // the larger warm-up costs more than it saves.
    const int64_t rows_q = part ? sp.n * sp.nl / (sp.L > 0 ? sp.L : 1) : sp.n;
    int32_t W = 2 * sp.R;
    const int32_t wmin = rows_q >= (int64_t)1 << 19 ? 2048 : 1024;
    if (W < wmin) W = wmin;
    if (streaming) W = 8192;  // a few queries (partitioned): a tighter first bound is cheap and every workgroup starts from it
    if (W > 8192) W = 8192;
    const size_t lut_bytes = ((size_t)tstride(sp.B) * 16 + 15) & ~(size_t)15;
    // (the spread warm-up may pad its table to whole 32-block code segments)
    const size_t spread_lut = seg_lut_bytes(sp.B);
    if (streaming && !part && sp.n > 0 && spread_lut <= 64 * 1024) {
        int64_t Ws = sp.n < kSpreadRows ? sp.n : kSpreadRows;
        const int64_t cap = kSpreadLookups / sp.B, floor_rows = sp.n < 8192 ? sp.n : 8192;
        if (Ws > cap) Ws = cap > floor_rows ? cap : floor_rows;
        const int nwg = (int)((Ws + kSpreadThreads - 1) / kSpreadThreads);  // at most kSpreadWG
        uint32_t* wpart = reinterpret_cast<uint32_t*>(base + lay.wpart);
        allow_lds(warmup_spread_kernel, spread_lut);
        hipLaunchKernelGGL(warmup_spread_kernel, dim3((unsigned)nwg, (unsigned)sp.nq), dim3(kSpreadThreads), spread_lut,
                           stream, p, st, (int32_t)Ws, wpart);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(warmup_spread_finish_kernel, dim3((unsigned)sp.nq), dim3(kNB), 0, stream, p, st,
                           (int32_t)Ws, nwg, wpart);
    } else if ((size_t)tstride(32 * (((sp.B + 1) / 2 + 15) / 16)) * 16 <= (size_t)kWaveLut) {
        // (the one-wave warm-up pads its table to whole 32-block code segments)
        hipLaunchKernelGGL(warmup_wave_kernel, dim3((unsigned)((sp.nq + 3) / 4)), dim3(kSelThreads), 0, stream, p, st, W);
    } else {
        allow_lds(warmup_kernel, seg_lut_bytes(sp.B) + (size_t)W * 8);
        hipLaunchKernelGGL(warmup_kernel, dim3((unsigned)sp.nq), dim3(kSelThreads), seg_lut_bytes(sp.B) + (size_t)W * 8, stream, p,
                           st, W);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t max_items = part ? (int64_t)sp.nq * sp.nl + sp.L : ma.n_items;
    int grid = device_cus();
    if (max_items < grid) grid = (int)(max_items > 0 ? max_items : 1);
    if (main_start && (e = hipEventRecord(main_start, stream)) != hipSuccess) return e;
    if (!streaming) {
        const bool staged = ma.nchunk > 1;
        const bool fast = ma.fast_codes != 0;
#define AH_MAIN(BIAS, ST, FAST) \
    hipLaunchKernelGGL((scan_main_kernel<BIAS, ST, FAST>), dim3(grid), dim3(kScanThreads), 0, stream, ma)
        if (ma.qbias) {
            if (!staged) AH_MAIN(true, false, false);
            else if (fast) AH_MAIN(true, true, true);
            else AH_MAIN(true, true, false);
        } else {
            if (!staged) AH_MAIN(false, false, false);
            else if (fast) AH_MAIN(false, true, true);
            else AH_MAIN(false, true, false);
        }
#undef AH_MAIN
    } else {
        const int nseg = ((sp.B + 1) / 2 + 15) / 16;
        if (spair && sg == 1) launch_stream<1, true>(nseg, grid, stbl, stream, ma);
        else if (spair) launch_stream<2, true>(nseg, grid, stbl, stream, ma);
        else if (sg == 1) launch_stream<1, false>(nseg, grid, stbl, stream, ma);
        else launch_stream<4, false>(nseg, grid, stbl, stream, ma);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (main_stop && (e = hipEventRecord(main_stop, stream)) != hipSuccess) return e;
    int Rp = 1;
    while (Rp < sp.R) Rp <<= 1;
    if (sp.nq <= kFewMaxQ)
        hipLaunchKernelGGL(final_select_few_kernel, dim3((unsigned)sp.nq), dim3(kFewThreads), 0, stream, p, st);
    else
        hipLaunchKernelGGL(final_select_wave_kernel, dim3((unsigned)((sp.nq + 3) / 4)), dim3(kSelThreads), 0, stream, p, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    allow_lds(final_select_kernel, (size_t)(kSelLds + Rp) * 8);
    hipLaunchKernelGGL(final_select_kernel, dim3((unsigned)sp.nq), dim3(kSelThreads), (size_t)(kSelLds + Rp) * 8, stream, p, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    allow_lds(fallback_kernel, (size_t)Rp * 8 + lut_bytes);
    hipLaunchKernelGGL(fallback_kernel, dim3(kFbSlots), dim3(kSelThreads), (size_t)Rp * 8 + lut_bytes, stream, p, st);
    return hipGetLastError();
}

// ------------------------------------------------------------------ tiled code layout
// One thread per destination 16-byte unit (tile t, segment j, row slot r, in
// that order): the unit holds bytes [16 j, 16 j + 16) of row 64 t + r, zero
// past the row's code bytes or past the last row.
__global__ void tile_codes_kernel(const uint8_t* __restrict__ src, int32_t stride, int64_t n, int32_t cb, int32_t S,
                                  uint4* __restrict__ dst, int64_t units) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < units;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = e / (64 * S);
        const int rem = (int)(e - t * 64 * S);
        const int j = rem >> 6, r = rem & 63;
        const int64_t row = t * 64 + r;
        uint32_t wd[4] = {0, 0, 0, 0};
        if (row < n) {
            const uint8_t* rp = src + row * stride;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int idx = 16 * j + k;
                if (idx < cb) wd[k >> 2] |= (uint32_t)rp[idx] << (8 * (k & 3));
            }
        }
        dst[e] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
}

size_t tiled_codes_bytes(int64_t n, int32_t B) {
    const int64_t S = ((B + 1) / 2 + 15) / 16;
    return (size_t)((n + 63) / 64) * 64 * (size_t)S * 16;
}

hipError_t launch_tile_codes(const uint8_t* codes, int32_t stride, int64_t n, int32_t B, uint8_t* tiled,
                             hipStream_t stream) {
    const int32_t cb = (B + 1) / 2, S = (cb + 15) / 16;
    const int64_t units = ((n + 63) / 64) * 64 * S;
    const int64_t blocks = (units + 255) / 256;
    hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream,
                       codes, stride, n, cb, S, reinterpret_cast<uint4*>(tiled), units);
    return hipGetLastError();
}

}  // namespace ah
