// Exact reorder: rescore each query's candidates with exact dot products against
// the stored rows and keep the best k.
//
// Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
// Product Search", section "Three stages of a search" (reordering rescores the
// best few hundred candidates with exact dot products) and "Failure modes"
// (reorder must keep more than k).
//
// Design: the kernel is a gather -- R rows of d elements per query, each row a
// contiguous 400 B .. 3 KB run -- so it is bound by HBM bandwidth.  One
// workgroup per query keeps the query in LDS; each wave streams candidate rows
// with 16-byte loads, G lanes per row (G = the row's 16-byte chunks over the
// chunks each lane takes, rounded up to a power of two, at most 64) so short
// rows still fill the wave, and four rows per lane group are in flight at once.  bf16 rows are widened exactly (bits
// << 16); every product of two fp32 values is exact in fp64 and the dot
// product is accumulated in fp64 (the gather leaves the ALUs mostly idle),
// then rounded once to fp32: scores agree with an fp64 reference to the
// rounding of the result, so near-ties at the k-th place are ordered as in
// fp64 unless they round to the same fp32 value (then the lower id wins).  A
// lane meets the same query elements in every row, so when a row takes one
// pass it holds them in registers, widened once.  The R scores become ranking
// keys; for k <= 64 of R <= 512 one wave takes the best k by k rounds of a wave
// maximum (the workgroup selection's radix passes and barriers cost 28% of the
// kernel at 1M x 100, R = 200, k = 10; this path 12%), otherwise the
// workgroup's exact top-k selection orders them.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kReorderThreads = 256;
constexpr int kReorderWaves = kReorderThreads / kWave;

// a += chunk x . qq (qq: the chunk's query elements, fp32 or already fp64)
struct ChunkF32 {
    static constexpr int kElems = 4;
    template <typename QT>
    __device__ static double dot(const uint4 x, const QT* qq, double a) {
        a = __fma_rn((double)__uint_as_float(x.x), (double)qq[0], a);
        a = __fma_rn((double)__uint_as_float(x.y), (double)qq[1], a);
        a = __fma_rn((double)__uint_as_float(x.z), (double)qq[2], a);
        a = __fma_rn((double)__uint_as_float(x.w), (double)qq[3], a);
        return a;
    }
};
struct ChunkBF16 {
    static constexpr int kElems = 8;
    template <typename QT>
    __device__ static double dot(const uint4 x, const QT* qq, double a) {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a = __fma_rn((double)__uint_as_float(w[t] << 16), (double)qq[2 * t], a);
            a = __fma_rn((double)__uint_as_float(w[t] & 0xFFFF0000u), (double)qq[2 * t + 1], a);
        }
        return a;
    }
};

__device__ __forceinline__ float load_elem(const void* base, int32_t dtype, int64_t i) {
    if (dtype == 0) return reinterpret_cast<const float*>(base)[i];
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

// G lanes per row, kNR rows per lane group in flight, each lane's (at most kCPL)
// 16-byte chunks of all kNR rows loaded before any is used.  kOnePass: a row
// takes one pass (at most kCPL x G chunks), so the lane's query elements stay
// in registers as fp64.
template <typename Chunk, int kCPL, bool kOnePass>
__device__ void score_rows_vec(const float* qs, int32_t d, const void* base, int64_t n, const int32_t* cand,
                               int32_t R, uint64_t* keys) {
    constexpr int kNR = 4;
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    const int C = d / Chunk::kElems;  // 16-byte chunks per row
    const int Cl = (C + kCPL - 1) / kCPL;  // chunks a lane group covers per pass
    int G = 1;
    while (G < Cl && G < kWave) G <<= 1;
    const int per = kWave / G;  // rows per wave pass
    const int sub = lane / G, gl = lane % G;
    const size_t row_bytes = (size_t)d * (Chunk::kElems == 4 ? 4 : 2);
    double qv[kOnePass ? kCPL : 1][Chunk::kElems];
    if (kOnePass) {
#pragma unroll
        for (int t = 0; t < kCPL; ++t) {
            const int j = gl + t * G;
#pragma unroll
            for (int e = 0; e < Chunk::kElems; ++e) qv[t][e] = j < C ? (double)qs[Chunk::kElems * j + e] : 0.0;
        }
    }
    for (int r0 = w * per * kNR; r0 < R; r0 += kReorderWaves * per * kNR) {
        int id[kNR];
        const char* row[kNR];
#pragma unroll
        for (int v = 0; v < kNR; ++v) {
            const int r = r0 + v * per + sub;
            int x = r < R ? cand[r] : -1;
            id[v] = x >= n ? -1 : x;
            row[v] = reinterpret_cast<const char*>(base) + (size_t)(id[v] < 0 ? 0 : id[v]) * row_bytes;
        }
        double sc[kNR] = {};
        for (int jb = gl; jb < C; jb += kCPL * G) {  // one pass unless the row exceeds kCPL x 64 chunks
            uint4 raw[kNR][kCPL];
#pragma unroll
            for (int v = 0; v < kNR; ++v)
#pragma unroll
                for (int t = 0; t < kCPL; ++t) {
                    const int j = jb + t * G;
                    raw[v][t] = (id[v] >= 0 && j < C) ? reinterpret_cast<const uint4*>(row[v])[j] : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
            for (int v = 0; v < kNR; ++v)
#pragma unroll
                for (int t = 0; t < kCPL; ++t) {
                    const int j = jb + t * G;
                    if (j < C) {
                        if (kOnePass) sc[v] = Chunk::dot(raw[v][t], qv[t], sc[v]);
                        else sc[v] = Chunk::dot(raw[v][t], qs + Chunk::kElems * j, sc[v]);
                    }
                }
        }
        static_assert(kNR == 4, "the reduce-scatter below splits four rows");
        if (G >= 4) {
            // reduce-scatter over the G lanes: the two top exchange steps each
            // halve the rows a lane carries (four rows, then two, then one), so
            // a pass costs log2(G) + 1 exchanges of a double instead of 4 log2(G)
            const int h = G >> 1, qb = G >> 2;
            const bool b1 = (gl & h) != 0, b0 = (gl & qb) != 0;
            double k0 = b1 ? sc[2] : sc[0], k1 = b1 ? sc[3] : sc[1];
            const double s0 = b1 ? sc[0] : sc[2], s1 = b1 ? sc[1] : sc[3];
            k0 += __shfl_xor(s0, h, kWave);
            k1 += __shfl_xor(s1, h, kWave);
            double a = b0 ? k1 : k0;
            a += __shfl_xor(b0 ? k0 : k1, qb, kWave);
            for (int o = qb >> 1; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
            // every lane of the group now holds the sum of row 2 b1 + b0
            if ((gl & (qb - 1)) == 0) {
                const int v = 2 * (int)b1 + (int)b0;
                const int r = r0 + v * per + sub;
                const int idv = v == 0 ? id[0] : (v == 1 ? id[1] : (v == 2 ? id[2] : id[3]));
                if (r < R) keys[r] = idv >= 0 ? float_key(__double2float_rn(a), idv) : 0ull;
            }
        } else {
#pragma unroll
            for (int v = 0; v < kNR; ++v) {
                double a = sc[v];
                for (int o = G >> 1; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
                sc[v] = a;
            }
            if (gl == 0) {
#pragma unroll
                for (int v = 0; v < kNR; ++v) {
                    const int r = r0 + v * per + sub;
                    if (r < R) keys[r] = id[v] >= 0 ? float_key(__double2float_rn(sc[v]), id[v]) : 0ull;
                }
            }
        }
    }
}

__device__ void score_rows_scalar(const float* qs, int32_t d, const void* base, int32_t dtype, int64_t n,
                                  const int32_t* cand, int32_t R, uint64_t* keys) {
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    for (int r = w; r < R; r += kReorderWaves) {
        const int id = cand[r] < n ? cand[r] : -1;
        double s = 0.0;
        if (id >= 0)
            for (int j = lane; j < d; j += kWave)
                s = __fma_rn((double)qs[j], (double)load_elem(base, dtype, (int64_t)id * d + j), s);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
        if (lane == 0) keys[r] = id >= 0 ? float_key(__double2float_rn(s), id) : 0ull;
    }
}

// The best k of the R keys in LDS (k <= 64, R <= 512), in descending order, into
// sel, by wave 0: each lane holds up to eight keys, and k rounds each take the
// wave's largest remaining key and clear one occurrence of it (the lowest lane,
// then its first slot, holding it), stopping at the zero keys of invalid
// candidates.  The same keys in the same order as the workgroup selection.
// Returns the number selected (wave 0 only).
__device__ __forceinline__ int wave_select_topk(const uint64_t* keys, int R, int k, uint64_t* sel) {
    const int lane = lane_id();
    uint64_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = lane + kWave * j;
        v[j] = r < R ? keys[r] : 0ull;
    }
    int m = 0;
    for (; m < k; ++m) {
        uint64_t best = v[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) best = v[j] > best ? v[j] : best;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const uint64_t other = __shfl_xor(best, o, kWave);
            best = other > best ? other : best;
        }
        if (best == 0) break;
        if (lane == 0) sel[m] = best;
        int slot = -1;
#pragma unroll
        for (int j = 7; j >= 0; --j)
            if (v[j] == best) slot = j;
        const uint64_t mk = __ballot(slot >= 0);
        if (lane == __ffsll((unsigned long long)mk) - 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j == slot) v[j] = 0ull;
        }
    }
    return m;
}

// LDS: [R keys][next_pow2(k) selected][d query floats].  kPath: 0 = element-wise
// (rows not in whole 16-byte chunks), else the chunk path with kCPL chunks per lane
// (kOnePass: every row in one pass).
template <int kPath, int kCPL, bool kOnePass>
__global__ __launch_bounds__(kReorderThreads) void reorder_kernel(
    const float* __restrict__ q, int32_t d, const void* __restrict__ base, int32_t dtype,
    int64_t n, const int32_t* __restrict__ cand, int32_t R, int32_t k, int32_t* __restrict__ ids_out,
    float* __restrict__ scores_out) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ SelectShared sh;
    __shared__ int sel_m;
    const int64_t qi = blockIdx.x;
    const int Kp = next_pow2(k);
    uint64_t* keys = reinterpret_cast<uint64_t*>(smem);
    uint64_t* sel = keys + R;
    float* qs = reinterpret_cast<float*>(sel + Kp);
    for (int j = threadIdx.x; j < d; j += kReorderThreads) qs[j] = q[qi * d + j];
    __syncthreads();
    const int32_t* c = cand + qi * R;
    if constexpr (kPath == 0) {
        score_rows_scalar(qs, d, base, dtype, n, c, R, keys);
    } else if (kPath == 1) {
        score_rows_vec<ChunkF32, kCPL, kOnePass>(qs, d, base, n, c, R, keys);
    } else {
        score_rows_vec<ChunkBF16, kCPL, kOnePass>(qs, d, base, n, c, R, keys);
    }
    __syncthreads();
    int m;
    if (k <= kWave && R <= 8 * kWave) {
        if (threadIdx.x < kWave) {
            const int mw = wave_select_topk(keys, R, k, sel);
            if (threadIdx.x == 0) sel_m = mw;
        }
        __syncthreads();
        m = sel_m;
    } else {
        m = wg_select_topk<kReorderThreads>(LdsKeys{keys}, R, k, sh, sel);
    }
    for (int r = threadIdx.x; r < k; r += kReorderThreads) {
        ids_out[qi * k + r] = r < m ? key_id(sel[r]) : -1;
        scores_out[qi * k + r] = r < m ? key_float_score(sel[r]) : -__builtin_huge_valf();
    }
}

template <int kPath, int kCPL, bool kOnePass = true>
static hipError_t launch_reorder1(size_t lds, const float* q, int64_t nq, int32_t d, const void* base, int32_t dtype,
                                  int64_t n, const int32_t* cand, int32_t R, int32_t k, int32_t* ids, float* scores,
                                  hipStream_t stream) {
    if (lds > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(reorder_kernel<kPath, kCPL, kOnePass>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((reorder_kernel<kPath, kCPL, kOnePass>), dim3((unsigned)nq), dim3(kReorderThreads), lds, stream, q, d,
                       base, dtype, n, cand, R, k, ids, scores);
    return hipGetLastError();
}

hipError_t launch_reorder(const float* q, int64_t nq, int32_t d, const void* base, int32_t dtype,
                          int64_t n, const int32_t* cand, int32_t R, int32_t k, int32_t* ids,
                          float* scores, hipStream_t stream) {
    if (nq == 0) return hipSuccess;
    const int elem = dtype == 0 ? 4 : 2;
    const bool vec = ((size_t)d * elem) % 16 == 0 && (reinterpret_cast<uintptr_t>(base) & 15) == 0;
    int Kp = 1;
    while (Kp < k) Kp <<= 1;
    const size_t lds = (size_t)R * 8 + (size_t)Kp * 8 + (size_t)d * 4;
    if (!vec) return launch_reorder1<0, 1>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream);
    // chunks per lane: ceil(C / 64) for rows of C > 64 chunks, else 1; longer rows
    // loop.  bf16 rows of 33-63 chunks take two per lane on a 32-lane group (twice
    // the rows in flight; 384 dims: 0.51 -> 0.47 ms at 10,000 x 300 candidates);
    // four per lane, or two on fp32 rows of 25 or 32 chunks, measured slower.
    const int C = (int)((size_t)d * elem / 16);
    const int cpl = (elem == 2 && C > 32 && C < 64) ? 2 : (C + kWave - 1) / kWave;
#define AH_RO(P)                                                                                             \
    do {                                                                                                     \
        if (cpl <= 1) return launch_reorder1<P, 1>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream); \
        if (cpl <= 2) return launch_reorder1<P, 2>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream); \
        if (cpl <= 4) return launch_reorder1<P, 4>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream); \
        return launch_reorder1<P, 4, false>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream);       \
    } while (0)
    if (dtype == 0) AH_RO(1);
    AH_RO(2);
#undef AH_RO
}

}  // namespace ah
