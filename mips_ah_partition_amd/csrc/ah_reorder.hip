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
// with 16-byte loads, G lanes per row (G = rows' 16-byte chunks rounded up to a
// power of two, at most 64) so short rows still fill the wave, and two rows per
// lane group are in flight at once.  bf16 rows are widened exactly (bits << 16)
// and accumulated in fp32.  The R scores become ranking keys and the
// workgroup's exact top-k selection orders them.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kReorderThreads = 256;
constexpr int kReorderWaves = kReorderThreads / kWave;

struct ChunkF32 {
    static constexpr int kElems = 4;
    __device__ static float dot(const uint4 x, int j, const float* qs) {
        const float* qq = qs + 4 * j;
        float a = __uint_as_float(x.x) * qq[0];
        a = __fmaf_rn(__uint_as_float(x.y), qq[1], a);
        a = __fmaf_rn(__uint_as_float(x.z), qq[2], a);
        a = __fmaf_rn(__uint_as_float(x.w), qq[3], a);
        return a;
    }
};
struct ChunkBF16 {
    static constexpr int kElems = 8;
    __device__ static float dot(const uint4 x, int j, const float* qs) {
        const float* qq = qs + 8 * j;
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        float a = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a = __fmaf_rn(__uint_as_float(w[t] << 16), qq[2 * t], a);
            a = __fmaf_rn(__uint_as_float(w[t] & 0xFFFF0000u), qq[2 * t + 1], a);
        }
        return a;
    }
};

__device__ __forceinline__ float load_elem(const void* base, int32_t dtype, int64_t i) {
    if (dtype == 0) return reinterpret_cast<const float*>(base)[i];
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
}

// G lanes per row, kNR rows per lane group in flight, each lane's (at most kCPL)
// 16-byte chunks of all kNR rows loaded before any is used.
template <typename Chunk, int kCPL>
__device__ void score_rows_vec(const float* qs, int32_t d, const void* base, int64_t n, const int32_t* cand,
                               int32_t R, uint64_t* keys) {
    constexpr int kNR = 4;
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    const int C = d / Chunk::kElems;  // 16-byte chunks per row
    int G = 1;
    while (G < C && G < kWave) G <<= 1;
    const int per = kWave / G;  // rows per wave pass
    const int sub = lane / G, gl = lane % G;
    const size_t row_bytes = (size_t)d * (Chunk::kElems == 4 ? 4 : 2);
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
        float sc[kNR] = {};
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
                    if (j < C) sc[v] += Chunk::dot(raw[v][t], j, qs);
                }
        }
#pragma unroll
        for (int v = 0; v < kNR; ++v) {
            float a = sc[v];
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1)
                if (o < G) a += __shfl_xor(a, o, kWave);
            sc[v] = a;
        }
        if (gl == 0) {
#pragma unroll
            for (int v = 0; v < kNR; ++v) {
                const int r = r0 + v * per + sub;
                if (r < R) keys[r] = id[v] >= 0 ? float_key(sc[v], id[v]) : 0ull;
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
        float s = 0.0f;
        if (id >= 0)
            for (int j = lane; j < d; j += kWave) s = __fmaf_rn(qs[j], load_elem(base, dtype, (int64_t)id * d + j), s);
        s = wave_sum(s);
        if (lane == 0) keys[r] = id >= 0 ? float_key(s, id) : 0ull;
    }
}

// LDS: [R keys][next_pow2(k) selected][d query floats].  kPath: 0 = element-wise
// (rows not in whole 16-byte chunks), else the chunk path with kCPL chunks per lane.
template <int kPath, int kCPL>
__global__ __launch_bounds__(kReorderThreads) void reorder_kernel(
    const float* __restrict__ q, int32_t d, const void* __restrict__ base, int32_t dtype,
    int64_t n, const int32_t* __restrict__ cand, int32_t R, int32_t k, int32_t* __restrict__ ids_out,
    float* __restrict__ scores_out) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ SelectShared sh;
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
        score_rows_vec<ChunkF32, kCPL>(qs, d, base, n, c, R, keys);
    } else {
        score_rows_vec<ChunkBF16, kCPL>(qs, d, base, n, c, R, keys);
    }
    __syncthreads();
    const int m = wg_select_topk<kReorderThreads>(LdsKeys{keys}, R, k, sh, sel);
    for (int r = threadIdx.x; r < k; r += kReorderThreads) {
        ids_out[qi * k + r] = r < m ? key_id(sel[r]) : -1;
        scores_out[qi * k + r] = r < m ? key_float_score(sel[r]) : -__builtin_huge_valf();
    }
}

template <int kPath, int kCPL>
static hipError_t launch_reorder1(size_t lds, const float* q, int64_t nq, int32_t d, const void* base, int32_t dtype,
                                  int64_t n, const int32_t* cand, int32_t R, int32_t k, int32_t* ids, float* scores,
                                  hipStream_t stream) {
    if (lds > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(reorder_kernel<kPath, kCPL>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((reorder_kernel<kPath, kCPL>), dim3((unsigned)nq), dim3(kReorderThreads), lds, stream, q, d,
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
    // chunks per lane: ceil(C / 64) for rows of C > 64 chunks, else 1; longer rows loop
    const int C = (int)((size_t)d * elem / 16);
    const int cpl = (C + kWave - 1) / kWave;
#define AH_RO(P)                                                                                             \
    do {                                                                                                     \
        if (cpl <= 1) return launch_reorder1<P, 1>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream); \
        if (cpl <= 2) return launch_reorder1<P, 2>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream); \
        return launch_reorder1<P, 4>(lds, q, nq, d, base, dtype, n, cand, R, k, ids, scores, stream);              \
    } while (0)
    if (dtype == 0) AH_RO(1);
    AH_RO(2);
#undef AH_RO
}

}  // namespace ah
