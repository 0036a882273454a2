// Int8 scalar-quantised flat search: per-vector int8 codes with a robust
// percentile step, exact int32 dot products on the matrix cores, and the top-R
// documents per query by the rescaled score.
//
// Source: page "Incoherence-Aware Asymmetric Quantization for Retrieval",
// sections on the robust per-vector int8 scale (the pct-th percentile of a
// vector's absolute values over 127; codes clip(round(x / s), -127, 127)) and
// "A Specialized int8 Retrieval Engine" (exact integer dot of a query and a
// document, scaled by both steps; best k by that score).  The page's engine
// runs on CPU SIMD; here the dots are an int8 contraction on gfx950.
//
// Readings: the percentile is the linear interpolation numpy computes for a
// float32 vector, every step in float32 (position (d-1) * pct/100, fraction t,
// a + (b-a) t below one half, else b - (b-a)(1-t)); the step
// s = max(P, 1e-8) / 127; x / s in float32, round half to even.  Score =
// ((float)dot * s_q) * s_d in float32; ranking (score desc, document id asc).
//
// Design: quantisation, one wave per vector: the two order statistics around
// the percentile position come from an MSD radix select over the float bits
// of |x| (four 8-bit passes over the row, a 256-bin LDS histogram per wave),
// then one pass writes the codes.  Scores: v_mfma_i32_16x16x64_i8 with A = 16
// documents and B = 16 queries, each lane feeding the 16 bytes k = 16 g .. 16 g
// + 15 of one row (g = lane / 16) to both operands (the same k map on both
// sides, so the contraction is exact whatever the hardware's internal k order);
// a workgroup computes 256 documents x 64 queries (four waves of 64 x 64), the
// int32 dots are rescaled in the epilogue into a score block, and the best R of
// each query's row come from the same selection kernels as the leaf choice.
// Bound: int8 MFMA (2 n d FLOP-equivalents per query).
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

// ------------------------------------------------------------------ quantisation
constexpr int kQzWaves = 4;

__global__ __launch_bounds__(kQzWaves * kWave) void sq8_quantize_kernel(const float* __restrict__ x, int64_t n,
                                                                        int32_t d, float pct,
                                                                        int8_t* __restrict__ codes,
                                                                        float* __restrict__ scale) {
#pragma clang fp contract(off)  // the step's arithmetic is defined operation by operation
    __shared__ uint32_t hist_all[kQzWaves][256];
    const int w = threadIdx.x / kWave, lane = lane_id();
    const int64_t i = (int64_t)blockIdx.x * kQzWaves + w;
    if (i >= n) return;  // whole waves; no workgroup barrier below
    uint32_t* hist = hist_all[w];
    const float* row = x + i * d;
    auto key = [&](int t) -> uint32_t { return __float_as_uint(fabsf(row[t])); };
    auto fence = [] {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };
    const float pos = (float)(d - 1) * pct;  // pct passed as pct / 100
    int lo = (int)floorf(pos);
    lo = lo < d - 1 ? lo : d - 1;
    // rank lo (0-based, ascending) by 8-bit digits, most significant first
    uint32_t prefix = 0, mask = 0;
    int need = lo;  // keys below the current bucket that are still to be skipped
    int inb = d;    // keys in the current bucket
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) hist[4 * lane + j] = 0;
        fence();
        for (int t = lane; t < d; t += kWave) {
            const uint32_t k = key(t);
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
        }
        fence();
        // ascending buckets: lane l owns bins 4l .. 4l+3
        uint32_t c[4];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[j] = hist[4 * lane + j];
            sum += (int)c[j];
        }
        const int incl = wave_inclusive_sum(sum);
        const uint64_t mk = __ballot(incl > need);
        const int l = __ffsll((unsigned long long)mk) - 1;
        int digit = 0, below = 0, cnt = 0;
        if (lane == l) {
            int cum = incl - sum;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (cum <= need && cum + (int)c[j] > need) {
                    digit = 4 * lane + j;
                    below = cum;
                    cnt = (int)c[j];
                }
                cum += (int)c[j];
            }
        }
        digit = __shfl(digit, l, kWave);
        below = __shfl(below, l, kWave);
        cnt = __shfl(cnt, l, kWave);
        fence();
        need -= below;
        inb = cnt;
        prefix |= (uint32_t)digit << shift;
        mask |= 255u << shift;
    }
    // prefix = the key of rank lo; need = its rank among the keys equal to it
    const float va = __uint_as_float(prefix);
    float vb = va;
    if (lo + 1 < d && need + 1 >= inb) {  // rank lo + 1 is the smallest key above it
        uint32_t mn = 0xFFFFFFFFu;
        for (int t = lane; t < d; t += kWave) {
            const uint32_t k = key(t);
            if (k > prefix && k < mn) mn = k;
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            const uint32_t o = __shfl_xor(mn, off, kWave);
            mn = o < mn ? o : mn;
        }
        vb = __uint_as_float(mn);
    }
    const float tf = pos - (float)lo;
    const float diff = vb - va;
    const float P = tf < 0.5f ? va + diff * tf : vb - diff * (1.0f - tf);
    const float s = (P > 1e-8f ? P : 1e-8f) / 127.0f;
    if (lane == 0) scale[i] = s;
    int8_t* out = codes + i * d;
    for (int t = lane; t < d; t += kWave) {
        float v = rintf(row[t] / s);
        v = v > 127.0f ? 127.0f : (v < -127.0f ? -127.0f : v);
        out[t] = (int8_t)(int)v;
    }
}

hipError_t launch_sq8_quantize(const float* x, int64_t n, int32_t d, double pct, int8_t* codes, float* scale,
                               hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(sq8_quantize_kernel, dim3((unsigned)((n + kQzWaves - 1) / kQzWaves)), dim3(kQzWaves * kWave),
                       0, stream, x, n, d, (float)(pct / 100.0), codes, scale);
    return hipGetLastError();
}

// ------------------------------------------------------------------ scores
constexpr int kSqThreads = 256;
constexpr int kSqDocs = 256;    // documents per workgroup (64 per wave)
constexpr int kSqQueries = 64;  // queries per workgroup

__global__ __launch_bounds__(kSqThreads) void sq8_scores_kernel(const int8_t* __restrict__ q8,
                                                                const float* __restrict__ qs, int64_t nq,
                                                                const int8_t* __restrict__ d8,
                                                                const float* __restrict__ ds, int64_t n, int32_t d,
                                                                float* __restrict__ S) {
#pragma clang fp contract(off)
    const int w = threadIdx.x / kWave, lane = lane_id();
    const int64_t ndt = (n + kSqDocs - 1) / kSqDocs;  // consecutive workgroups share a query tile
    const int64_t q0 = ((int64_t)blockIdx.x / ndt) * kSqQueries;
    const int64_t doc0 = ((int64_t)blockIdx.x % ndt) * kSqDocs + 64 * w;
    const int r16 = lane & 15, g = lane >> 4;
    v4i acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = v4i{0, 0, 0, 0};
    // row pointers (rows past the end read the last row; their results are dropped)
    const int8_t* arow[4];
    const int8_t* brow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int64_t r = doc0 + 16 * m + r16;
        arow[m] = d8 + (r < n ? r : n - 1) * d;
        const int64_t c = q0 + 16 * m + r16;
        brow[m] = q8 + (c < nq ? c : nq - 1) * d;
    }
    for (int k0 = 0; k0 < d; k0 += 64) {
        const int kk = k0 + 16 * g;
        const bool in = kk < d;  // d is a multiple of 16: a chunk is whole or absent
        v4i a[4], b[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            a[m] = in ? *reinterpret_cast<const v4i*>(arow[m] + kk) : v4i{0, 0, 0, 0};
            b[m] = in ? *reinterpret_cast<const v4i*>(brow[m] + kk) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[m][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[m], b[t], acc[m][t], 0, 0, 0);
    }
    // D[doc][query]: lane holds documents 4 g + i of query column r16
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t qq = q0 + 16 * t + r16;
        if (qq >= nq) continue;
        const float sq = qs[qq];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t doc = doc0 + 16 * m + 4 * g + i;
                if (doc < n) S[qq * n + doc] = ((float)acc[m][t][i] * sq) * ds[doc];
            }
    }
}

static int64_t sq8_chunk(int64_t nq, int64_t n) {
    int64_t c = ((int64_t)1 << 28) / (n > 0 ? n : 1);  // score block up to 1 GiB
    c = c < kSqQueries ? kSqQueries : (c / kSqQueries) * kSqQueries;
    return c < nq ? c : (nq > 0 ? nq : 1);
}

size_t sq8_workspace_bytes(int64_t nq, int64_t n) { return (size_t)sq8_chunk(nq, n) * (size_t)n * 4 + 256; }

hipError_t launch_sq8_topk(const int8_t* q8, const float* qs, int64_t nq, const int8_t* d8, const float* ds,
                           int64_t n, int32_t d, int32_t R, int32_t* ids, float* scores, void* ws,
                           hipStream_t stream) {
    if (nq == 0) return hipSuccess;
    float* S = reinterpret_cast<float*>(ws);
    const int64_t chunk = sq8_chunk(nq, n);
    for (int64_t a = 0; a < nq; a += chunk) {
        const int64_t m = nq - a < chunk ? nq - a : chunk;
        const int64_t grid = ((m + kSqQueries - 1) / kSqQueries) * ((n + kSqDocs - 1) / kSqDocs);
        hipLaunchKernelGGL(sq8_scores_kernel, dim3((unsigned)grid), dim3(kSqThreads), 0, stream, q8 + a * d, qs + a, m,
                           d8, ds, n, d, S);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if ((e = launch_rows_topk(S, m, (int32_t)n, R, ids + a * R, scores ? scores + a * R : nullptr, stream)) !=
            hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace ah
