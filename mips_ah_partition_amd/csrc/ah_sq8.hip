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
// a workgroup computes 256 documents x 64 queries (four waves of 64 x 64) and
// rescales the int32 dots in the epilogue.  Top R: for small n or large R the
// epilogue writes a score block that a row selection reduces; otherwise a bound
// from sampled 64-row group maxima lets the epilogue append only the scores at
// or above it to a per-query candidate list, which one wave selects (an exact
// rescan redoes a query whose list overflowed).
// Bound: int8 MFMA (2 n d FLOP-equivalents per query).
#include "ah_device.hpp"
#include "ah_kernels.hpp"

#include <limits.h>

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
constexpr int kSqGroup = 64;    // documents per group (one wave's rows) for the threshold
constexpr int kSqCap = 4096;    // candidates kept per query
constexpr int kSqFb = 8;        // fallback workgroups
constexpr int kSqMaxSel = 512;  // largest R the candidate path selects

enum SqMode { kSqWriteS = 0, kSqGroupMax = 1, kSqEmit = 2 };

struct SqOut {
    float* S;              // kSqWriteS: [nq][n]
    float* gmax;           // kSqGroupMax: [nq][G0], group j = documents of 64-row tile j * gstep
    int32_t G0;
    int64_t gstep;
    const float* tau;      // kSqEmit: the query's bound at tau[q * tau_stride + tau_stride - 1]
    int32_t tau_stride;
    uint32_t* cnt;         // kSqEmit: [nq] candidates appended
    float* cs;             // kSqEmit: [nq][cap] scores
    int32_t* ci;           //          [nq][cap] document ids
    int32_t cap;
};

// The documents' codes: int8 rows [n][d], or (d4 non-null) 4-bit codes [n][d/2]
// (low nibble = even dimension) whose nibbles stand for the int8 values lv
// (16 bytes, nibble c -> byte c), expanded as they are loaded.
struct DocSrc {
    const int8_t* d8;
    const uint8_t* d4;
    uint32_t lv[4];
};

__device__ __forceinline__ uint32_t nib_value(const DocSrc& s, uint32_t c) {
    const uint32_t w = c < 8 ? (c < 4 ? s.lv[0] : s.lv[1]) : (c < 12 ? s.lv[2] : s.lv[3]);
    return (w >> (8 * (c & 3))) & 255u;
}

// The 16 values k = kk .. kk+15 of document row r (kk a multiple of 16, below d).
// kForm: 0 = either (decided by d4), 1 = int8 rows, 2 = 4-bit codes.
template <int kForm = 0>
__device__ __forceinline__ v4i doc_chunk(const DocSrc& s, int64_t r, int32_t d, int kk) {
    if (kForm == 1 || (kForm == 0 && !s.d4)) return *reinterpret_cast<const v4i*>(s.d8 + r * d + kk);
    const uint2 c = *reinterpret_cast<const uint2*>(s.d4 + r * (d >> 1) + (kk >> 1));
    v4i out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t h = ((w < 2 ? c.x : c.y) >> (16 * (w & 1))) & 0xFFFFu;  // dimensions kk+4w .. kk+4w+3
        out[w] = (int)(nib_value(s, h & 15u) | (nib_value(s, (h >> 4) & 15u) << 8) |
                       (nib_value(s, (h >> 8) & 15u) << 16) | (nib_value(s, h >> 12) << 24));
    }
    return out;
}

// The document-stationary kernel's argument: only what its form needs.
template <bool kNib>
struct DocArg {
    const int8_t* d8;
    __device__ v4i chunk(int64_t r, int32_t d, int kk) const {
        return *reinterpret_cast<const v4i*>(d8 + r * d + kk);
    }
};
template <>
struct DocArg<true> {
    DocSrc s;
    __device__ v4i chunk(int64_t r, int32_t d, int kk) const { return doc_chunk<2>(s, r, d, kk); }
};

// The rescaled score of one (query, document) pair: the same expression in
// every mode, so the threshold and the candidates agree bit for bit.
__device__ __forceinline__ float sq8_score(int32_t dot, float sq, float sd) {
#pragma clang fp contract(off)
    return ((float)dot * sq) * sd;
}

// Generic form (any d that is a multiple of 16): each wave computes 64
// documents x 64 queries with operands loaded straight from global memory.
template <int kMode>
__global__ __launch_bounds__(kSqThreads) void sq8_scores_kernel(const int8_t* __restrict__ q8,
                                                                const float* __restrict__ qs, int64_t nq,
                                                                DocSrc dsrc,
                                                                const float* __restrict__ ds, int64_t n, int32_t d,
                                                                int64_t ndt, SqOut o) {
    const int w = threadIdx.x / kWave, lane = lane_id();
    // consecutive workgroups share a query tile; ndt doc tiles per query tile
    const int64_t q0 = ((int64_t)blockIdx.x / ndt) * kSqQueries;
    const int64_t dt = (int64_t)blockIdx.x % ndt;
    int64_t doc0;
    int32_t grp = 0;
    if constexpr (kMode == kSqGroupMax) {
        grp = (int32_t)(dt * 4 + w);
        if (grp >= o.G0) return;  // whole waves; no barrier in this kernel
        doc0 = (int64_t)grp * o.gstep * kSqGroup;
    } else {
        doc0 = dt * kSqDocs + 64 * w;
        if (doc0 >= n) return;
    }
    const int r16 = lane & 15, g = lane >> 4;
    v4i acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = v4i{0, 0, 0, 0};
    // row pointers (rows past the end read the last row; their results are dropped)
    int64_t arow[4];
    const int8_t* brow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int64_t r = doc0 + 16 * m + r16;
        arow[m] = r < n ? r : n - 1;
        const int64_t c = q0 + 16 * m + r16;
        brow[m] = q8 + (c < nq ? c : nq - 1) * d;
    }
    for (int k0 = 0; k0 < d; k0 += 64) {
        const int kk = k0 + 16 * g;
        const bool in = kk < d;  // d is a multiple of 16: a chunk is whole or absent
        v4i a[4], b[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            a[m] = in ? doc_chunk(dsrc, arow[m], d, kk) : v4i{0, 0, 0, 0};
            b[m] = in ? *reinterpret_cast<const v4i*>(brow[m] + kk) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[m][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[m], b[t], acc[m][t], 0, 0, 0);
    }
    // D[doc][query]: lane holds documents 16 m + 4 g + i of query column 16 t + r16
    float sdv[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t doc = doc0 + 16 * m + 4 * g + i;
            sdv[m][i] = ds[doc < n ? doc : n - 1];
        }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t qq = q0 + 16 * t + r16;
        const bool qok = qq < nq;
        const float sq = qs[qok ? qq : nq - 1];
        if constexpr (kMode == kSqWriteS) {
            if (!qok) continue;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t doc = doc0 + 16 * m + 4 * g + i;
                    if (doc < n) o.S[qq * n + doc] = sq8_score(acc[m][t][i], sq, sdv[m][i]);
                }
        } else if constexpr (kMode == kSqGroupMax) {
            float mx = -__builtin_huge_valf();
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t doc = doc0 + 16 * m + 4 * g + i;
                    const float v = sq8_score(acc[m][t][i], sq, sdv[m][i]);
                    if (doc < n && v > mx) mx = v;
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));  // the four lanes of a query column
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            if (g == 0 && qok) o.gmax[qq * o.G0 + grp] = mx;
        } else {
            if (!qok) continue;
            const float tq = o.tau[qq * o.tau_stride + o.tau_stride - 1];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t doc = doc0 + 16 * m + 4 * g + i;
                    const float v = sq8_score(acc[m][t][i], sq, sdv[m][i]);
                    if (doc < n && v >= tq) {
                        const uint32_t pos = atomicAdd(&o.cnt[qq], 1u);
                        if (pos < (uint32_t)o.cap) {
                            o.cs[qq * o.cap + pos] = v;
                            o.ci[qq * o.cap + pos] = (int32_t)doc;
                        }
                    }
                }
        }
    }
}

// Document-stationary form for d <= 64 KS: each wave keeps its 48 documents'
// codes for the whole K in registers (KS k-steps x 3 row groups x 16 bytes per
// lane, loaded once), and the workgroup (8 waves, two per SIMD, so one wave's
// epilogue overlaps the other's matrix work) streams blocks of 64 queries
// through LDS, double-buffered, rows padded by 16 bytes so the 16 lanes of a
// row group read 16 different bank groups.  Per block a wave issues 12 KS
// MFMAs and reads the block's 64 x 64 KS bytes from LDS once (96 int8 ops per
// LDS byte).  Workgroup x covers 384 documents (or, for the group maxima,
// eight sampled groups of 48) and query blocks [qb0, qb1) of its split.
constexpr int kDsQB = 64;                  // queries per block
constexpr int kDsM = 3;                    // 16-row groups per wave
constexpr int kDsW = 8;                    // waves per workgroup
constexpr int kDsRows = 16 * kDsM;         // documents per wave (= rows per threshold group)
constexpr int kDsThreads = kDsW * kWave;   // 512
constexpr int kDsDocs = kDsRows * kDsW;    // documents per workgroup
constexpr int kDsLog = 256;                // candidate log entries per wave

__device__ __forceinline__ void wave_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// A block's staging: rows x (4 KS) 16-byte chunks, thread tid taking chunks
// tid + 512 j (chunks past d re-read the row's last chunk: those k meet zero
// document codes), and the block's 64 query steps and bounds (threads 0..127).
template <int KS>
struct DsStage {
    static constexpr int kPer = (64 * 4 * KS + kDsThreads - 1) / kDsThreads;
    v4i v[kPer];
    float meta;
};
template <int KS, int kMode>
__device__ __forceinline__ void ds_stage_load(const int8_t* __restrict__ q8, const float* __restrict__ qs,
                                              const SqOut& o, int64_t nq, int32_t d, int64_t qb, int tid,
                                              DsStage<KS>& st) {
#pragma unroll
    for (int j = 0; j < DsStage<KS>::kPer; ++j) {
        int c = tid + kDsThreads * j;
        c = c < 64 * 4 * KS ? c : 64 * 4 * KS - 1;  // KS = 1: the second half re-reads the last chunk
        const int row = c / (4 * KS), col = c % (4 * KS);
        int64_t q = qb * kDsQB + row;
        q = q < nq ? q : nq - 1;
        const int off = col * 16 < d ? col * 16 : d - 16;
        st.v[j] = *reinterpret_cast<const v4i*>(q8 + q * d + off);
    }
    int64_t q = qb * kDsQB + (tid & 63);
    q = q < nq ? q : nq - 1;
    // one unconditional load per thread (threads 64..127 take the bound when there is one)
    const float* src = qs + q;
    if (kMode == kSqEmit && tid >= 64 && tid < 128) src = o.tau + q * o.tau_stride + o.tau_stride - 1;
    st.meta = *src;
}
template <int KS>
__device__ __forceinline__ void ds_stage_store(int8_t* buf, float* meta, int tid, const DsStage<KS>& st) {
    constexpr int kRow = KS * 64 + 16;
#pragma unroll
    for (int j = 0; j < DsStage<KS>::kPer; ++j) {
        const int c = tid + kDsThreads * j;
        const int row = c / (4 * KS), col = c % (4 * KS);
        if (c < 64 * 4 * KS) *reinterpret_cast<v4i*>(buf + row * kRow + col * 16) = st.v[j];
    }
    if (tid < 128) meta[tid] = st.meta;
}

template <int KS, int kMode, bool kNib>
__global__ __launch_bounds__(kDsThreads, 1) void sq8_dstat_kernel(const int8_t* __restrict__ q8,
                                                                   const float* __restrict__ qs, int64_t nq,
                                                                   DocArg<kNib> dsrc,
                                                                   const float* __restrict__ ds, int64_t n, int32_t d,
                                                                   int64_t ndt, int64_t qb_per, SqOut o) {
    constexpr int kRow = KS * 64 + 16;
    constexpr int kLogN = kMode == kSqEmit ? kDsLog : 1;
    __shared__ __align__(16) int8_t qbuf[2][kDsQB * kRow];
    __shared__ float qmeta[2][128];  // [0, 64): query steps, [64, 128): bounds
    // candidates found by each wave, appended to the global lists in batches
    __shared__ int32_t logq[kDsW][kLogN], logd[kDsW][kLogN];
    __shared__ float logs[kDsW][kLogN];
    __shared__ uint32_t logn[kDsW];
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t dt = (int64_t)blockIdx.x % ndt;
    const int64_t nqb = (nq + kDsQB - 1) / kDsQB;
    const int64_t qb0 = ((int64_t)blockIdx.x / ndt) * qb_per;
    const int64_t qb1 = qb0 + qb_per < nqb ? qb0 + qb_per : nqb;
    if (qb0 >= qb1) return;  // the whole workgroup
    // this wave's 48 documents; a wave with none still stages and meets the barriers
    int64_t doc0;
    int32_t grp = 0;
    bool active;
    if constexpr (kMode == kSqGroupMax) {
        grp = (int32_t)(dt * kDsW + w);
        active = grp < o.G0;
        doc0 = active ? (int64_t)grp * o.gstep * kDsRows : 0;
    } else {
        doc0 = dt * kDsDocs + kDsRows * w;
        active = doc0 < n;
        doc0 = active ? doc0 : 0;
    }
    DsStage<KS> st;
    ds_stage_load<KS, kMode>(q8, qs, o, nq, d, qb0, tid, st);
    v4i a[KS][kDsM];
#pragma unroll
    for (int m = 0; m < kDsM; ++m) {
        int64_t r = doc0 + 16 * m + r16;
        r = r < n ? r : n - 1;  // rows past the end read the last row; their results are dropped
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kk = ks * 64 + 16 * g;
            a[ks][m] = kk < d ? dsrc.chunk(r, d, kk) : v4i{0, 0, 0, 0};
        }
    }
    float sdv[kDsM][4];
    float sdmax = 0.f;  // the wave's largest document step (for the candidate pre-filter)
#pragma unroll
    for (int m = 0; m < kDsM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t doc = doc0 + 16 * m + 4 * g + i;
            sdv[m][i] = ds[doc < n ? doc : n - 1];
            sdmax = fmaxf(sdmax, sdv[m][i]);
        }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) sdmax = fmaxf(sdmax, __shfl_xor(sdmax, off, kWave));
    // rows of this wave that are real: local index 16 m + 4 g + i < nloc
    const int32_t nloc = n - doc0 < kDsRows ? (int32_t)(n - doc0) : kDsRows;
    ds_stage_store<KS>(qbuf[0], qmeta[0], tid, st);
    if (lane == 0) logn[w] = 0;
    // nothing is left in flight at the loop's entry, so the only memory waits
    // inside the loop are for the next block's staging
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the wave's log: appends to the query's global list, one atomic per lane
    auto flush = [&](uint32_t cnt) {
        wave_fence();
        for (uint32_t e = lane; e < cnt; e += kWave) {
            const int32_t qq = logq[w][e];
            const uint32_t pos = atomicAdd(&o.cnt[qq], 1u);
            if (pos < (uint32_t)o.cap) {
                o.cs[(int64_t)qq * o.cap + pos] = logs[w][e];
                o.ci[(int64_t)qq * o.cap + pos] = logd[w][e];
            }
        }
        wave_fence();
        if (lane == 0) logn[w] = 0;
        wave_fence();
    };
    for (int64_t qb = qb0; qb < qb1; ++qb) {
        const int buf = (int)((qb - qb0) & 1);
        const bool more = qb + 1 < qb1;
        if (more) ds_stage_load<KS, kMode>(q8, qs, o, nq, d, qb + 1, tid, st);  // in flight during the block
        v4i acc[kDsM][4];
#pragma unroll
        for (int m = 0; m < kDsM; ++m)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[m][t] = v4i{0, 0, 0, 0};
        const int8_t* qb_lds = qbuf[buf] + r16 * kRow + 16 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            v4i b[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) b[t] = *reinterpret_cast<const v4i*>(qb_lds + 16 * t * kRow + ks * 64);
#pragma unroll
            for (int m = 0; m < kDsM; ++m)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[m][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[ks][m], b[t], acc[m][t], 0, 0, 0);
        }
        // the next block goes to the other buffer now (its loads have had the
        // whole block to arrive; the previous block's stores are long done)
        if (more) ds_stage_store<KS>(qbuf[buf ^ 1], qmeta[buf ^ 1], tid, st);
        // lane holds documents 16 m + 4 g + i of query column 16 t + r16
        if (active) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int32_t qloc = (int32_t)(nq - qb * kDsQB) - 16 * t;  // query column real if r16 < qloc
                const bool qok = r16 < qloc;
                const int64_t qq = qb * kDsQB + 16 * t + r16;
                const float sq = qmeta[buf][16 * t + r16];
                if constexpr (kMode == kSqWriteS) {
                    if (!qok) continue;
#pragma unroll
                    for (int m = 0; m < kDsM; ++m)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (16 * m + 4 * g + i < nloc)
                                o.S[qq * n + doc0 + 16 * m + 4 * g + i] = sq8_score(acc[m][t][i], sq, sdv[m][i]);
                } else if constexpr (kMode == kSqGroupMax) {
                    // the group's best score, exactly (rows past the end are skipped)
                    float mx = -__builtin_huge_valf();
                    if (nloc == kDsRows) {
#pragma unroll
                        for (int m = 0; m < kDsM; ++m)
#pragma unroll
                            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sq8_score(acc[m][t][i], sq, sdv[m][i]));
                    } else {
#pragma unroll
                        for (int m = 0; m < kDsM; ++m)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float v = sq8_score(acc[m][t][i], sq, sdv[m][i]);
                                mx = 16 * m + 4 * g + i < nloc && v > mx ? v : mx;
                            }
                    }
                    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                    if (g == 0 && qok) o.gmax[qq * o.G0 + grp] = mx;
                } else {
                    if (!qok) continue;
                    const float tq = qmeta[buf][64 + 16 * t + r16];
                    // pre-filter: the exact score is within (1 + 2^-24)^3 of acc sq sd and
                    // fl(fl(acc sd) sq) within (1 - 2^-24)^3 of it, so no score of the lane's
                    // column reaches tq > 0 unless max_e fl(acc_e sd_e) * sq >= tq (1 - 2^-20)
                    if (tq > 0.f) {
                        float ym = -__builtin_huge_valf();
#pragma unroll
                        for (int m = 0; m < kDsM; ++m)
#pragma unroll
                            for (int i = 0; i < 4; ++i) ym = fmaxf(ym, (float)acc[m][t][i] * sdv[m][i]);
                        if (ym * sq < tq * 0.99999905f) continue;
                    }
#pragma unroll
                    for (int m = 0; m < kDsM; ++m)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int32_t li = 16 * m + 4 * g + i;
                            const float v = sq8_score(acc[m][t][i], sq, sdv[m][i]);
                            if (li < nloc && v >= tq) {
                                const int64_t doc = doc0 + li;
                                const uint32_t p = atomicAdd(&logn[w], 1u);
                                if (p < (uint32_t)kDsLog) {
                                    logq[w][p] = (int32_t)qq;
                                    logd[w][p] = (int32_t)doc;
                                    logs[w][p] = v;
                                } else {  // the log is full (many ties at the bound): append directly
                                    const uint32_t pos = atomicAdd(&o.cnt[qq], 1u);
                                    if (pos < (uint32_t)o.cap) {
                                        o.cs[qq * o.cap + pos] = v;
                                        o.ci[qq * o.cap + pos] = (int32_t)doc;
                                    }
                                }
                            }
                        }
                }
            }
        }
        if constexpr (kMode == kSqEmit) {
            wave_fence();
            uint32_t c = logn[w];
            c = c < (uint32_t)kDsLog ? c : (uint32_t)kDsLog;
            if (c > (uint32_t)(kDsLog / 2) || (!more && c > 0)) flush(c);
        }
        __syncthreads();
    }
}

__global__ void sq8_zero_kernel(uint32_t* p, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

// A query whose candidates overflowed the list (many documents tied at its
// bound) is redone exactly: every document's score into a private slot, then
// the workgroup selection.  Workgroup b takes queries b, b + kSqFb, ...
struct SlotKeys {
    const float* s;
    __device__ uint64_t operator()(int64_t i) const { return float_key(s[i], (int32_t)i); }
};

__global__ __launch_bounds__(kSqThreads) void sq8_fallback_kernel(const int8_t* __restrict__ q8,
                                                                  const float* __restrict__ qs, int64_t nq,
                                                                  DocSrc dsrc,
                                                                  const float* __restrict__ ds, int64_t n, int32_t d,
                                                                  int32_t R, const uint32_t* __restrict__ cnt,
                                                                  int32_t cap, float* __restrict__ slots,
                                                                  int32_t* __restrict__ ids, float* __restrict__ scores) {
    __shared__ SelectShared sh;
    __shared__ uint64_t sel[kSqMaxSel];
    float* slot = slots + (int64_t)blockIdx.x * n;
    const int tid = threadIdx.x;
    for (int64_t q = blockIdx.x; q < nq; q += gridDim.x) {
        if (cnt[q] <= (uint32_t)cap) continue;  // the same value for every thread
        const int8_t* qr = q8 + q * d;
        const float sq = qs[q];
        for (int64_t i = tid; i < n; i += kSqThreads) {
            int32_t dot = 0;
            for (int k = 0; k < d; k += 16) {
                const v4i a = *reinterpret_cast<const v4i*>(qr + k);
                const v4i b = doc_chunk(dsrc, i, d, k);
#pragma unroll
                for (int j = 0; j < 4; ++j) dot = __builtin_amdgcn_sdot4(a[j], b[j], dot, false);
            }
            slot[i] = sq8_score(dot, sq, ds[i]);
        }
        __syncthreads();
        const int m = wg_select_topk<kSqThreads>(SlotKeys{slot}, n, R, sh, sel);
        for (int r = tid; r < R; r += kSqThreads) {
            ids[q * R + r] = r < m ? key_id(sel[r]) : -1;
            if (scores) scores[q * R + r] = r < m ? key_float_score(sel[r]) : -__builtin_huge_valf();
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ host side
// Two ways to the top R:
//  * direct (small n, R above kSqMaxSel, or fewer 64-row groups than R): the
//    score block of a chunk of queries, then the row selection;
//  * candidate path: (1) scores of G0 sampled 64-row groups (every gstep-th),
//    keeping each group's maximum; the R-th largest maximum is a lower bound on
//    the query's R-th best score, as R distinct documents reach it; (2) all
//    scores again, appending those at or above the bound to the query's list;
//    (3) the one-wave selection of the list; (4) the exact fallback for lists
//    that overflowed.  The sample is sized so that about 512 documents per
//    query pass the bound for scores in random order.
struct SqPlan {
    bool direct;
    int64_t chunk;  // queries per pass
    int32_t G0;
    int64_t gstep;
    size_t off_gmax, off_tid, off_tsc, off_cnt, off_cs, off_ci, off_slots, total;
};

static size_t sq_align(size_t x) { return (x + 255) & ~(size_t)255; }

// rows per threshold group: one wave's documents in the scoring kernel used for d
static int32_t sq8_group_rows(int32_t d) { return d <= 8 * 64 ? kDsRows : kSqGroup; }

static SqPlan sq8_plan(int64_t nq, int64_t n, int32_t d, int32_t R) {
    SqPlan p{};
    const int32_t gsz = sq8_group_rows(d);
    const int64_t ngroups = (n + gsz - 1) / gsz;
    p.direct = n <= 4096 || R > kSqMaxSel || ngroups < R;
    const int64_t q1 = nq > 0 ? nq : 1;
    if (p.direct) {
        int64_t c = ((int64_t)1 << 28) / n;  // score block up to 1 GiB
        c = c < kSqQueries ? kSqQueries : (c / kSqQueries) * kSqQueries;
        p.chunk = c < q1 ? c : q1;
        p.total = (size_t)p.chunk * (size_t)n * 4 + 256;
        return p;
    }
    int64_t g0 = (ngroups * R + 511) / 512;
    g0 = g0 < R ? R : g0;
    g0 = g0 > ngroups ? ngroups : g0;
    p.G0 = (int32_t)g0;
    p.gstep = ngroups / g0;
    const size_t per_q = (size_t)g0 * 4 + (size_t)R * 8 + 4 + (size_t)kSqCap * 8;
    int64_t c = (int64_t)(((size_t)1 << 29) / per_q);  // lists and maxima up to 512 MiB per pass
    c = c < kSqQueries ? kSqQueries : (c / kSqQueries) * kSqQueries;
    p.chunk = c < q1 ? c : q1;
    size_t o = 0;
    p.off_gmax = o;  o = sq_align(o + (size_t)p.chunk * g0 * 4);
    p.off_tid = o;   o = sq_align(o + (size_t)p.chunk * R * 4);
    p.off_tsc = o;   o = sq_align(o + (size_t)p.chunk * R * 4);
    p.off_cnt = o;   o = sq_align(o + (size_t)p.chunk * 4);
    p.off_cs = o;    o = sq_align(o + (size_t)p.chunk * kSqCap * 4);
    p.off_ci = o;    o = sq_align(o + (size_t)p.chunk * kSqCap * 4);
    p.off_slots = o; o = sq_align(o + (size_t)kSqFb * (size_t)n * 4);
    p.total = o;
    return p;
}

size_t sq8_workspace_bytes(int64_t nq, int64_t n, int32_t d, int32_t R) { return sq8_plan(nq, n, d, R).total; }

// One scoring pass over `units` work units along the documents (256-document
// tiles, or for the group maxima four sampled groups per unit).
template <int kMode, int KS>
static void launch_dstat(const int8_t* q8, const float* qs, int64_t m, const DocSrc& d8, const float* ds, int64_t n,
                         int32_t d, const SqOut& o, hipStream_t stream) {
    const int64_t units = kMode == kSqGroupMax ? (o.G0 + kDsW - 1) / kDsW : (n + kDsDocs - 1) / kDsDocs;
    const int64_t nqb = (m + kDsQB - 1) / kDsQB;
    int64_t split = (1024 + units - 1) / units;  // about 1024 workgroups
    const int64_t most = nqb / 4 > 1 ? nqb / 4 : 1;  // at least four query blocks per workgroup
    split = split < most ? split : most;
    const int64_t per = (nqb + split - 1) / split;
    split = (nqb + per - 1) / per;
    if (d8.d4)
        hipLaunchKernelGGL((sq8_dstat_kernel<KS, kMode, true>), dim3((unsigned)(units * split)), dim3(kDsThreads), 0,
                           stream, q8, qs, m, DocArg<true>{d8}, ds, n, d, units, per, o);
    else
        hipLaunchKernelGGL((sq8_dstat_kernel<KS, kMode, false>), dim3((unsigned)(units * split)), dim3(kDsThreads), 0,
                           stream, q8, qs, m, DocArg<false>{d8.d8}, ds, n, d, units, per, o);
}

template <int kMode>
static hipError_t launch_scores(const int8_t* q8, const float* qs, int64_t m, const DocSrc& d8, const float* ds,
                                int64_t n, int32_t d, const SqOut& o, hipStream_t stream) {
    switch ((d + 63) / 64) {
        case 1: launch_dstat<kMode, 1>(q8, qs, m, d8, ds, n, d, o, stream); break;
        case 2: launch_dstat<kMode, 2>(q8, qs, m, d8, ds, n, d, o, stream); break;
        case 3: launch_dstat<kMode, 3>(q8, qs, m, d8, ds, n, d, o, stream); break;
        case 4: launch_dstat<kMode, 4>(q8, qs, m, d8, ds, n, d, o, stream); break;
        case 5: launch_dstat<kMode, 5>(q8, qs, m, d8, ds, n, d, o, stream); break;
        case 6: launch_dstat<kMode, 6>(q8, qs, m, d8, ds, n, d, o, stream); break;
        case 7: launch_dstat<kMode, 7>(q8, qs, m, d8, ds, n, d, o, stream); break;
        case 8: launch_dstat<kMode, 8>(q8, qs, m, d8, ds, n, d, o, stream); break;
        default: {
            const int64_t units = kMode == kSqGroupMax ? (o.G0 + 3) / 4 : (n + kSqDocs - 1) / kSqDocs;
            const int64_t qt = (m + kSqQueries - 1) / kSqQueries;
            hipLaunchKernelGGL(sq8_scores_kernel<kMode>, dim3((unsigned)(qt * units)), dim3(kSqThreads), 0, stream,
                               q8, qs, m, d8, ds, n, d, units, o);
        }
    }
    return hipGetLastError();
}

hipError_t launch_sq8_topk(const int8_t* q8, const float* qs, int64_t nq, const int8_t* d8_rows, const float* ds,
                           int64_t n, int32_t d, int32_t R, int32_t* ids, float* scores, void* ws,
                           hipStream_t stream, const uint8_t* d4, const int8_t* levels) {
    DocSrc d8{d8_rows, d4, {0, 0, 0, 0}};
    if (d4)
        for (int c = 0; c < 16; ++c) d8.lv[c >> 2] |= (uint32_t)(uint8_t)levels[c] << (8 * (c & 3));
    if (nq == 0) return hipSuccess;
    const SqPlan p = sq8_plan(nq, n, d, R);
    char* base = reinterpret_cast<char*>(ws);
    for (int64_t a = 0; a < nq; a += p.chunk) {
        const int64_t m = nq - a < p.chunk ? nq - a : p.chunk;
        const int8_t* qa = q8 + a * d;
        const float* qsa = qs + a;
        int32_t* ida = ids + a * R;
        float* sca = scores ? scores + a * R : nullptr;
        SqOut o{};
        hipError_t e;
        if (p.direct) {
            o.S = reinterpret_cast<float*>(base);
            if ((e = launch_scores<kSqWriteS>(qa, qsa, m, d8, ds, n, d, o, stream)) != hipSuccess) return e;
            if ((e = launch_rows_topk(o.S, m, (int32_t)n, R, ida, sca, stream)) != hipSuccess) return e;
            continue;
        }
        o.gmax = reinterpret_cast<float*>(base + p.off_gmax);
        o.G0 = p.G0;
        o.gstep = p.gstep;
        int32_t* tid = reinterpret_cast<int32_t*>(base + p.off_tid);
        float* tsc = reinterpret_cast<float*>(base + p.off_tsc);
        o.tau = tsc;
        o.tau_stride = R;
        o.cnt = reinterpret_cast<uint32_t*>(base + p.off_cnt);
        o.cs = reinterpret_cast<float*>(base + p.off_cs);
        o.ci = reinterpret_cast<int32_t*>(base + p.off_ci);
        o.cap = kSqCap;
        float* slots = reinterpret_cast<float*>(base + p.off_slots);
        // (1) sampled group maxima and the bound
        if ((e = launch_scores<kSqGroupMax>(qa, qsa, m, d8, ds, n, d, o, stream)) != hipSuccess) return e;
        if ((e = launch_rows_topk(o.gmax, m, p.G0, R, tid, tsc, stream)) != hipSuccess) return e;
        // (2) candidates at or above the bound
        hipLaunchKernelGGL(sq8_zero_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, stream, o.cnt, m);
        if ((e = launch_scores<kSqEmit>(qa, qsa, m, d8, ds, n, d, o, stream)) != hipSuccess) return e;
        // (3) selection of each list, (4) exact redo of overflowed lists
        if ((e = launch_list_topk(o.cs, o.ci, o.cnt, m, kSqCap, R, ida, sca, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL(sq8_fallback_kernel, dim3(kSqFb), dim3(kSqThreads), 0, stream, qa, qsa, m, d8, ds, n, d, R,
                           o.cnt, kSqCap, slots, ida, sca);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ah
