// Per-query lookup table of q.center for every block of dimensions and every one
// of the 16 centers, and its int8 form with one per-query step and bias.
//
// Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
// Product Search", section "Three stages of a search" (a table of q.center per
// block); worked example: the table costs blocks x 16 x dims_per_block
// multiply-adds, negligible.  The int8 form (per-block centre folded into one
// per-query bias, one symmetric per-query step, round half to even) is this
// library's reading of "int8 with a per-query scale and bias"; ah.h states it.
//
// Design: the contraction has K = dims_per_block (1..16), far too short for a
// matrix core, and the kernel's traffic is the table it writes, so it runs on
// the vector ALUs.  One wave per query up to 64 blocks (four queries per
// workgroup, no barrier), 4 or 16 waves beyond; a thread owns four consecutive
// centres of one block (four threads per block), computes their values once
// from 16-byte codebook loads (the group's 4 x dims_per_block floats are
// contiguous), with every load of its kIt groups issued up front, and keeps
// them in registers for both the block statistics (in-thread, then 4-lane
// shuffles) and the quantisation, whose four int8 results go out as one
// 32-bit store.  Only the block centres (for the bias, summed in block order)
// and the widest range pass through LDS.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

// Group values for dims_per_block = kDpb (1, 2 or 4; 0 = any, loaded one float
// at a time): a group's four centres are 4 kDpb consecutive floats of the
// codebook (kDpb 16-byte loads) and its query slice kDpb consecutive floats.
// Each value is summed in float64 in t order (every product of two floats is
// exact in float64, so a fused multiply-add rounds only the sum) and rounded
// once to float32: the table is then a fixed function of q and the codebook,
// independent of any float32 operation order.
template <int kDpb>
__device__ __forceinline__ void group_values(const float* __restrict__ qrow, const float* __restrict__ cb, int b,
                                             int c0, int dpb, float (&v)[4]) {
    const float* cen = cb + ((int64_t)b * 16 + c0) * (kDpb ? kDpb : dpb);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if constexpr (kDpb == 0) {
        for (int t = 0; t < dpb; ++t) {
            const double qv = qrow[b * dpb + t];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __fma_rn(qv, (double)cen[j * dpb + t], acc[j]);
        }
    } else {
        float c[4 * kDpb], qq[kDpb];
#pragma unroll
        for (int k = 0; k < kDpb; ++k) {
            const float4 x = reinterpret_cast<const float4*>(cen)[k];
            c[4 * k] = x.x;
            c[4 * k + 1] = x.y;
            c[4 * k + 2] = x.z;
            c[4 * k + 3] = x.w;
        }
        if constexpr (kDpb == 1) {
            qq[0] = qrow[b];
        } else if constexpr (kDpb == 2) {
            const float2 x = reinterpret_cast<const float2*>(qrow)[b];
            qq[0] = x.x;
            qq[1] = x.y;
        } else {
            const float4 x = reinterpret_cast<const float4*>(qrow)[b];
            qq[0] = x.x;
            qq[1] = x.y;
            qq[2] = x.z;
            qq[3] = x.w;
        }
#pragma unroll
        for (int t = 0; t < kDpb; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __fma_rn((double)qq[t], (double)c[j * kDpb + t], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __double2float_rn(acc[j]);
}

// kWq waves per query (1, 4 or 16), kIt groups of four centres per thread; a
// workgroup of max(256, 64 kWq) threads holds 4 / kWq queries (one when kWq >= 4).
template <int kWq, int kIt, int kDpb>
__global__ __launch_bounds__(kWq >= 4 ? kWq * kWave : 4 * kWave) void build_lut_kernel(
    const float* __restrict__ q, int64_t nq, int32_t d, const float* __restrict__ cb, int32_t B, int32_t dpb,
    float* __restrict__ lut_f32, int8_t* __restrict__ lut_i8, float* __restrict__ scale,
    float* __restrict__ bias, bool vec_out) {
    constexpr int kQs = kWq >= 4 ? 1 : 4 / kWq;                    // queries per workgroup
    constexpr int kTq = kWq * kWave;                               // threads per query
    constexpr int kMid = kWq == 1 ? 16 * kIt : AH_LUT_MAX_BLOCKS;  // blocks per query slot
    __shared__ __align__(16) float mid_all[kQs][kMid];
    __shared__ float wmax_all[kQs][kWq];
    const int tid = threadIdx.x;
    const int qs = tid / kTq, tq = tid % kTq;
    const int64_t qi = (int64_t)blockIdx.x * kQs + qs;
    if (kQs > 1 && qi >= nq) return;  // whole waves leave; no workgroup barrier when kWq == 1
    float* mid_s = mid_all[qs];
    const float* qrow = q + qi * d;
    const int G = B * 4;  // groups of four centres
    const int c0 = (tq & 3) * 4;
    float v[kIt][4];
#pragma unroll
    for (int i = 0; i < kIt; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][j] = 0.0f;
    // table values: v[i][j] = sum_t q[b*dpb + t] * cb[b][c0 + j][t] (float64 in t order, rounded once)
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
        const int g = tq + i * kTq;
        if (g < G) group_values<kDpb>(qrow, cb, g >> 2, c0, dpb, v[i]);
    }
    // block statistics: centre (lo + hi) / 2 and the widest range
    float mid[kIt];
    float wmax = 0.0f;
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
        float lo = fminf(fminf(v[i][0], v[i][1]), fminf(v[i][2], v[i][3]));
        float hi = fmaxf(fmaxf(v[i][0], v[i][1]), fmaxf(v[i][2], v[i][3]));
#pragma unroll
        for (int o = 2; o > 0; o >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, o, 4));
            hi = fmaxf(hi, __shfl_xor(hi, o, 4));
        }
        const float sum = lo + hi;
        mid[i] = 0.5f * sum;
        const int g = tq + i * kTq;
        if (g < G) {
            if ((tq & 3) == 0) mid_s[g >> 2] = mid[i];
            wmax = fmaxf(wmax, hi - lo);
            if (lut_f32) {
                float* dst = lut_f32 + qi * (int64_t)G * 4 + (int64_t)g * 4;
                if (vec_out) {
                    *reinterpret_cast<float4*>(dst) = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) dst[j] = v[i][j];
                }
            }
        }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, o, kWave));
    float rng = wmax;
    if constexpr (kWq == 1) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    } else {
        if ((tq & (kWave - 1)) == 0) wmax_all[qs][tq / kWave] = wmax;
        __syncthreads();
        rng = wmax_all[qs][0];
#pragma unroll
        for (int w = 1; w < kWq; ++w) rng = fmaxf(rng, wmax_all[qs][w]);
    }

    if (tq == 0) {
        float beta = 0.0f;
#pragma unroll 16
        for (int b = 0; b < B; ++b) beta = beta + mid_s[b];  // block order, fp32
        bias[qi] = beta;
        scale[qi] = rng > 0.0f ? rng / 254.0f : 0.0f;
    }

    // quantise: round half to even, clamp to +-127, four codes per 32-bit store
    const float inv = rng > 0.0f ? 254.0f / rng : 0.0f;
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
        const int g = tq + i * kTq;
        if (g >= G) break;
        uint32_t packed = 0;
        if (rng > 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float diff = v[i][j] - mid[i];
                float r = rintf(diff * inv);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                packed |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * j);
            }
        }
        int8_t* dst = lut_i8 + qi * (int64_t)G * 4 + (int64_t)g * 4;
        if (vec_out) {
            *reinterpret_cast<uint32_t*>(dst) = packed;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j] = (int8_t)(packed >> (8 * j));
        }
    }
}

template <int kWq, int kIt, int kDpb>
static void launch_lut(const float* q, int64_t nq, int32_t d, const float* cb, int32_t B, int32_t dpb,
                       float* lut_f32, int8_t* lut_i8, float* scale, float* bias, bool vec_out,
                       hipStream_t stream) {
    constexpr int kQs = kWq >= 4 ? 1 : 4 / kWq;
    constexpr int kThreads = kWq >= 4 ? kWq * kWave : 4 * kWave;
    hipLaunchKernelGGL((build_lut_kernel<kWq, kIt, kDpb>), dim3((unsigned)((nq + kQs - 1) / kQs)), dim3(kThreads), 0,
                       stream, q, nq, d, cb, B, dpb, lut_f32, lut_i8, scale, bias, vec_out);
}

hipError_t launch_build_lut(const float* q, int64_t nq, int32_t d, const float* cb, int32_t B,
                            int32_t dpb, float* lut_f32, int8_t* lut_i8, float* scale, float* bias,
                            hipStream_t stream) {
    if (nq == 0) return hipSuccess;
    if (B > AH_LUT_MAX_BLOCKS) return hipErrorInvalidValue;  // 16 waves x 16 groups x 4 centres
    // whole-group stores need a 4-byte aligned int8 table and a 16-byte aligned fp32 one
    const bool vec_out =
        !(reinterpret_cast<uintptr_t>(lut_i8) & 3) && !(lut_f32 && (reinterpret_cast<uintptr_t>(lut_f32) & 15));
    // whole-group loads need 16-byte aligned codebooks and query rows
    const bool vec_in = !(reinterpret_cast<uintptr_t>(cb) & 15) && !(reinterpret_cast<uintptr_t>(q) & 15);
    const int kd = vec_in && (dpb == 1 || dpb == 2 || dpb == 4) ? dpb : 0;
    // one wave per query up to 64 blocks, then four, then sixteen
    const int G = B * 4;
#define AH_LUT_D(W, I, D) launch_lut<W, I, D>(q, nq, d, cb, B, dpb, lut_f32, lut_i8, scale, bias, vec_out, stream)
#define AH_LUT(W, I)            \
    do {                        \
        if (kd == 1)            \
            AH_LUT_D(W, I, 1);  \
        else if (kd == 2)       \
            AH_LUT_D(W, I, 2);  \
        else if (kd == 4)       \
            AH_LUT_D(W, I, 4);  \
        else                    \
            AH_LUT_D(W, I, 0);  \
    } while (0)
    if (G <= 64) AH_LUT(1, 1);
    else if (G <= 128) AH_LUT(1, 2);
    else if (G <= 256) AH_LUT(1, 4);
    else if (G <= 512) AH_LUT(4, 2);
    else if (G <= 1024) AH_LUT(4, 4);
    else if (G <= 2048) AH_LUT(16, 2);
    else if (G <= 4096) AH_LUT(16, 4);
    else if (G <= 8192) AH_LUT(16, 8);
    else AH_LUT(16, 16);
#undef AH_LUT
#undef AH_LUT_D
    return hipGetLastError();
}

}  // namespace ah
