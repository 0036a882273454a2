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
// the vector ALUs.  One workgroup per query; a 16-lane group owns one block,
// so the per-block min/max is a 16-lane shuffle reduction.  The table value is
// computed twice (once for the block statistics, once to quantise) with the
// same instruction sequence, which keeps both passes bit-identical without
// staging the whole table in LDS.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kLutThreads = 256;

__device__ __forceinline__ float table_entry(const float* __restrict__ qrow,
                                             const float* __restrict__ cb, int b, int c, int dpb) {
    const float* cen = cb + ((int64_t)b * 16 + c) * dpb;
    const float* qb = qrow + (int64_t)b * dpb;
    float v = 0.0f;
    for (int t = 0; t < dpb; ++t) v = __fmaf_rn(qb[t], cen[t], v);
    return v;
}

__global__ __launch_bounds__(kLutThreads) void build_lut_kernel(
    const float* __restrict__ q, int32_t d, const float* __restrict__ cb, int32_t B, int32_t dpb,
    float* __restrict__ lut_f32, int8_t* __restrict__ lut_i8, float* __restrict__ scale,
    float* __restrict__ bias) {
    __shared__ float mid_s[AH_LUT_MAX_BLOCKS];
    __shared__ float wmax_s[kLutThreads / kWave];
    const int64_t qi = blockIdx.x;
    const float* qrow = q + qi * d;
    const int tid = threadIdx.x;
    const int c = tid & 15;
    const int E = B * 16;

    // pass 1: block centres and the widest block range
    float wmax = 0.0f;
    for (int base = 0; base < E; base += kLutThreads) {
        const int e = base + tid;
        const int b = e >> 4;
        const bool ok = e < E;
        float v = ok ? table_entry(qrow, cb, b, c, dpb) : 0.0f;
        if (ok && lut_f32) lut_f32[qi * E + e] = v;
        float lo = v, hi = v;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, o, 16));
            hi = fmaxf(hi, __shfl_xor(hi, o, 16));
        }
        if (ok) {
            if (c == 0) {
                const float sum = lo + hi;
                mid_s[b] = 0.5f * sum;
            }
            wmax = fmaxf(wmax, hi - lo);
        }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, o, kWave));
    if ((tid & (kWave - 1)) == 0) wmax_s[tid / kWave] = wmax;
    __syncthreads();
    float rng = wmax_s[0];
#pragma unroll
    for (int w = 1; w < kLutThreads / kWave; ++w) rng = fmaxf(rng, wmax_s[w]);

    if (tid == 0) {
        float beta = 0.0f;
        for (int b = 0; b < B; ++b) beta = beta + mid_s[b];  // block order, fp32
        bias[qi] = beta;
        scale[qi] = rng > 0.0f ? rng / 254.0f : 0.0f;
    }

    // pass 2: quantise
    const float inv = rng > 0.0f ? 254.0f / rng : 0.0f;
    for (int base = 0; base < E; base += kLutThreads) {
        const int e = base + tid;
        if (e >= E) break;
        const int b = e >> 4;
        int8_t out = 0;
        if (rng > 0.0f) {
            const float v = table_entry(qrow, cb, b, c, dpb);
            const float diff = v - mid_s[b];
            float r = rintf(diff * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            out = (int8_t)(int)r;
        }
        lut_i8[qi * E + e] = out;
    }
}

hipError_t launch_build_lut(const float* q, int64_t nq, int32_t d, const float* cb, int32_t B,
                            int32_t dpb, float* lut_f32, int8_t* lut_i8, float* scale, float* bias,
                            hipStream_t stream) {
    if (nq == 0) return hipSuccess;
    hipLaunchKernelGGL(build_lut_kernel, dim3((unsigned)nq), dim3(kLutThreads), 0, stream, q, d, cb,
                       B, dpb, lut_f32, lut_i8, scale, bias);
    return hipGetLastError();
}

}  // namespace ah
