// Training-free rotation quantiser: a block-wise cascaded fast Walsh-Hadamard
// rotation with sign flips and a permutation, then per-coordinate 4-bit codes
// against a fixed 16-level Lloyd-Max codebook, with one per-row scale that
// restores the row's L2 norm in the reconstruction.
//
// Source: page "RSLM: Training-Free Vector Quantization for Approximate
// Nearest Neighbor Search", method points (block FWHT of size 128 for an O(D)
// rotation, sign flips and a permutation, an overlapping block for the tail
// dimensions; a fixed Lloyd-Max codebook of at most 16 centroids; the final
// reconstruction's norm corrected by a global scale).
//
// Readings (ah.h states them): block size b = min(128, largest power of two
// <= d); full blocks [k b, (k+1) b) first, then the tail block [d-b, d) when b
// does not divide d; y = x * signs, y'[j] = y[perm[j]] before the blocks; the
// orthonormal Sylvester Hadamard H_b / sqrt(b) per block.  Encoding: u = y *
// float32(sqrt(d) / |y|), code = number of level midpoints strictly below u
// (nearest level, ties to the lower), row step = (|y| / |L[code]|) / Lam, the
// norms' squares summed in float64.
//
// Design: rotation, one workgroup per row with the row in LDS; each stage of
// butterflies of every full block runs in parallel over the workgroup, the tail
// block after them.  Encoding, one wave per row (four per workgroup, no
// barrier), the 15 midpoints in registers.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kRotThreads = 256;

__global__ __launch_bounds__(kRotThreads) void rslm_rotate_kernel(const float* __restrict__ x, int32_t d,
                                                                  const float* __restrict__ signs,
                                                                  const int32_t* __restrict__ perm,
                                                                  float* __restrict__ y, int32_t b) {
#pragma clang fp contract(off)
    extern __shared__ float w[];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const float* xr = x + row * d;
    for (int j = tid; j < d; j += kRotThreads) {
        const int32_t p = perm[j];
        w[j] = xr[p] * signs[p];
    }
    __syncthreads();
    const float inv = 1.0f / sqrtf((float)b);
    const int nfull = d / b, half = b >> 1;
    // butterflies over the elements [base, base + len * b): len blocks of size b
    auto transform = [&](int base, int len) {
        for (int h = 1; h < b; h <<= 1) {
            for (int p = tid; p < len * half; p += kRotThreads) {
                const int blk = p / half, q = p - blk * half;
                const int i = base + blk * b + (q / h) * 2 * h + (q % h);
                const float a = w[i], c = w[i + h];
                w[i] = a + c;
                w[i + h] = a - c;
            }
            __syncthreads();
        }
        for (int j = tid; j < len * b; j += kRotThreads) w[base + j] *= inv;
        __syncthreads();
    };
    transform(0, nfull);
    if (d % b) transform(d - b, 1);
    float* yr = y + row * d;
    for (int j = tid; j < d; j += kRotThreads) yr[j] = w[j];
}

hipError_t launch_rslm_rotate(const float* x, int64_t n, int32_t d, const float* signs, const int32_t* perm,
                              float* y, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    int32_t b = 1;
    while (b * 2 <= (d < 128 ? d : 128)) b *= 2;
    const size_t lds = (size_t)d * 4;
    if (lds > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(rslm_rotate_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(rslm_rotate_kernel, dim3((unsigned)n), dim3(kRotThreads), lds, stream, x, d, signs, perm, y, b);
    return hipGetLastError();
}

struct RslmTable {
    float lv[16];
    float mid[15];
};

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__global__ __launch_bounds__(4 * kWave) void rslm_encode_kernel(const float* __restrict__ y, int64_t n, int32_t d,
                                                                RslmTable t, double lam, uint8_t* __restrict__ codes,
                                                                float* __restrict__ step) {
#pragma clang fp contract(off)
    const int lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (row >= n) return;
    const float* yr = y + row * d;
    double ss = 0.0;
    for (int j = lane; j < d; j += kWave) ss += (double)yr[j] * (double)yr[j];
    ss = wave_sum_f64(ss);
    const float f = ss > 0.0 ? (float)(sqrt((double)d) / sqrt(ss)) : 0.0f;
    // lane takes the dimension pairs (2p, 2p+1) of the bytes p = lane, lane + 64, ...
    const int nb = (d + 1) >> 1;
    double g2 = 0.0;
    uint8_t* cr = codes + row * (int64_t)nb;
    for (int p = lane; p < nb; p += kWave) {
        uint32_t byte = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int j = 2 * p + e;
            if (j >= d) break;
            const float u = yr[j] * f;
            uint32_t c = 0;
#pragma unroll
            for (int k = 0; k < 15; ++k) c += u > t.mid[k] ? 1u : 0u;
            const double l = (double)t.lv[c];
            g2 += l * l;
            byte |= c << (4 * e);
        }
        cr[p] = (uint8_t)byte;
    }
    g2 = wave_sum_f64(g2);
    if (lane == 0) step[row] = (float)(sqrt(ss) / sqrt(g2) / lam);
}

hipError_t launch_rslm_encode(const float* y, int64_t n, int32_t d, const float* levels, const float* mids,
                              double lam, uint8_t* codes, float* step, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    RslmTable t;
    for (int c = 0; c < 16; ++c) t.lv[c] = levels[c];
    for (int c = 0; c < 15; ++c) t.mid[c] = mids[c];
    hipLaunchKernelGGL(rslm_encode_kernel, dim3((unsigned)((n + 3) / 4)), dim3(4 * kWave), 0, stream, y, n, d, t, lam,
                       codes, step);
    return hipGetLastError();
}

}  // namespace ah
