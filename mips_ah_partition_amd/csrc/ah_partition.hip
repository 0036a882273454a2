// Centroid scoring and leaf choice: S = Q . C^T in fp32, then the best nl leaves
// of each query by (score desc, leaf id asc).
//
// Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
// Product Search", section "Three stages of a search" (a query scores every
// centroid and descends into the best num_leaves_to_search) and the worked
// example (1,000 centroids x 128 dims of multiply-adds per query).
//
// Design: a dense fp32 contraction (M = queries, N = leaves, K = d) on the
// gfx950 matrix cores with v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate;
// bf16 inputs would not hold the 1e-4 relative bound).  Workgroup tile 64 x 64,
// four waves of 32 x 32, K staged through LDS 32 at a time with rows padded to
// 36 floats so the 16-byte operand reads are bank-conflict free.  Within each
// group of four k-steps a lane feeds k = 4*(lane/16) + j, so one ds_read_b128
// serves four MFMAs; A and B use the same k permutation, which leaves the
// contraction unchanged.  Scores go to the workspace; a second kernel selects
// each query's best nl with the exact workgroup top-K selection.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kGemmThreads = 256;
constexpr int kGT = 64;       // tile rows / cols
constexpr int kGK = 32;       // K per LDS stage
constexpr int kGS = kGK + 4;  // padded row stride (floats)

__global__ __launch_bounds__(kGemmThreads) void centroid_scores_kernel(
    const float* __restrict__ q, int64_t nq, int32_t d, const float* __restrict__ cent, int32_t L,
    float* __restrict__ S) {
    __shared__ __align__(16) float qa[kGT * kGS];
    __shared__ __align__(16) float cb[kGT * kGS];
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int64_t ntl = (L + kGT - 1) / kGT;  // leaf tiles; consecutive blocks share a query tile
    const int64_t q0 = ((int64_t)blockIdx.x / ntl) * kGT;
    const int64_t l0 = ((int64_t)blockIdx.x % ntl) * kGT;
    const int wm = (w >> 1) * 32, wn = (w & 1) * 32;  // wave's 32x32 sub-tile
    v4f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < d; k0 += kGK) {
        // stage 64 x 32 of Q and of C (zero beyond the edges)
        for (int e = tid; e < kGT * kGK; e += kGemmThreads) {
            const int r = e / kGK, kk = e % kGK;
            const int64_t qr = q0 + r, lr = l0 + r;
            const int kd = k0 + kk;
            qa[r * kGS + kk] = (qr < nq && kd < d) ? q[qr * d + kd] : 0.0f;
            cb[r * kGS + kk] = (lr < L && kd < d) ? cent[lr * d + kd] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < kGK; kb += 16) {
            const int kk = kb + 4 * (lane >> 4);
            float4 av[2], bv[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                av[a] = *reinterpret_cast<const float4*>(&qa[(wm + 16 * a + (lane & 15)) * kGS + kk]);
#pragma unroll
            for (int b = 0; b < 2; ++b)
                bv[b] = *reinterpret_cast<const float4*>(&cb[(wn + 16 * b + (lane & 15)) * kGS + kk]);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].x, bv[b].x, acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].y, bv[b].y, acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].z, bv[b].z, acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].w, bv[b].w, acc[a][b], 0, 0, 0);
                }
        }
        __syncthreads();
    }
    // D[row][col]: lane holds rows 4*(lane/16)+i of column lane%16
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t qr = q0 + wm + 16 * a + 4 * (lane >> 4) + i;
                const int64_t lc = l0 + wn + 16 * b + (lane & 15);
                if (qr < nq && lc < L) S[qr * L + lc] = acc[a][b][i];
            }
}

struct ScoreKeys {
    const float* s;
    __device__ uint64_t operator()(int64_t i) const { return float_key(s[i], (int32_t)i); }
};

constexpr int kSelThreads = 256;

__global__ __launch_bounds__(kSelThreads) void leaf_select_kernel(const float* __restrict__ S, int32_t L,
                                                                  int32_t nl, int32_t* __restrict__ leaves,
                                                                  float* __restrict__ scores) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ SelectShared sh;
    uint64_t* sel = reinterpret_cast<uint64_t*>(smem);
    const int64_t qi = blockIdx.x;
    const int m = wg_select_topk<kSelThreads>(ScoreKeys{S + qi * L}, L, nl, sh, sel);
    for (int r = threadIdx.x; r < nl; r += kSelThreads) {
        leaves[qi * nl + r] = r < m ? key_id(sel[r]) : -1;
        if (scores) scores[qi * nl + r] = r < m ? key_float_score(sel[r]) : -__builtin_huge_valf();
    }
}

size_t partition_workspace_bytes(int64_t nq, int32_t L) { return (size_t)nq * (size_t)L * 4 + 256; }

hipError_t launch_partition(const float* q, int64_t nq, int32_t d, const float* cent, int32_t L,
                            int32_t nl, int32_t* leaves, float* scores, void* ws, hipStream_t stream) {
    if (nq == 0) return hipSuccess;
    float* S = reinterpret_cast<float*>(ws);
    dim3 grid((unsigned)(((L + kGT - 1) / kGT) * ((nq + kGT - 1) / kGT)));
    hipLaunchKernelGGL(centroid_scores_kernel, grid, dim3(kGemmThreads), 0, stream, q, nq, d, cent, L, S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int Kp = 1;
    while (Kp < nl) Kp <<= 1;
    if ((size_t)Kp * 8 > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(leaf_select_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, Kp * 8);
    hipLaunchKernelGGL(leaf_select_kernel, dim3((unsigned)nq), dim3(kSelThreads), (size_t)Kp * 8, stream,
                       S, L, nl, leaves, scores);
    return hipGetLastError();
}

}  // namespace ah
