// The center update of anisotropic codebook training, block by block.
//
// Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
// Product Search", section "Training an anisotropic codebook yourself" (the
// update is a closed-form linear solve per center; eta = 1 gives k-means) and
// its note that the blocks' codes are coupled through the parallel residual.
// With the other blocks' centers fixed, block b's center c minimises
// sum_i (eta-1)(s_i - p_ib + u_ib.(x_ib - c))^2 + |x_ib - c|^2 over its rows,
// i.e. solves
//     sum_i [(eta-1) u_ib u_ib^T + I] c = sum_i [x_ib + (eta-1)(s_i - p_ib + u_ib.x_ib) u_ib]
// (u = x/|x|, p_ib = u_ib.(x_ib - center), s_i = sum_b p_ib at the current
// centers).  Blocks go in order; after block b its p_ib and s_i are refreshed.
//
// Design: per block three launches.  Accumulate: each workgroup sums its rows'
// (dpb x dpb matrix, right-hand side, count) per center in LDS with float64
// atomics, then adds them to the global sums; solve: one thread per center,
// Gaussian elimination with partial pivoting in float64 (a center with no rows,
// or a singular system, keeps its value), which also clears the global sums for
// the next block; refresh: one thread per row.  The float64 sums are taken in
// no fixed order, so results agree with a row-order sum to float64 rounding.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kTrMaxDpb = 16;
constexpr int kTrThreads = 256;

struct TrainState {
    double* invn;  // [n]
    double* p;     // [n][B]
    double* s;     // [n]
    double* acc;   // [16][dpb*dpb + dpb + 1]
};

static size_t tr_align(size_t x) { return (x + 255) & ~(size_t)255; }

size_t pq_update_workspace_bytes(int64_t n, int32_t B, int32_t dpb) {
    const size_t n1 = (size_t)(n > 0 ? n : 1);
    return tr_align(n1 * 8) + tr_align(n1 * (size_t)B * 8) + tr_align(n1 * 8) +
           tr_align((size_t)16 * (dpb * dpb + dpb + 1) * 8);
}

__device__ __forceinline__ int code_at(const uint8_t* codes, int32_t stride, int64_t i, int b) {
    return (codes[i * (int64_t)stride + (b >> 1)] >> (4 * (b & 1))) & 15;
}

__global__ void pq_init_kernel(const float* __restrict__ x, int64_t n, int32_t d, const uint8_t* __restrict__ codes,
                               int32_t stride, int32_t B, int32_t dpb, const float* __restrict__ cb, TrainState st,
                               int32_t nacc) {
#pragma clang fp contract(off)
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < 16 * (int64_t)nacc) st.acc[i] = 0.0;
    if (i >= n) return;
    const float* xr = x + i * d;
    double ss = 0.0;
    for (int j = 0; j < d; ++j) ss += (double)xr[j] * (double)xr[j];
    const double invn = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
    st.invn[i] = invn;
    double s = 0.0;
    for (int b = 0; b < B; ++b) {
        const float* cen = cb + ((int64_t)b * 16 + code_at(codes, stride, i, b)) * dpb;
        double pr = 0.0;
        for (int t = 0; t < dpb; ++t) {
            const double xv = xr[b * dpb + t];
            pr += (xv * invn) * (xv - (double)cen[t]);
        }
        st.p[i * B + b] = pr;
        s += pr;
    }
    st.s[i] = s;
}

__global__ __launch_bounds__(kTrThreads) void pq_accumulate_kernel(const float* __restrict__ x, int64_t n, int32_t d,
                                                                    const uint8_t* __restrict__ codes, int32_t stride,
                                                                    int32_t B, int32_t dpb, double eta, int32_t b,
                                                                    TrainState st, int32_t nacc) {
#pragma clang fp contract(off)
    extern __shared__ double lacc[];  // [16][nacc]
    for (int e = threadIdx.x; e < 16 * nacc; e += kTrThreads) lacc[e] = 0.0;
    __syncthreads();
    const double em1 = eta - 1.0;
    for (int64_t i = (int64_t)blockIdx.x * kTrThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kTrThreads) {
        const int c = code_at(codes, stride, i, b);
        const float* xb = x + i * d + (int64_t)b * dpb;
        double u[kTrMaxDpb], ux = 0.0;
        for (int t = 0; t < dpb; ++t) {
            u[t] = (double)xb[t] * st.invn[i];
            ux += u[t] * (double)xb[t];
        }
        const double w = em1 * (st.s[i] - st.p[i * B + b] + ux);
        double* a = lacc + c * nacc;
        for (int r = 0; r < dpb; ++r) {
            for (int t = 0; t < dpb; ++t) unsafeAtomicAdd(&a[r * dpb + t], em1 * u[r] * u[t] + (r == t ? 1.0 : 0.0));
            unsafeAtomicAdd(&a[dpb * dpb + r], (double)xb[r] + w * u[r]);
        }
        unsafeAtomicAdd(&a[dpb * dpb + dpb], 1.0);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * nacc; e += kTrThreads)
        if (lacc[e] != 0.0) unsafeAtomicAdd(&st.acc[e], lacc[e]);
}

__global__ void pq_solve_kernel(int32_t B, int32_t dpb, int32_t b, float* __restrict__ cb, TrainState st,
                                int32_t nacc) {
#pragma clang fp contract(off)
    const int c = threadIdx.x;
    if (c >= 16) return;
    double A[kTrMaxDpb * kTrMaxDpb], r[kTrMaxDpb];
    double* g = st.acc + c * nacc;
    for (int e = 0; e < dpb * dpb; ++e) A[e] = g[e];
    for (int e = 0; e < dpb; ++e) r[e] = g[dpb * dpb + e];
    const double cnt = g[dpb * dpb + dpb];
    for (int e = 0; e < nacc; ++e) g[e] = 0.0;  // ready for the next block
    if (cnt == 0.0) return;
    for (int k = 0; k < dpb; ++k) {
        int piv = k;
        for (int a = k + 1; a < dpb; ++a)
            if (fabs(A[a * dpb + k]) > fabs(A[piv * dpb + k])) piv = a;
        if (A[piv * dpb + k] == 0.0) return;  // singular: the center keeps its value
        if (piv != k) {
            for (int t = 0; t < dpb; ++t) {
                const double tmp = A[k * dpb + t];
                A[k * dpb + t] = A[piv * dpb + t];
                A[piv * dpb + t] = tmp;
            }
            const double tmp = r[k];
            r[k] = r[piv];
            r[piv] = tmp;
        }
        for (int a = k + 1; a < dpb; ++a) {
            const double f = A[a * dpb + k] / A[k * dpb + k];
            for (int t = k; t < dpb; ++t) A[a * dpb + t] -= f * A[k * dpb + t];
            r[a] -= f * r[k];
        }
    }
    for (int k = dpb - 1; k >= 0; --k) {
        double v = r[k];
        for (int t = k + 1; t < dpb; ++t) v -= A[k * dpb + t] * r[t];
        r[k] = v / A[k * dpb + k];
    }
    for (int t = 0; t < dpb; ++t) cb[((int64_t)b * 16 + c) * dpb + t] = (float)r[t];
}

__global__ void pq_refresh_kernel(const float* __restrict__ x, int64_t n, int32_t d, const uint8_t* __restrict__ codes,
                                  int32_t stride, int32_t B, int32_t dpb, int32_t b, const float* __restrict__ cb,
                                  TrainState st) {
#pragma clang fp contract(off)
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float* cen = cb + ((int64_t)b * 16 + code_at(codes, stride, i, b)) * dpb;
    const float* xb = x + i * d + (int64_t)b * dpb;
    double pr = 0.0;
    for (int t = 0; t < dpb; ++t) {
        const double xv = xb[t];
        pr += (xv * st.invn[i]) * (xv - (double)cen[t]);
    }
    st.s[i] += pr - st.p[i * B + b];
    st.p[i * B + b] = pr;
}

hipError_t launch_pq_update(const float* x, int64_t n, int32_t d, const uint8_t* codes, int32_t stride, int32_t B,
                            int32_t dpb, double eta, float* cb, void* ws, hipStream_t stream) {
    const size_t n1 = (size_t)(n > 0 ? n : 1);
    char* base = reinterpret_cast<char*>(ws);
    TrainState st;
    st.invn = reinterpret_cast<double*>(base);
    st.p = reinterpret_cast<double*>(base + tr_align(n1 * 8));
    st.s = reinterpret_cast<double*>(base + tr_align(n1 * 8) + tr_align(n1 * (size_t)B * 8));
    st.acc = reinterpret_cast<double*>(base + tr_align(n1 * 8) + tr_align(n1 * (size_t)B * 8) + tr_align(n1 * 8));
    const int32_t nacc = dpb * dpb + dpb + 1;
    const int64_t cover = n > 16 * nacc ? n : 16 * nacc;
    const unsigned g1 = (unsigned)((cover + 255) / 256);
    hipLaunchKernelGGL(pq_init_kernel, dim3(g1), dim3(256), 0, stream, x, n, d, codes, stride, B, dpb, cb, st, nacc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0) return e;
    const int64_t wgs = (n + kTrThreads - 1) / kTrThreads;
    const unsigned ga = (unsigned)(wgs < 1024 ? wgs : 1024);
    const size_t lds = (size_t)16 * nacc * 8;
    if (lds > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(pq_accumulate_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const unsigned gr = (unsigned)((n + 255) / 256);
    for (int32_t b = 0; b < B; ++b) {
        hipLaunchKernelGGL(pq_accumulate_kernel, dim3(ga), dim3(kTrThreads), lds, stream, x, n, d, codes, stride, B, dpb,
                           eta, b, st, nacc);
        hipLaunchKernelGGL(pq_solve_kernel, dim3(1), dim3(64), 0, stream, B, dpb, b, cb, st, nacc);
        hipLaunchKernelGGL(pq_refresh_kernel, dim3(gr), dim3(256), 0, stream, x, n, d, codes, stride, B, dpb, b, cb, st);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ah
