// Measurement hook behind include/ah_instrument.h: a plain stream of 16-byte
// nontemporal loads over a buffer, the reference for how many bytes per second a kernel
// that reads HBM once can reach on this GPU.  Not part of the search path.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 4;  // independent 16-byte loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
    const int64_t step = (int64_t)gridDim.x * kProbeThreads * kProbeLoads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads * kProbeLoads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeLoads - 1) * kProbeThreads < n16; i += step) {
        uint4 v[kProbeLoads];
#pragma unroll
        for (int j = 0; j < kProbeLoads; ++j) {
            // nontemporal, as a read-once stream should be
            const v4u32 t = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p + i + j * kProbeThreads));
            v[j] = make_uint4(t.x, t.y, t.z, t.w);
        }
#pragma unroll
        for (int j = 0; j < kProbeLoads; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) {
        if (i + j * kProbeThreads < n16) {
            const uint4 v = p[i + j * kProbeThreads];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_read_probe(const void* data, int64_t n16, int32_t blocks_per_cu, uint32_t* sink,
                             hipStream_t stream) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)(cus * blocks_per_cu)), dim3(kProbeThreads), 0, stream,
                       reinterpret_cast<const uint4*>(data), n16, sink);
    return hipGetLastError();
}

}  // namespace ah
