// Device-side helpers shared by the gfx950 kernels of the AH search path:
// ranking keys, wave64 primitives and a workgroup-wide exact top-K selection.
//
// Every ranking in the path orders by score descending, then id ascending
// (the kept set is then unique).  Both are packed into one 64-bit key whose
// unsigned order is exactly that ranking: high word = order-preserving image of
// the score, low word = 0xFFFFFFFF - id.  Key 0 is reserved for "no entry".
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ah {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- keys
__device__ __forceinline__ uint64_t int_key(int32_t score, int32_t id) {
    return ((uint64_t)((uint32_t)score ^ 0x80000000u) << 32) |
           (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int32_t key_int_score(uint64_t k) {
    return (int32_t)((uint32_t)(k >> 32) ^ 0x80000000u);
}
__device__ __forceinline__ int32_t key_id(uint64_t k) {
    return (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}
// Order-preserving map of a float onto uint32 (-0 and +0 map to the same value).
__device__ __forceinline__ uint32_t float_order(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t float_key(float score, int32_t id) {
    return ((uint64_t)float_order(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ float key_float_score(uint64_t k) { return order_float((uint32_t)(k >> 32)); }

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(v, o, kWave);
        if (l >= o) v += t;
    }
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// ---------------------------------------------------------------- workgroup top-K
// Scratch the selection needs in LDS.
struct SelectShared {
    uint32_t hist[256];
    uint64_t prefix;
    uint32_t need;
    uint32_t found;
    uint32_t count;
    uint32_t valid;
};

// In-place bitonic sort of a[0..P) (P a power of two) into descending order.
template <int NT>
__device__ void bitonic_sort_desc(uint64_t* a, int P) {
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (P >> 1); i += NT) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                uint64_t x = a[lo], y = a[hi];
                if ((x < y) == desc) { a[lo] = y; a[hi] = x; }
            }
            __syncthreads();
        }
    }
}

// Bitonic sort (descending) of P keys (P a power of two) in LDS by one wave,
// with no workgroup barrier: a wave's LDS accesses complete in issue order, and
// the wave-scope fence between stages keeps the compiler from reordering them.
__device__ __forceinline__ void wave_bitonic_sort_desc(uint64_t* a, int P) {
    const int lane = (int)__lane_id();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = lane; i < (P >> 1); i += 64) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t x = a[lo], y = a[hi];
                if ((x < y) == desc) { a[lo] = y; a[hi] = x; }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    }
}

__device__ __forceinline__ int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Exact K-th largest non-zero key among src(0..count) (K >= 1), by MSD radix
// select over 8-bit digits.  Returns 0 when fewer than K keys are non-zero;
// *nvalid_out receives the number of non-zero keys.  Keys must be unique.  All
// threads of the block must call it; it ends with a barrier.
template <int NT, typename Src>
__device__ uint64_t wg_kth_largest(const Src& src, int64_t count, int K, SelectShared& sh, int* nvalid_out) {
    const int tid = threadIdx.x;
    if (tid == 0) { sh.valid = 0; sh.count = 0; }
    __syncthreads();
    uint32_t v = 0;
    for (int64_t i = tid; i < count; i += NT) v += src(i) != 0;
    atomicAdd(&sh.valid, v);
    __syncthreads();
    const int nvalid = (int)sh.valid;
    *nvalid_out = nvalid;
    if (nvalid < K) return 0;
    uint64_t prefix = 0, mask = 0;
    uint32_t need = (uint32_t)K;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
        __syncthreads();
        for (int64_t i = tid; i < count; i += NT) {
            const uint64_t k = src(i);
            if (k != 0 && (k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns digits 255-4l .. 252-4l (highest digits first)
            uint32_t c[4];
            int s = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) { c[j] = sh.hist[255 - 4 * tid - j]; s += (int)c[j]; }
            const int incl = wave_inclusive_sum(s);
            uint32_t cum = (uint32_t)(incl - s);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (cum < need && cum + c[j] >= need) {
                    sh.found = (uint32_t)(255 - 4 * tid - j);
                    sh.need = need - cum;
                }
                cum += c[j];
            }
        }
        __syncthreads();
        prefix |= (uint64_t)sh.found << shift;
        mask |= 0xFFull << shift;
        need = sh.need;
        __syncthreads();
    }
    return prefix;
}

// Exact selection of the K largest non-zero keys among src(0..count), written to
// out[0..m) in descending order, m = min(K, #non-zero keys); out[m..P) is
// zero-filled, P = next_pow2(max(m,1)).  `out` must hold next_pow2(K) keys and
// live in LDS.  Keys must be unique (they are: ids are unique per query).  The
// K-th largest key is found exactly by radix select, every key not below it is
// collected, and the collection is sorted.  All threads of the block must call
// it; it ends with a barrier.
template <int NT, typename Src>
__device__ int wg_select_topk(const Src& src, int64_t count, int K, SelectShared& sh, uint64_t* out) {
    const int tid = threadIdx.x;
    int nvalid = 0;
    uint64_t kth = wg_kth_largest<NT>(src, count, K, sh, &nvalid);
    const int m = nvalid < K ? nvalid : K;
    if (nvalid <= K) kth = 1;
    const int P = next_pow2(m > 0 ? m : 1);
    for (int i = tid; i < P; i += NT) out[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < count; i += NT) {
        const uint64_t k = src(i);
        if (k != 0 && k >= kth) {
            const uint32_t pos = atomicAdd(&sh.count, 1u);
            if (pos < (uint32_t)P) out[pos] = k;
        }
    }
    __syncthreads();
    bitonic_sort_desc<NT>(out, P);
    return m;
}

// Key sources.
struct LdsKeys {
    const uint64_t* k;
    __device__ uint64_t operator()(int64_t i) const { return k[i]; }
};
struct GlobalKeysAbove {  // candidate keys, dropping those whose score is below tau
    const uint64_t* k;
    int32_t tau;
    __device__ uint64_t operator()(int64_t i) const {
        const uint64_t x = k[i];
        return key_int_score(x) >= tau ? x : 0ull;
    }
};

}  // namespace ah
