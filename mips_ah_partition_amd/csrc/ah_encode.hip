// Anisotropic coupled encoding of rows with given per-block codebooks: the
// step that produces the codes the query path scans.
//
// Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
// Product Search", sections "The loss in one paragraph" (a row's loss is
// (eta - 1) (u.r)^2 + |r|^2 for its residual r and direction u) and "Training
// an anisotropic codebook yourself" (block choices are coupled through u.r and
// are refined iteratively).  Reading taken for the refinement: block-coordinate
// descent from the per-block nearest centers, `sweeps` sweeps over b = 0..B-1,
// each block taking the center that minimises the row's loss with the other
// blocks fixed (lowest index on ties).
//
// Design: rows are independent, one thread per row, no barriers.  Every lane
// of a wave visits the same block and center at the same time, so codebook
// reads are wave-uniform (scalar loads).  The decision is an argmin of float64
// losses computed in one fixed order (x_t / |x| formed as x_t * (1 / |x|),
// per-block sums over t in order, loss = ((eta - 1) par) par + |r_b|^2 with
// par = (s - p_b(current)) + p_b(candidate)), with contraction into fused
// multiply-adds switched off, so the codes are reproducible bit for bit.  The
// per-block parallel terms are recomputed from the current code instead of
// stored, which gives the same float64 values.  Bound: float64 vector ALU
// (16 dpb x 5 + 4 flops per block and candidate per sweep).
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kEncThreads = 256;

template <bool kBf16>
__device__ __forceinline__ double row_elem(const void* rows, int64_t idx) {
    if (kBf16) return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(rows)[idx] << 16);
    return (double)reinterpret_cast<const float*>(rows)[idx];
}

// kDpb: dims per block as a constant (1, 2 or 4), or 0 to read it from dpb_rt
template <int kDpb, bool kBf16>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(const void* __restrict__ rows, int64_t n, int32_t d,
                                                             const float* __restrict__ cb, int32_t B, int32_t dpb_rt,
                                                             double eta, int32_t sweeps, uint8_t* __restrict__ codes,
                                                             int32_t stride, bool vec_rows, bool from_codes) {
#pragma clang fp contract(off)
    constexpr int kMaxDpb = 16;
    const int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
    if (i >= n) return;
    const int dpb = kDpb ? kDpb : dpb_rt;
    const int64_t base = i * d;
    double ss = 0.0;
    for (int j = 0; j < d; ++j) {
        const double x = row_elem<kBf16>(rows, base + j);
        ss += x * x;
    }
    const double invn = ss > 0.0 ? 1.0 / __dsqrt_rn(ss) : 0.0;
    const double em1 = eta - 1.0;
    uint8_t* row = codes + i * (int64_t)stride;
    for (int k = (B + 1) / 2; k < stride; ++k) row[k] = 0;

    double xb[kMaxDpb], xi[kMaxDpb];  // the block's values and x_t * (1 / |x|)
    // The row is read in chunks of 128 bytes (eight 16-byte loads per lane, so
    // each cache line a wave touches is used whole, within a few instructions)
    // when rows are 16-byte aligned and dpb is a constant; a block's values are
    // then picked from the chunk's registers by a wave-uniform index.
    constexpr int kVals = kBf16 ? 8 : 4;  // values per 16-byte load
    constexpr int kLd = kBf16 ? 8 : 4;    // loads per chunk (128 or 64 bytes)
    constexpr int kCW = 4 * kLd;          // dwords per chunk
    uint32_t chunk[kCW];
    int chunk_v0 = -1;  // first value of the chunk in registers
    const bool vec = kDpb != 0 && vec_rows;
    auto load_block = [&](int b) {
        if (kDpb != 0 && vec) {
            const int v = b * kDpb, v0 = v - v % (kVals * kLd);
            if (v0 != chunk_v0) {
                const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rows) +
                                                                  (base + v0) * (kBf16 ? 2 : 4));
#pragma unroll
                for (int k = 0; k < kLd; ++k) {
                    const uint4 u = v0 + k * kVals < d ? src[k] : make_uint4(0, 0, 0, 0);
                    chunk[4 * k] = u.x;
                    chunk[4 * k + 1] = u.y;
                    chunk[4 * k + 2] = u.z;
                    chunk[4 * k + 3] = u.w;
                }
                chunk_v0 = v0;
            }
#pragma unroll
            for (int t = 0; t < (kDpb ? kDpb : 1); ++t) {
                const int e = v - v0 + t;  // value index within the chunk (wave-uniform)
                if (kBf16) {
                    const uint32_t w = chunk[(e >> 1) & (kCW - 1)];
                    xb[t] = (double)__uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                } else {  // a dword pair, then the half (indexing single dwords here spilled to scratch)
                    const uint32_t lo = chunk[((e >> 1) << 1) & (kCW - 1)], hi = chunk[(((e >> 1) << 1) + 1) & (kCW - 1)];
                    xb[t] = (double)__uint_as_float((e & 1) ? hi : lo);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < (kDpb ? kDpb : kMaxDpb); ++t)
                if (kDpb || t < dpb) xb[t] = row_elem<kBf16>(rows, base + (int64_t)b * dpb + t);
        }
#pragma unroll
        for (int t = 0; t < (kDpb ? kDpb : kMaxDpb); ++t)
            if (kDpb || t < dpb) xi[t] = xb[t] * invn;
    };
    // p_b(c) = sum_t (x_t * invn) * (x_t - c_t) and |x_b - c|^2, t in order
    auto terms = [&](const float* cen, double& p, double& nr) {
        p = 0.0;
        nr = 0.0;
#pragma unroll
        for (int t = 0; t < (kDpb ? kDpb : kMaxDpb); ++t) {
            if (kDpb || t < dpb) {
                const double r = xb[t] - (double)cen[t];
                p += xi[t] * r;
                nr += r * r;
            }
        }
    };
    // |x_b - c|^2 alone (the nearest-center start)
    auto dist2 = [&](const float* cen) {
        double nr = 0.0;
#pragma unroll
        for (int t = 0; t < (kDpb ? kDpb : kMaxDpb); ++t) {
            if (kDpb || t < dpb) {
                const double r = xb[t] - (double)cen[t];
                nr += r * r;
            }
        }
        return nr;
    };
    auto get_code = [&](int b) -> int { return (row[b >> 1] >> (4 * (b & 1))) & 15; };

    // per-block nearest centers (unless the sweeps start from the given codes);
    // a byte is written once both of its nibbles are known
    uint32_t pend = 0;
    for (int b = 0; b < (from_codes ? 0 : B); ++b) {
        load_block(b);
        double best = __builtin_huge_val();
        int bc = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {  // unrolled: the block's codebook loads issue together
            const double nr = dist2(cb + ((int64_t)b * 16 + c) * dpb);
            if (nr < best) {
                best = nr;
                bc = c;
            }
        }
        pend |= (uint32_t)bc << (4 * (b & 1));
        if ((b & 1) || b == B - 1) {
            row[b >> 1] = (uint8_t)pend;
            pend = 0;
        }
    }
    for (int sw = 0; sw < sweeps; ++sw) {
        double s = 0.0;
        for (int b = 0; b < B; ++b) {
            load_block(b);
            double p, nr;
            terms(cb + ((int64_t)b * 16 + get_code(b)) * dpb, p, nr);
            s += p;
        }
        uint32_t byte = 0;
        for (int b = 0; b < B; ++b) {
            if (!(b & 1)) byte = row[b >> 1];
            load_block(b);
            double pc, nrc;
            terms(cb + ((int64_t)b * 16 + ((byte >> (4 * (b & 1))) & 15)) * dpb, pc, nrc);
            const double sm = s - pc;
            double best = __builtin_huge_val(), bp = 0.0;
            int bc = 0;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                double p, nr;
                terms(cb + ((int64_t)b * 16 + c) * dpb, p, nr);
                const double par = sm + p;
                const double L = (em1 * par) * par + nr;
                if (L < best) {
                    best = L;
                    bc = c;
                    bp = p;
                }
            }
            byte = (byte & ~(15u << (4 * (b & 1)))) | ((uint32_t)bc << (4 * (b & 1)));
            s = sm + bp;
            if ((b & 1) || b == B - 1) row[b >> 1] = (uint8_t)byte;
        }
    }
}

template <int kDpb, bool kBf16>
static void launch_enc(const void* rows, int64_t n, int32_t d, const float* cb, int32_t B, int32_t dpb, double eta,
                       int32_t sweeps, uint8_t* codes, int32_t stride, bool from_codes, hipStream_t stream) {
    // chunked row reads: 16-byte aligned rows
    const bool vec_rows = (reinterpret_cast<uintptr_t>(rows) & 15) == 0 && ((size_t)d * (kBf16 ? 2 : 4)) % 16 == 0;
    hipLaunchKernelGGL((encode_kernel<kDpb, kBf16>), dim3((unsigned)((n + kEncThreads - 1) / kEncThreads)),
                       dim3(kEncThreads), 0, stream, rows, n, d, cb, B, dpb, eta, sweeps, codes, stride, vec_rows,
                       from_codes);
}

hipError_t launch_encode(const void* rows, int32_t dtype, int64_t n, int32_t d, const float* cb, int32_t B,
                         int32_t dpb, double eta, int32_t sweeps, uint8_t* codes, int32_t stride,
                         hipStream_t stream, bool from_codes) {
    if (n == 0) return hipSuccess;
    const bool bf = dtype != 0;
#define AH_ENC(D)                                                                                           \
    do {                                                                                                    \
        if (bf) launch_enc<D, true>(rows, n, d, cb, B, dpb, eta, sweeps, codes, stride, from_codes, stream); \
        else launch_enc<D, false>(rows, n, d, cb, B, dpb, eta, sweeps, codes, stride, from_codes, stream);  \
    } while (0)
    if (dpb == 1) AH_ENC(1);
    else if (dpb == 2) AH_ENC(2);
    else if (dpb == 4) AH_ENC(4);
    else AH_ENC(0);
#undef AH_ENC
    return hipGetLastError();
}

}  // namespace ah
