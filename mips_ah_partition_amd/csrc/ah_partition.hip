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
// bf16 inputs would not hold the 1e-4 relative bound).  Workgroup tile
// 128 x 128, four waves of 64 x 64 (16 MFMA tiles, so each operand fragment
// read from LDS feeds four MFMAs of each of four tiles), K staged through LDS
// 16 at a time with rows padded to 20 floats (conflict-free 16-byte reads)
// and the next stage loaded from memory into registers while the current one
// computes.  A lane feeds k = 4*(lane/16) + j to the j-th MFMA of a group, so
// one ds_read_b128 serves four MFMAs; A and B use the same k permutation,
// which leaves the contraction unchanged.  Scores go to the workspace; a
// second kernel selects each query's best nl with the exact workgroup top-K
// selection over the query's scores staged in LDS.
#include "ah_device.hpp"
#include "ah_kernels.hpp"

namespace ah {

constexpr int kGemmThreads = 256;
constexpr int kGT = 128;      // tile rows / cols
constexpr int kGK = 16;       // K per LDS stage
constexpr int kGS = kGK + 4;  // padded row stride (floats)

// Four consecutive k of row r of a [rows x d] matrix, zero outside it.  kVec:
// d % 4 == 0 and a 16-byte aligned base, so one float4 load.
template <bool kVec>
__device__ __forceinline__ float4 fetch4(const float* __restrict__ m, int64_t rows, int32_t d, int64_t r, int k) {
    if (kVec) {
        if (r < rows && k < d) return *reinterpret_cast<const float4*>(m + r * d + k);
        return make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (r < rows && k + e < d) ? m[r * d + k + e] : 0.f;
    return make_float4(t[0], t[1], t[2], t[3]);
}

// kVec: d % 4 == 0 and 16-byte aligned rows, so stages load as float4
template <bool kVec>
__global__ __launch_bounds__(kGemmThreads) void centroid_scores_kernel(
    const float* __restrict__ q, int64_t nq, int32_t d, const float* __restrict__ cent, int32_t L,
    float* __restrict__ S, int32_t kchunk) {
    __shared__ __align__(16) float qa[kGT * kGS];
    __shared__ __align__(16) float cb[kGT * kGS];
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    const int64_t ntl = (L + kGT - 1) / kGT;  // leaf tiles; consecutive blocks share a query tile
    const int64_t tiles = ((nq + kGT - 1) / kGT) * ntl;
    const int64_t kz = (int64_t)blockIdx.x / tiles, t = (int64_t)blockIdx.x - kz * tiles;  // K split, tile
    const int64_t q0 = (t / ntl) * kGT;
    const int64_t l0 = (t % ntl) * kGT;
    // this split's K range (kchunk is a multiple of kGK, so stages never cross it)
    const int kb0 = (int)kz * kchunk, kb1 = kb0 + kchunk < d ? kb0 + kchunk : d;
    S += kz * nq * (int64_t)L;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 64;  // wave's 64x64 sub-tile
    v4f acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    // staging: thread t holds rows t/4 and t/4 + 64 of each operand, k 4*(t%4)..+3
    const int sr = tid >> 2, sk = 4 * (tid & 3);
    float4 nq0, nq1, nc0, nc1;
#define AH_FETCH(K0)                                                                         \
    do {                                                                                      \
        nq0 = fetch4<kVec>(q, nq, d, q0 + sr, (K0) + sk);                                     \
        nq1 = fetch4<kVec>(q, nq, d, q0 + sr + 64, (K0) + sk);                                \
        nc0 = fetch4<kVec>(cent, L, d, l0 + sr, (K0) + sk);                                   \
        nc1 = fetch4<kVec>(cent, L, d, l0 + sr + 64, (K0) + sk);                              \
    } while (0)
    AH_FETCH(kb0);
    for (int k0 = kb0; k0 < kb1; k0 += kGK) {
        *reinterpret_cast<float4*>(&qa[sr * kGS + sk]) = nq0;
        *reinterpret_cast<float4*>(&qa[(sr + 64) * kGS + sk]) = nq1;
        *reinterpret_cast<float4*>(&cb[sr * kGS + sk]) = nc0;
        *reinterpret_cast<float4*>(&cb[(sr + 64) * kGS + sk]) = nc1;
        __syncthreads();
        if (k0 + kGK < kb1) AH_FETCH(k0 + kGK);  // in flight while this stage computes
        const int kk = 4 * (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < kGK; kb += 16) {
            float4 av[4], bv[4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
                av[a] = *reinterpret_cast<const float4*>(&qa[(wm + 16 * a + (lane & 15)) * kGS + kb + kk]);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                bv[b] = *reinterpret_cast<const float4*>(&cb[(wn + 16 * b + (lane & 15)) * kGS + kb + kk]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
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
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t qr = q0 + wm + 16 * a + 4 * (lane >> 4) + i;
                const int64_t lc = l0 + wn + 16 * b + (lane & 15);
                if (qr < nq && lc < L) S[qr * L + lc] = acc[a][b][i];
            }
}
#undef AH_FETCH

struct ScoreKeys {
    const float* s;
    __device__ uint64_t operator()(int64_t i) const { return float_key(s[i], (int32_t)i); }
};

constexpr int kSelThreads = 256;

constexpr int kLeafLds = 8192;  // scores staged in LDS as keys up to this many leaves

__global__ __launch_bounds__(kSelThreads) void leaf_select_kernel(const float* __restrict__ S, int32_t L,
                                                                  int32_t nl, int32_t* __restrict__ leaves,
                                                                  float* __restrict__ scores) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ SelectShared sh;
    uint64_t* sel = reinterpret_cast<uint64_t*>(smem);
    const int64_t qi = blockIdx.x;
    int m;
    if (L <= kLeafLds) {  // the query's L scores read once, as keys, into LDS
        const int Kp = next_pow2(nl);
        uint64_t* keys = sel + Kp;
        for (int i = threadIdx.x; i < L; i += kSelThreads) keys[i] = float_key(S[qi * L + i], i);
        __syncthreads();
        m = wg_select_topk<kSelThreads>(LdsKeys{keys}, L, nl, sh, sel);
    } else {
        m = wg_select_topk<kSelThreads>(ScoreKeys{S + qi * L}, L, nl, sh, sel);
    }
    for (int r = threadIdx.x; r < nl; r += kSelThreads) {
        leaves[qi * nl + r] = r < m ? key_id(sel[r]) : -1;
        if (scores) scores[qi * nl + r] = r < m ? key_float_score(sel[r]) : -__builtin_huge_valf();
    }
}

// One wave per query (four per workgroup, no workgroup barrier) for L <=
// kWaveLeaves and nl <= kLeafSort: the query's scores, as order-preserving
// uint32, sit in registers (kPer per lane, all loads in flight at once); a
// radix select narrows the candidates with 256 LDS buckets per pass: one pass
// of equal-width buckets over the query's score range, then passes over the
// chosen bucket's range of score orders, then, if one score value still holds
// too many, over the leaf ids (lower id first), until every key at or above
// the current bucket's lower edge fits in Pt = next_pow2(max(nl, 64)) keys;
// those are sorted in registers and the first nl taken.  At the last id digit
// the bucket is the nl-th key itself, so the candidates never exceed Pt.
// Scores are assumed finite (NaN has no place in the order).
constexpr int kWaveLeaves = 4096;
constexpr int kLeafSort = 512;
constexpr int kLeafQ = 4;

// one select pass: the bucket (of 256, highest first) holding the need-th
// largest counted candidate, and the count above it
struct SelDigit {
    int digit, before, cnt;
};
__device__ __forceinline__ SelDigit pick_digit(const uint32_t* hist, int need, int lane) {
    uint32_t c[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        sum += (int)c[j];
    }
    const int incl = wave_inclusive_sum(sum);
    const uint64_t mk = __ballot(incl >= need);
    const int l = __ffsll((unsigned long long)mk) - 1;
    SelDigit r{0, 0, 0};
    if (lane == l) {
        int cum = incl - sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (cum < need && cum + (int)c[j] >= need) r = SelDigit{255 - 4 * lane - j, cum, (int)c[j]};
            cum += (int)c[j];
        }
    }
    r.digit = __shfl(r.digit, l, kWave);
    r.before = __shfl(r.before, l, kWave);
    r.cnt = __shfl(r.cnt, l, kWave);
    return r;
}

// Sorts the 64*E keys of srt (descending) in registers, key k*64+lane held by
// the lane in v[k], and writes the first nl as leaf ids (and scores).  Strides
// below 64 swap across lanes, larger ones within a lane.
template <int E>
__device__ __forceinline__ void wave_sort_emit(const uint64_t* srt, int nl, int lane, int32_t* leaves, float* scores) {
    uint64_t v[E];
#pragma unroll
    for (int k = 0; k < E; ++k) v[k] = srt[k * kWave + lane];
#pragma unroll
    for (int size = 2; size <= E * kWave; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= kWave) {
                const int ks = stride / kWave;
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    if (k & ks) continue;
                    const bool desc = ((k * kWave) & size) == 0;
                    const uint64_t x = v[k], y = v[k | ks];
                    const bool sw = (x < y) == desc;
                    v[k] = sw ? y : x;
                    v[k | ks] = sw ? x : y;
                }
            } else {
                const bool lower = (lane & stride) == 0;
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const bool desc = ((k * kWave + lane) & size) == 0;
                    const uint32_t plo = (uint32_t)__shfl_xor((int)(uint32_t)v[k], stride, kWave);
                    const uint32_t phi = (uint32_t)__shfl_xor((int)(uint32_t)(v[k] >> 32), stride, kWave);
                    const uint64_t p = ((uint64_t)phi << 32) | plo;
                    const bool take_max = lower == desc;
                    v[k] = take_max ? (p > v[k] ? p : v[k]) : (p < v[k] ? p : v[k]);
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int r = k * kWave + lane;
        if (r < nl) {
            leaves[r] = key_id(v[k]);
            if (scores) scores[r] = key_float_score(v[k]);
        }
    }
}

// kMap: the row is a candidate list, its element j carrying the id idmap[row * L
// + j] (unique within the row) and only the first rowcnt[row] elements being
// real; a row with more than L of them is skipped (left to the caller).
template <int kPer, int kWv, bool kMap = false>
__global__ __launch_bounds__(kLeafQ * kWave, kMap ? 2 : (kPer <= 16 ? 5 : 3)) void leaf_select_wave_kernel(const float* __restrict__ S, int64_t nq,
                                                                          int32_t L, int32_t nl,
                                                                          int32_t* __restrict__ leaves,
                                                                          float* __restrict__ scores, int32_t nsplit,
                                                                          const float* __restrict__ bias,
                                                                          const int32_t* __restrict__ idmap = nullptr,
                                                                          const uint32_t* __restrict__ rowcnt = nullptr) {
    constexpr int kQs = kLeafQ / kWv;  // queries per workgroup
    static_assert(kWv == 1 || kQs == 1, "a query spread over waves fills its workgroup");
    __shared__ uint32_t hist_all[kQs][256];
    __shared__ uint64_t srt_all[kQs][kLeafSort];
    __shared__ uint32_t red_all[kQs][kWv][2];
    __shared__ int cnt_all[kQs];
    const int w = threadIdx.x / kWave, lane = lane_id();
    const int qs = w / kWv, wq = w % kWv;  // query slot, wave within the query
    const int64_t qi = (int64_t)blockIdx.x * kQs + qs;
    if (kWv == 1 && qi >= nq) return;  // a multi-wave query is never partial: kQs == 1 there
    uint32_t* hist = hist_all[qs];
    uint64_t* srt = srt_all[qs];
    uint32_t(*red)[2] = red_all[qs];
    const float* s = S + qi * L;
    int32_t Lr = L;  // real elements in the row
    if constexpr (kMap) {
        const uint32_t c = rowcnt[qi];
        if (c > (uint32_t)L) return;  // every wave of the query leaves (kQs == 1 when kWv > 1)
        Lr = (int32_t)c;
    }
    // element i = (j * kWv + wq) * 64 + lane
    const int first = wq * kWave + lane;
    const int nv = first < Lr ? (Lr - first + kWv * kWave - 1) / (kWv * kWave) : 0;  // o[0 .. nv) are real
    // the score is the sum of the K splits' partial planes, in split order
    float sv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) sv[j] = j < nv ? s[j * kWv * kWave + first] : 0.f;
    for (int z = 1; z < nsplit; ++z) {
        const float* sz = s + z * nq * (int64_t)L;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j < nv) sv[j] += sz[j * kWv * kWave + first];
    }
    if (bias) {  // per-leaf additive term (nearest-centroid assignment)
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j < nv) sv[j] += bias[j * kWv * kWave + first];
    }
    uint32_t o[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) o[j] = j < nv ? float_order(sv[j]) : 0u;
    uint32_t idv[kMap ? kPer : 1];
    if constexpr (kMap) {
        const int32_t* im = idmap + qi * L;
#pragma unroll
        for (int j = 0; j < kPer; ++j) idv[j] = j < nv ? (uint32_t)im[j * kWv * kWave + first] : 0u;
    }
    auto sync = [] {
        if constexpr (kWv == 1) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        } else {
            __syncthreads();
        }
    };
    // min and max over the query's keys (all its waves)
    auto range_of = [&](uint32_t mn, uint32_t mx, uint32_t& rmin, uint32_t& rmax) {
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            const uint32_t x = __shfl_xor(mn, off, kWave), y = __shfl_xor(mx, off, kWave);
            mn = x < mn ? x : mn;
            mx = y > mx ? y : mx;
        }
        if constexpr (kWv > 1) {
            if (lane == 0) {
                red[wq][0] = mn;
                red[wq][1] = mx;
            }
            __syncthreads();
#pragma unroll
            for (int v = 0; v < kWv; ++v) {
                mn = red[v][0] < mn ? red[v][0] : mn;
                mx = red[v][1] > mx ? red[v][1] : mx;
            }
            __syncthreads();
        }
        rmin = mn;
        rmax = mx;
    };
    auto clear_hist = [&] {
#pragma unroll
        for (int j = wq * kWave + lane; j < 256; j += kWv * kWave) hist[j] = 0;
        sync();
    };
    uint32_t omin, omax;
    {
        uint32_t mn = 0xFFFFFFFFu, mx = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j < nv) {
                mn = o[j] < mn ? o[j] : mn;
                mx = o[j] > mx ? o[j] : mx;
            }
        }
        range_of(mn, mx, omin, omax);
    }
    auto key = [&](int j) -> uint64_t {
        uint32_t id;
        if constexpr (kMap) id = idv[j];
        else id = (uint32_t)(j * kWv * kWave + first);
        return ((uint64_t)o[j] << 32) | (uint64_t)(0xFFFFFFFFu - id);
    };
    int need = nl;   // still to pick at or below the current bucket
    int above = 0;   // keys known to be selected (above the bucket)
    int inb = Lr;    // keys in the current bucket
    const int Pt = next_pow2(nl > kWave ? nl : kWave);  // candidates to reach: one sort of Pt keys
    // First pass, on the score values: 256 equal-width buckets over [fmin, fmax]
    // (the bucket is non-decreasing in the score, so a bucket's members are
    // exactly the scores between its smallest and largest order).  The order
    // space is far from linear in the score, so this pass splits a typical
    // score distribution much better than the first order digit would.
    {
        const float fmin = order_float(omin), range = order_float(omax) - fmin;
        if (above + inb > Pt && range > 0.f && range < __builtin_huge_valf()) {
            const float scale = 256.f / range;
            auto lbin = [&](int j) -> int {
                const int b = (int)((order_float(o[j]) - fmin) * scale);
                return b < 255 ? b : 255;
            };
            clear_hist();
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if (j < nv) atomicAdd(&hist[lbin(j)], 1u);
            sync();
            const SelDigit r = pick_digit(hist, need, lane);  // every wave of the query, same result
            sync();
            need -= r.before;
            above += r.before;
            inb = r.cnt;
            uint32_t mn = 0xFFFFFFFFu, mx = 0;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                if (j < nv && lbin(j) == r.digit) {
                    mn = o[j] < mn ? o[j] : mn;
                    mx = o[j] > mx ? o[j] : mx;
                }
            }
            range_of(mn, mx, omin, omax);
        }
    }
    // score-order passes: 256 buckets of width 2^sh over [lo, hi)
    uint32_t lo = omin;
    uint64_t hi = (uint64_t)omax + 1;  // exclusive
    int sh = 0;
    while (sh < 24 && ((omax - omin) >> sh) > 255u) ++sh;
    uint64_t edge = (uint64_t)lo << 32;  // the current bucket's lower edge as a key
    bool tied = false;
    while (above + inb > Pt) {
        if (sh < 0) {  // one score value holds too many: resolve by id below
            tied = true;
            break;
        }
        clear_hist();
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j < nv && o[j] >= lo && (uint64_t)o[j] < hi) atomicAdd(&hist[(o[j] - lo) >> sh], 1u);
        sync();
        const SelDigit r = pick_digit(hist, need, lane);
        sync();
        need -= r.before;
        above += r.before;
        inb = r.cnt;
        lo += (uint32_t)r.digit << sh;
        hi = hi < (uint64_t)lo + (1ull << sh) ? hi : (uint64_t)lo + (1ull << sh);
        edge = (uint64_t)lo << 32;
        sh = sh >= 8 ? sh - 8 : (sh > 0 ? 0 : -1);
    }
    if (tied) {
        // every key left in the bucket has score order lo: 8-bit passes over ~id
        uint64_t prefix = (uint64_t)lo << 32, mask = 0xFFFFFFFF00000000ull;
        for (int shift = 24; shift >= 0 && above + inb > Pt; shift -= 8) {
            clear_hist();
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const uint64_t k = key(j);
                if (j < nv && (k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
            }
            sync();
            const SelDigit r = pick_digit(hist, need, lane);
            sync();
            need -= r.before;
            above += r.before;
            inb = r.cnt;
            prefix |= (uint64_t)r.digit << shift;
            mask |= (uint64_t)0xFF << shift;
        }
        edge = prefix;
    }
    // collect the keys at or above the bucket's lower edge, sort, take nl
    if constexpr (kWv > 1) {
        if (threadIdx.x == 0) cnt_all[qs] = 0;
        __syncthreads();
    }
    int n = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const uint64_t k = key(j);
        const bool keep = j < nv && k >= edge;
        const uint64_t mk = __ballot(keep);
        if (mk == 0) continue;
        int base = n;
        if constexpr (kWv > 1) {
            if (lane == 0) base = atomicAdd(&cnt_all[qs], __popcll(mk));
            base = __shfl(base, 0, kWave);
        }
        const int pos = base + __popcll(mk & lanemask_lt());
        if (keep && pos < Pt) srt[pos] = k;  // never more than Pt for finite scores
        n += __popcll(mk);
    }
    sync();
    if (wq != 0) return;
    if constexpr (kWv > 1) n = cnt_all[qs];
    for (int j = n + lane; j < Pt; j += kWave) srt[j] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int32_t* lq = leaves + qi * nl;
    float* sq = scores ? scores + qi * nl : nullptr;
    if (Pt == kWave) wave_sort_emit<1>(srt, nl, lane, lq, sq);
    else if (Pt == 2 * kWave) wave_sort_emit<2>(srt, nl, lane, lq, sq);
    else if (Pt == 4 * kWave) wave_sort_emit<4>(srt, nl, lane, lq, sq);
    else wave_sort_emit<8>(srt, nl, lane, lq, sq);
}

template <int kPer, int kWv>
static void launch_leaf_wave(const float* S, int64_t nq, int32_t L, int32_t nl, int32_t* leaves, float* scores,
                             int32_t nsplit, hipStream_t stream, const float* bias = nullptr) {
    constexpr int kQs = kLeafQ / kWv;
    hipLaunchKernelGGL((leaf_select_wave_kernel<kPer, kWv>), dim3((unsigned)((nq + kQs - 1) / kQs)),
                       dim3(kLeafQ * kWave), 0, stream, S, nq, L, nl, leaves, scores, nsplit, bias, nullptr,
                       nullptr);
}

// K splits of the contraction: when the tile grid has fewer than 256 tiles (one
// per CU) and the one-wave selection (which adds the partial planes) applies,
// up to four splits bring it to about 512 workgroups.
static int max_splits(int64_t nq, int32_t L) {
    const int64_t tiles = ((nq + kGT - 1) / kGT) * ((L + kGT - 1) / kGT);
    if (L > kWaveLeaves || tiles >= 256 || tiles == 0) return 1;  // tiles == 0: no queries or no leaves
    const int64_t want = (512 + tiles - 1) / tiles;
    return (int)(want < 4 ? want : 4);
}

size_t partition_workspace_bytes(int64_t nq, int32_t L) {
    return (size_t)max_splits(nq, L) * (size_t)nq * (size_t)L * 4 + 256;
}

hipError_t launch_partition(const float* q, int64_t nq, int32_t d, const float* cent, int32_t L,
                            int32_t nl, int32_t* leaves, float* scores, void* ws, hipStream_t stream) {
    if (nq == 0) return hipSuccess;
    float* S = reinterpret_cast<float*>(ws);
    const bool wave_sel = L <= kWaveLeaves && nl <= kLeafSort;
    const int nstage = (d + kGK - 1) / kGK;
    int nsplit = wave_sel ? max_splits(nq, L) : 1;
    nsplit = nsplit < nstage ? nsplit : nstage;
    const int kchunk = ((nstage + nsplit - 1) / nsplit) * kGK;
    nsplit = (d + kchunk - 1) / kchunk;  // no empty split
    const int64_t tiles = ((L + kGT - 1) / kGT) * ((nq + kGT - 1) / kGT);
    dim3 grid((unsigned)(tiles * nsplit));
    const bool vec = (d % 4) == 0 && (reinterpret_cast<uintptr_t>(q) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(cent) & 15) == 0;
    if (vec) hipLaunchKernelGGL(centroid_scores_kernel<true>, grid, dim3(kGemmThreads), 0, stream, q, nq, d, cent, L, S, kchunk);
    else hipLaunchKernelGGL(centroid_scores_kernel<false>, grid, dim3(kGemmThreads), 0, stream, q, nq, d, cent, L, S, kchunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (wave_sel) {
        if (L <= 4 * kWave) launch_leaf_wave<4, 1>(S, nq, L, nl, leaves, scores, nsplit, stream);
        else if (L <= 8 * kWave) launch_leaf_wave<8, 1>(S, nq, L, nl, leaves, scores, nsplit, stream);
        else if (L <= 16 * kWave) launch_leaf_wave<16, 1>(S, nq, L, nl, leaves, scores, nsplit, stream);
        else if (L <= 32 * kWave) launch_leaf_wave<32, 1>(S, nq, L, nl, leaves, scores, nsplit, stream);
        else launch_leaf_wave<16, 4>(S, nq, L, nl, leaves, scores, nsplit, stream);
        return hipGetLastError();
    }
    int Kp = 1;
    while (Kp < nl) Kp <<= 1;
    const size_t lds = (size_t)Kp * 8 + (L <= kLeafLds ? (size_t)L * 8 : 0);
    if (lds > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(leaf_select_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(leaf_select_kernel, dim3((unsigned)nq), dim3(kSelThreads), lds, stream,
                       S, L, nl, leaves, scores);
    return hipGetLastError();
}

// ------------------------------------------------------------------ nearest-centroid assignment
// The k-means assignment step of the partitioning (the ScaNN page's
// "Three stages of a search": rows are grouped under the centroid they are
// closest to): argmin_l |x - c_l|^2 = argmax_l (x . c_l - |c_l|^2 / 2), lowest
// leaf id on ties.  The same fp32 MFMA contraction as the centroid scoring, in
// row chunks whose score block fits the workspace, then the one-wave selection
// of the single best leaf with -|c_l|^2 / 2 added to every score.
__global__ void half_norm_kernel(const float* __restrict__ cent, int32_t L, int32_t d, float* __restrict__ bias) {
    const int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (l >= L) return;
    float s = 0.f;
    for (int t = 0; t < d; ++t) s = __fmaf_rn(cent[l * d + t], cent[l * d + t], s);
    bias[l] = -0.5f * s;
}

constexpr int64_t kAssignChunk = 65536;  // rows per contraction and selection

static int64_t assign_chunk(int64_t n) { return n < kAssignChunk ? (n > 0 ? n : 1) : kAssignChunk; }

size_t assign_workspace_bytes(int64_t n, int32_t L) {
    return (((size_t)L * 4 + 255) & ~(size_t)255) + (size_t)assign_chunk(n) * (size_t)L * 4 + 256;
}

hipError_t launch_assign(const float* x, int64_t n, int32_t d, const float* cent, int32_t L, int32_t* leaves,
                         float* scores, void* ws, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    float* bias = reinterpret_cast<float*>(ws);
    float* S = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (((size_t)L * 4 + 255) & ~(size_t)255));
    hipLaunchKernelGGL(half_norm_kernel, dim3((unsigned)((L + 255) / 256)), dim3(256), 0, stream, cent, L, d, bias);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t chunk = assign_chunk(n);
    for (int64_t r0 = 0; r0 < n; r0 += chunk) {
        const int64_t m = n - r0 < chunk ? n - r0 : chunk;
        const float* q = x + r0 * d;
        const int64_t tiles = ((L + kGT - 1) / kGT) * ((m + kGT - 1) / kGT);
        const int kchunk = ((d + kGK - 1) / kGK) * kGK;
        const bool vec = (d % 4) == 0 && (reinterpret_cast<uintptr_t>(q) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(cent) & 15) == 0;
        if (vec) hipLaunchKernelGGL(centroid_scores_kernel<true>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream, q, m, d, cent, L, S, kchunk);
        else hipLaunchKernelGGL(centroid_scores_kernel<false>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream, q, m, d, cent, L, S, kchunk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        int32_t* lo = leaves + r0;
        float* so = scores ? scores + r0 : nullptr;
        if (L <= 4 * kWave) launch_leaf_wave<4, 1>(S, m, L, 1, lo, so, 1, stream, bias);
        else if (L <= 8 * kWave) launch_leaf_wave<8, 1>(S, m, L, 1, lo, so, 1, stream, bias);
        else if (L <= 16 * kWave) launch_leaf_wave<16, 1>(S, m, L, 1, lo, so, 1, stream, bias);
        else if (L <= 32 * kWave) launch_leaf_wave<32, 1>(S, m, L, 1, lo, so, 1, stream, bias);
        else launch_leaf_wave<16, 4>(S, m, L, 1, lo, so, 1, stream, bias);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------------------ k-means update
// The update step of the partitioning's k-means: each leaf's centroid becomes
// the mean of its rows (float64 sums, float32 result); a leaf with no rows
// keeps its centroid.  Sums by float64 atomic adds (a wave per row, one lane
// per dimension), so their order is not fixed: results agree with a row-order
// sum to float64 rounding, i.e. to within one float32 unit.
__global__ void kmeans_zero_kernel(double* __restrict__ sum, int64_t count, uint32_t* __restrict__ cnt, int32_t L) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
        sum[i] = 0.0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < L; i += (int64_t)gridDim.x * blockDim.x)
        cnt[i] = 0;
}

__global__ __launch_bounds__(256) void kmeans_accumulate_kernel(const float* __restrict__ x, int64_t n, int32_t d,
                                                                const int32_t* __restrict__ leaf, int32_t L,
                                                                double* __restrict__ sum, uint32_t* __restrict__ cnt) {
    const int lane = lane_id();
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t i = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; i < n; i += waves) {
        const int32_t l = leaf[i];
        if (l < 0 || l >= L) continue;  // rows without a valid leaf are left out
        if (lane == 0) atomicAdd(&cnt[l], 1u);
        const float* xr = x + i * d;
        double* sr = sum + (int64_t)l * d;
        for (int t = lane; t < d; t += kWave) unsafeAtomicAdd(&sr[t], (double)xr[t]);
    }
}

__global__ void kmeans_finish_kernel(const double* __restrict__ sum, const uint32_t* __restrict__ cnt, int32_t L,
                                     int32_t d, float* __restrict__ cent, int32_t* __restrict__ counts) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)L * d) return;
    const int32_t l = (int32_t)(e / d);
    const uint32_t c = cnt[l];
    if (counts && e % d == 0) counts[l] = (int32_t)c;
    if (c > 0) cent[e] = (float)(sum[e] / (double)c);
}

size_t kmeans_workspace_bytes(int32_t L, int32_t d) {
    return (((size_t)L * d * 8 + 255) & ~(size_t)255) + (size_t)L * 4;
}

hipError_t launch_kmeans_update(const float* x, int64_t n, int32_t d, const int32_t* leaf, int32_t L, float* cent,
                                int32_t* counts, void* ws, hipStream_t stream) {
    double* sum = reinterpret_cast<double*>(ws);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + (((size_t)L * d * 8 + 255) & ~(size_t)255));
    const int64_t cells = (int64_t)L * d;
    hipLaunchKernelGGL(kmeans_zero_kernel, dim3((unsigned)((cells + 255) / 256 < 4096 ? (cells + 255) / 256 : 4096)),
                       dim3(256), 0, stream, sum, cells, cnt, L);
    if (n > 0) {
        const int64_t blocks = (n + 3) / 4;
        hipLaunchKernelGGL(kmeans_accumulate_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0,
                           stream, x, n, d, leaf, L, sum, cnt);
    }
    hipLaunchKernelGGL(kmeans_finish_kernel, dim3((unsigned)((cells + 255) / 256)), dim3(256), 0, stream, sum, cnt, L, d,
                       cent, counts);
    return hipGetLastError();
}

// ------------------------------------------------------------------ residual leaf terms
// The residual (leaf-relative) variant scores a row as q.c_leaf + q.residual; the
// int8 table approximates q.residual as bias + step * sum, so, in table units,
// the leaf contributes q.c_leaf / step, taken relative to the query's first
// leaf (a per-query constant does not change the ranking) and rounded half to
// even.  One thread per (query, probed leaf); all float32, as defined.
__global__ void residual_bias_kernel(const float* __restrict__ scores, const float* __restrict__ step, int64_t nq,
                                     int32_t nl, int32_t bound, int32_t* __restrict__ bias) {
#pragma clang fp contract(off)
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= nq * nl) return;
    const int64_t q = e / nl;
    const float st = step[q];
    int32_t v = 0;
    if (st > 0.f) {
        float r = rintf((scores[e] - scores[q * nl]) / st);
        r = fminf(fmaxf(r, -(float)bound), (float)bound);
        v = (int32_t)r;
    }
    bias[e] = v;
}

hipError_t launch_residual_bias(const float* scores, const float* step, int64_t nq, int32_t nl, int32_t bound,
                                int32_t* bias, hipStream_t stream) {
    const int64_t total = nq * nl;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(residual_bias_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, scores, step,
                       nq, nl, bound, bias);
    return hipGetLastError();
}

// The best k columns of each row of a score block [rows][L] by (score desc,
// column asc): the one-wave selection for L <= kWaveLeaves and k <= kLeafSort,
// else the workgroup selection (launch_rows_topk); launch_list_topk does the
// same for candidate lists with their own ids and lengths.
hipError_t launch_list_topk(const float* S, const int32_t* idmap, const uint32_t* rowcnt, int64_t rows, int32_t cap,
                            int32_t k, int32_t* ids, float* scores, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (cap > kWaveLeaves || k > kLeafSort) return hipErrorInvalidValue;
#define AH_LIST(P, W)                                                                                          \
    hipLaunchKernelGGL((leaf_select_wave_kernel<P, W, true>), dim3((unsigned)((rows + kLeafQ / W - 1) / (kLeafQ / W))), \
                       dim3(kLeafQ * kWave), 0, stream, S, rows, cap, k, ids, scores, 1, nullptr, idmap, rowcnt)
    if (cap <= 4 * kWave) AH_LIST(4, 1);
    else if (cap <= 8 * kWave) AH_LIST(8, 1);
    else if (cap <= 16 * kWave) AH_LIST(16, 1);
    else if (cap <= 32 * kWave) AH_LIST(32, 1);
    else AH_LIST(16, 4);
#undef AH_LIST
    return hipGetLastError();
}

hipError_t launch_rows_topk(const float* S, int64_t rows, int32_t L, int32_t k, int32_t* ids, float* scores,
                            hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (L <= kWaveLeaves && k <= kLeafSort) {
        if (L <= 4 * kWave) launch_leaf_wave<4, 1>(S, rows, L, k, ids, scores, 1, stream);
        else if (L <= 8 * kWave) launch_leaf_wave<8, 1>(S, rows, L, k, ids, scores, 1, stream);
        else if (L <= 16 * kWave) launch_leaf_wave<16, 1>(S, rows, L, k, ids, scores, 1, stream);
        else if (L <= 32 * kWave) launch_leaf_wave<32, 1>(S, rows, L, k, ids, scores, 1, stream);
        else launch_leaf_wave<16, 4>(S, rows, L, k, ids, scores, 1, stream);
        return hipGetLastError();
    }
    int Kp = 1;
    while (Kp < k) Kp <<= 1;
    const size_t lds = (size_t)Kp * 8 + (L <= kLeafLds ? (size_t)L * 8 : 0);
    if (lds > 48 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(leaf_select_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(leaf_select_kernel, dim3((unsigned)rows), dim3(kSelThreads), lds, stream, S, L, k, ids, scores);
    return hipGetLastError();
}

}  // namespace ah
