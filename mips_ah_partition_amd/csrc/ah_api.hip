// C ABI of the AH search path (declared in include/ah.h): argument checks on the
// host, workspace sizing, and the kernel launches.  Nothing here allocates,
// synchronises or keeps state between calls.
#include "../../include/ah.h"
#include "../../include/ah_instrument.h"
#include "ah_kernels.hpp"

#include <mutex>

// Scan scratch of ah_scan_topk_noalloc: every GPU that runs the library holds
// one copy of this array for the life of the process.  In host code the name
// is only a stand-in; the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[AH_SCAN_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that
// device, with the device current).
int current_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return AH_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return AH_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AH_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return AH_OK;
}

inline bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? AH_OK : AH_ERR_HIP; }

}  // namespace

extern "C" {

const char* ah_status_string(int status) {
    switch (status) {
        case AH_OK: return "ok";
        case AH_ERR_NULL: return "a required pointer is NULL";
        case AH_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case AH_ERR_UNSUPPORTED: return "unsupported argument (dtype, alignment or a size above the library limits)";
        case AH_ERR_WORKSPACE: return "workspace missing or smaller than required";
        case AH_ERR_HIP: return "a HIP kernel launch failed";
        default: return "unknown status";
    }
}

int ah_version(void) { return 1; }

size_t ah_partition_workspace_bytes(int64_t nq, int32_t L) {
    if (nq < 0 || L < 0) return 0;
    return ah::partition_workspace_bytes(nq, L);
}

int ah_partition_score(const float* q, int64_t nq, int32_t d, const float* centroids, int32_t L,
                       int32_t nl, int32_t* leaves_out, float* leaf_scores_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (nq < 0 || d < 1 || L < 1 || nl < 1 || nl > L) return AH_ERR_SHAPE;
    if (d > AH_MAX_DIM || nl > AH_MAX_R) return AH_ERR_UNSUPPORTED;
    if (nq == 0) return AH_OK;
    if (!q || !centroids || !leaves_out || !workspace) return AH_ERR_NULL;
    if (workspace_bytes < ah::partition_workspace_bytes(nq, L)) return AH_ERR_WORKSPACE;
    return hip_status(ah::launch_partition(q, nq, d, centroids, L, nl, leaves_out, leaf_scores_out,
                                           workspace, static_cast<hipStream_t>(stream)));
}

int ah_build_lut(const float* q, int64_t nq, int32_t d, const float* codebooks, int32_t B,
                 int32_t dpb, float* lut_f32_out, int8_t* lut_i8_out, float* scale_out,
                 float* bias_out, void* stream) {
    if (nq < 0 || B < 1 || dpb < 1 || (int64_t)B * dpb != d) return AH_ERR_SHAPE;
    if (B > AH_MAX_BLOCKS || dpb > AH_MAX_DPB || B > AH_LUT_MAX_BLOCKS) return AH_ERR_UNSUPPORTED;
    if (nq == 0) return AH_OK;
    if (!q || !codebooks || !lut_i8_out || !scale_out || !bias_out) return AH_ERR_NULL;
    return hip_status(ah::launch_build_lut(q, nq, d, codebooks, B, dpb, lut_f32_out, lut_i8_out,
                                           scale_out, bias_out, static_cast<hipStream_t>(stream)));
}

size_t ah_scan_workspace_bytes(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R) {
    if (nq < 0 || n < 0 || B < 1 || R < 1) return 0;
    return ah::scan_workspace_bytes(nq, B, n, L, nl, R);
}

// The argument checks of ah_scan_topk that come before the workspace (AH_OK
// also when nq == 0, which needs no workspace).
static int scan_check(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes, int32_t code_stride,
                      int64_t n, const int64_t* leaf_offsets, int32_t L, const int32_t* leaves, int32_t nl,
                      const int32_t* leaf_bias, int32_t bias_bound, int32_t R, const int32_t* cand_ids_out,
                      const int32_t* cand_scores_out) {
    const bool tiled = code_stride == AH_CODES_TILED;
    if (nq < 0 || n < 0 || B < 1 || R < 1 || (!tiled && code_stride < (B + 1) / 2)) return AH_ERR_SHAPE;
    if (leaves && (L < 1 || nl < 1 || nl > L || !leaf_offsets)) return AH_ERR_SHAPE;
    if (leaf_bias && (!leaves || bias_bound < 0)) return AH_ERR_SHAPE;
    if (B > AH_MAX_BLOCKS || R > AH_MAX_R || n >= ((int64_t)1 << 31)) return AH_ERR_UNSUPPORTED;
    if (leaf_bias && bias_bound > AH_MAX_LEAF_BIAS) return AH_ERR_UNSUPPORTED;
    if (nq == 0) return AH_OK;
    if (!lut_i8 || !cand_ids_out || !cand_scores_out || (n > 0 && !codes)) return AH_ERR_NULL;
    if (!a16(lut_i8) || (tiled && !a16(codes))) return AH_ERR_UNSUPPORTED;
    return AH_OK;
}

static int scan_impl(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes, int32_t code_stride,
                     int64_t n, const int32_t* ids, const int64_t* leaf_offsets, int32_t L, const int32_t* leaves,
                     int32_t nl, const int32_t* leaf_bias, int32_t bias_bound, int32_t R, int32_t* cand_ids_out,
                     int32_t* cand_scores_out, void* workspace, size_t workspace_bytes, void* stream,
                     void* main_start_event, void* main_stop_event) {
    const int chk = scan_check(lut_i8, nq, B, codes, code_stride, n, leaf_offsets, L, leaves, nl, leaf_bias,
                               bias_bound, R, cand_ids_out, cand_scores_out);
    if (chk != AH_OK || nq == 0) return chk;
    const bool tiled = code_stride == AH_CODES_TILED;
    const int32_t Lw = leaves ? L : 0, nlw = leaves ? nl : 0;
    if (!workspace || workspace_bytes < ah::scan_workspace_bytes(nq, B, n, Lw, nlw, R)) return AH_ERR_WORKSPACE;
    const int32_t seg16 = ((B + 1) / 2 + 15) / 16;  // 16-byte segments per row
    ah::ScanProblem sp{lut_i8, nq, B, codes, tiled ? 16 * seg16 : code_stride, n, ids,
                       leaves ? leaf_offsets : nullptr, Lw, leaves, nlw, R, cand_ids_out, cand_scores_out,
                       tiled ? (int64_t)1024 * seg16 : 0, leaf_bias, leaf_bias ? bias_bound : 0};
    return hip_status(ah::launch_scan(sp, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                                      static_cast<hipEvent_t>(main_start_event),
                                      static_cast<hipEvent_t>(main_stop_event)));
}

int ah_scan_topk_timed(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes,
                       int32_t code_stride, int64_t n, const int32_t* ids, const int64_t* leaf_offsets,
                       int32_t L, const int32_t* leaves, int32_t nl, int32_t R, int32_t* cand_ids_out,
                       int32_t* cand_scores_out, void* workspace, size_t workspace_bytes, void* stream,
                       void* main_start_event, void* main_stop_event) {
    return scan_impl(lut_i8, nq, B, codes, code_stride, n, ids, leaf_offsets, L, leaves, nl, nullptr, 0, R,
                     cand_ids_out, cand_scores_out, workspace, workspace_bytes, stream, main_start_event,
                     main_stop_event);
}

int ah_scan_topk_noalloc(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes,
                         int32_t code_stride, int64_t n, const int32_t* ids, const int64_t* leaf_offsets,
                         int32_t L, const int32_t* leaves, int32_t nl, int32_t R, int32_t* cand_ids_out,
                         int32_t* cand_scores_out, void* stream) {
    // the checks of ah_scan_topk, then the scratch it needs against the array
    const int chk = scan_check(lut_i8, nq, B, codes, code_stride, n, leaf_offsets, L, leaves, nl, nullptr, 0, R,
                               cand_ids_out, cand_scores_out);
    if (chk != AH_OK || nq == 0) return chk;
    const int32_t Lw = leaves ? L : 0, nlw = leaves ? nl : 0;
    if (ah::scan_workspace_bytes(nq, B, n, Lw, nlw, R) > (size_t)AH_SCAN_SCRATCH_BYTES) return AH_ERR_UNSUPPORTED;
    void* ws = nullptr;
    const int st = current_scratch(&ws);
    if (st != AH_OK) return st;
    return scan_impl(lut_i8, nq, B, codes, code_stride, n, ids, leaf_offsets, L, leaves, nl, nullptr, 0, R,
                     cand_ids_out, cand_scores_out, ws, (size_t)AH_SCAN_SCRATCH_BYTES, stream, nullptr, nullptr);
}

int ah_scan_workspace_counters(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R,
                               size_t* appended_offset, size_t* control_offset) {
    if (!appended_offset || !control_offset) return AH_ERR_NULL;
    if (nq < 0 || n < 0 || B < 1 || R < 1) return AH_ERR_SHAPE;
    ah::scan_counter_offsets(nq, B, n, L, nl, R, appended_offset, control_offset);
    return AH_OK;
}

int ah_hbm_read_probe(const void* data, size_t bytes, int32_t blocks_per_cu, uint32_t* sink, void* stream) {
    if ((bytes & 15) != 0 || blocks_per_cu < 1 || blocks_per_cu > 64) return AH_ERR_SHAPE;
    if (bytes == 0) return AH_OK;
    if (!data || !sink) return AH_ERR_NULL;
    if (!a16(data)) return AH_ERR_UNSUPPORTED;
    return hip_status(ah::launch_read_probe(data, (int64_t)(bytes / 16), blocks_per_cu, sink,
                                            static_cast<hipStream_t>(stream)));
}

int ah_scan_topk(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes,
                 int32_t code_stride, int64_t n, const int32_t* ids, const int64_t* leaf_offsets,
                 int32_t L, const int32_t* leaves, int32_t nl, int32_t R, int32_t* cand_ids_out,
                 int32_t* cand_scores_out, void* workspace, size_t workspace_bytes, void* stream) {
    return scan_impl(lut_i8, nq, B, codes, code_stride, n, ids, leaf_offsets, L, leaves, nl, nullptr, 0, R,
                     cand_ids_out, cand_scores_out, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int ah_scan_topk_residual(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes, int32_t code_stride,
                          int64_t n, const int32_t* ids, const int64_t* leaf_offsets, int32_t L,
                          const int32_t* leaves, int32_t nl, const int32_t* leaf_bias, int32_t bias_bound, int32_t R,
                          int32_t* cand_ids_out, int32_t* cand_scores_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (!leaves || !leaf_bias) {
        if (nq < 0) return AH_ERR_SHAPE;
        if (nq == 0) return AH_OK;
        return !leaves ? AH_ERR_SHAPE : AH_ERR_NULL;
    }
    return scan_impl(lut_i8, nq, B, codes, code_stride, n, ids, leaf_offsets, L, leaves, nl, leaf_bias, bias_bound,
                     R, cand_ids_out, cand_scores_out, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int ah_residual_leaf_bias(const float* leaf_scores, const float* step, int64_t nq, int32_t nl, int32_t bias_bound,
                          int32_t* bias_out, void* stream) {
    if (nq < 0 || nl < 1 || bias_bound < 0) return AH_ERR_SHAPE;
    if (bias_bound > AH_MAX_LEAF_BIAS) return AH_ERR_UNSUPPORTED;
    if (nq == 0) return AH_OK;
    if (!leaf_scores || !step || !bias_out) return AH_ERR_NULL;
    return hip_status(ah::launch_residual_bias(leaf_scores, step, nq, nl, bias_bound, bias_out,
                                               static_cast<hipStream_t>(stream)));
}

int ah_sq8_quantize(const float* x, int64_t n, int32_t d, double pct, int8_t* codes_out, float* scale_out,
                    void* stream) {
    if (n < 0 || d < 1 || !(pct >= 0.0 && pct <= 100.0)) return AH_ERR_SHAPE;
    if (d > AH_MAX_DIM) return AH_ERR_UNSUPPORTED;
    if (n == 0) return AH_OK;
    if (!x || !codes_out || !scale_out) return AH_ERR_NULL;
    return hip_status(ah::launch_sq8_quantize(x, n, d, pct, codes_out, scale_out, static_cast<hipStream_t>(stream)));
}

size_t ah_sq8_workspace_bytes(int64_t nq, int64_t n, int32_t d, int32_t R) {
    if (nq < 0 || n < 1 || d < 1 || R < 1) return 0;
    return ah::sq8_workspace_bytes(nq, n, d, R);
}

int ah_sq8_scan_topk(const int8_t* q8, const float* q_scale, int64_t nq, const int8_t* d8, const float* d_scale,
                     int64_t n, int32_t d, int32_t R, int32_t* ids_out, float* scores_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (nq < 0 || n < 1 || d < 1 || R < 1 || R > n) return AH_ERR_SHAPE;
    if (d % 16 != 0 || d > AH_MAX_DIM || R > AH_MAX_R || n >= ((int64_t)1 << 31)) return AH_ERR_UNSUPPORTED;
    if (nq == 0) return AH_OK;
    if (!q8 || !q_scale || !d8 || !d_scale || !ids_out) return AH_ERR_NULL;
    if (!a16(q8) || !a16(d8)) return AH_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < ah::sq8_workspace_bytes(nq, n, d, R)) return AH_ERR_WORKSPACE;
    return hip_status(ah::launch_sq8_topk(q8, q_scale, nq, d8, d_scale, n, d, R, ids_out, scores_out, workspace,
                                          static_cast<hipStream_t>(stream)));
}

int ah_rslm_rotate(const float* x, int64_t n, int32_t d, const float* signs, const int32_t* perm, float* y_out,
                   void* stream) {
    if (n < 0 || d < 1) return AH_ERR_SHAPE;
    if (d > AH_MAX_DIM) return AH_ERR_UNSUPPORTED;
    if (n == 0) return AH_OK;
    if (!x || !signs || !perm || !y_out) return AH_ERR_NULL;
    return hip_status(ah::launch_rslm_rotate(x, n, d, signs, perm, y_out, static_cast<hipStream_t>(stream)));
}

int ah_rslm_encode(const float* y, int64_t n, int32_t d, const float* levels, uint8_t* codes_out, float* step_out,
                   void* stream) {
    if (n < 0 || d < 1) return AH_ERR_SHAPE;
    if (d > AH_MAX_DIM) return AH_ERR_UNSUPPORTED;
    if (!levels) return AH_ERR_NULL;
    for (int c = 0; c < 15; ++c)
        if (!(levels[c] < levels[c + 1])) return AH_ERR_SHAPE;
    if (!(levels[15] > 0.0f)) return AH_ERR_SHAPE;
    if (n == 0) return AH_OK;
    if (!y || !codes_out || !step_out) return AH_ERR_NULL;
    float mids[15];
    for (int c = 0; c < 15; ++c) mids[c] = (float)(((double)levels[c] + (double)levels[c + 1]) / 2.0);
    const double lam = 127.0 / (double)levels[15];
    return hip_status(ah::launch_rslm_encode(y, n, d, levels, mids, lam, codes_out, step_out,
                                             static_cast<hipStream_t>(stream)));
}

int ah_rslm_scan_topk(const int8_t* q8, const float* q_scale, int64_t nq, const uint8_t* codes, const float* step,
                      int64_t n, int32_t d, const int8_t* levels_i8, int32_t R, int32_t* ids_out, float* scores_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (nq < 0 || n < 1 || d < 1 || R < 1 || R > n) return AH_ERR_SHAPE;
    if (d % 16 != 0 || d > AH_MAX_DIM || R > AH_MAX_R || n >= ((int64_t)1 << 31)) return AH_ERR_UNSUPPORTED;
    if (nq == 0) return AH_OK;
    if (!q8 || !q_scale || !codes || !step || !levels_i8 || !ids_out) return AH_ERR_NULL;
    if (!a16(q8) || (reinterpret_cast<uintptr_t>(codes) & 7)) return AH_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < ah::sq8_workspace_bytes(nq, n, d, R)) return AH_ERR_WORKSPACE;
    return hip_status(ah::launch_sq8_topk(q8, q_scale, nq, nullptr, step, n, d, R, ids_out, scores_out, workspace,
                                          static_cast<hipStream_t>(stream), codes, levels_i8));
}

size_t ah_kmeans_workspace_bytes(int32_t L, int32_t d) {
    if (L < 1 || d < 1) return 0;
    return ah::kmeans_workspace_bytes(L, d);
}

int ah_kmeans_update(const float* x, int64_t n, int32_t d, const int32_t* leaf_of_row, int32_t L, float* centroids,
                     int32_t* counts_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 0 || d < 1 || L < 1) return AH_ERR_SHAPE;
    if (d > AH_MAX_DIM || n >= ((int64_t)1 << 32)) return AH_ERR_UNSUPPORTED;
    if (!centroids || (n > 0 && (!x || !leaf_of_row))) return AH_ERR_NULL;
    if (!workspace || workspace_bytes < ah::kmeans_workspace_bytes(L, d)) return AH_ERR_WORKSPACE;
    return hip_status(ah::launch_kmeans_update(x, n, d, leaf_of_row, L, centroids, counts_out, workspace,
                                               static_cast<hipStream_t>(stream)));
}

size_t ah_assign_workspace_bytes(int64_t n, int32_t L) {
    if (n < 0 || L < 1) return 0;
    return ah::assign_workspace_bytes(n, L);
}

int ah_assign_leaves(const float* x, int64_t n, int32_t d, const float* centroids, int32_t L, int32_t* leaf_out,
                     float* score_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 0 || d < 1 || L < 1) return AH_ERR_SHAPE;
    if (L > AH_MAX_ASSIGN_LEAVES || d > AH_MAX_DIM) return AH_ERR_UNSUPPORTED;
    if (n == 0) return AH_OK;
    if (!x || !centroids || !leaf_out) return AH_ERR_NULL;
    if (!workspace || workspace_bytes < ah::assign_workspace_bytes(n, L)) return AH_ERR_WORKSPACE;
    return hip_status(ah::launch_assign(x, n, d, centroids, L, leaf_out, score_out, workspace,
                                        static_cast<hipStream_t>(stream)));
}

int ah_encode(const void* rows, int32_t rows_dtype, int64_t n, int32_t d, const float* codebooks, int32_t B,
              int32_t dpb, double eta, int32_t sweeps, uint8_t* codes_out, int32_t code_stride, void* stream) {
    if (n < 0 || B < 1 || dpb < 1 || (int64_t)B * dpb != d || code_stride < (B + 1) / 2 || sweeps < 0 ||
        sweeps > 64 || !(eta >= 0.0) || !(eta < 1e300))
        return AH_ERR_SHAPE;
    if ((rows_dtype != AH_F32 && rows_dtype != AH_BF16) || dpb > AH_MAX_DPB || B > AH_MAX_BLOCKS)
        return AH_ERR_UNSUPPORTED;
    if (n == 0) return AH_OK;
    if (!rows || !codebooks || !codes_out) return AH_ERR_NULL;
    return hip_status(ah::launch_encode(rows, rows_dtype, n, d, codebooks, B, dpb, eta, sweeps, codes_out,
                                        code_stride, static_cast<hipStream_t>(stream)));
}

int ah_encode_sweep(const void* rows, int32_t rows_dtype, int64_t n, int32_t d, const float* codebooks, int32_t B,
                    int32_t dpb, double eta, int32_t sweeps, uint8_t* codes_inout, int32_t code_stride, void* stream) {
    if (n < 0 || B < 1 || dpb < 1 || (int64_t)B * dpb != d || code_stride < (B + 1) / 2 || sweeps < 0 ||
        sweeps > 64 || !(eta >= 0.0) || !(eta < 1e300))
        return AH_ERR_SHAPE;
    if ((rows_dtype != AH_F32 && rows_dtype != AH_BF16) || dpb > AH_MAX_DPB || B > AH_MAX_BLOCKS)
        return AH_ERR_UNSUPPORTED;
    if (n == 0) return AH_OK;
    if (!rows || !codebooks || !codes_inout) return AH_ERR_NULL;
    return hip_status(ah::launch_encode(rows, rows_dtype, n, d, codebooks, B, dpb, eta, sweeps, codes_inout,
                                        code_stride, static_cast<hipStream_t>(stream), true));
}

size_t ah_pq_update_workspace_bytes(int64_t n, int32_t B, int32_t dpb) {
    if (n < 0 || B < 1 || dpb < 1 || dpb > AH_MAX_DPB) return 0;
    return ah::pq_update_workspace_bytes(n, B, dpb);
}

int ah_pq_update(const float* x, int64_t n, int32_t d, const uint8_t* codes, int32_t code_stride, int32_t B,
                 int32_t dpb, double eta, float* codebooks, void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 0 || B < 1 || dpb < 1 || (int64_t)B * dpb != d || code_stride < (B + 1) / 2 || !(eta >= 0.0) ||
        !(eta < 1e300))
        return AH_ERR_SHAPE;
    if (dpb > AH_MAX_DPB || B > AH_MAX_BLOCKS) return AH_ERR_UNSUPPORTED;
    if (!codebooks || (n > 0 && (!x || !codes))) return AH_ERR_NULL;
    if (!workspace || workspace_bytes < ah::pq_update_workspace_bytes(n, B, dpb)) return AH_ERR_WORKSPACE;
    return hip_status(ah::launch_pq_update(x, n, d, codes, code_stride, B, dpb, eta, codebooks, workspace,
                                           static_cast<hipStream_t>(stream)));
}

size_t ah_tiled_codes_bytes(int64_t n, int32_t B) {
    if (n < 0 || B < 1) return 0;
    return ah::tiled_codes_bytes(n, B);
}

int ah_tile_codes(const uint8_t* codes, int32_t code_stride, int64_t n, int32_t B, uint8_t* tiled_out,
                  size_t tiled_bytes, void* stream) {
    if (n < 0 || B < 1 || code_stride < (B + 1) / 2) return AH_ERR_SHAPE;
    if (B > AH_MAX_BLOCKS || n >= ((int64_t)1 << 31)) return AH_ERR_UNSUPPORTED;
    if (tiled_bytes < ah::tiled_codes_bytes(n, B)) return AH_ERR_SHAPE;
    if (n == 0) return AH_OK;
    if (!codes || !tiled_out) return AH_ERR_NULL;
    if (!a16(tiled_out)) return AH_ERR_UNSUPPORTED;
    return hip_status(ah::launch_tile_codes(codes, code_stride, n, B, tiled_out, static_cast<hipStream_t>(stream)));
}

int ah_reorder_exact(const float* q, int64_t nq, int32_t d, const void* base, int32_t base_dtype,
                     int64_t n, const int32_t* cand_ids, int32_t R, int32_t k, int32_t* ids_out,
                     float* scores_out, void* stream) {
    if (nq < 0 || d < 1 || n < 0 || R < 1 || k < 1 || k > R) return AH_ERR_SHAPE;
    if ((base_dtype != AH_F32 && base_dtype != AH_BF16) || R > AH_MAX_R || d > AH_MAX_DIM) return AH_ERR_UNSUPPORTED;
    if (nq == 0) return AH_OK;
    if (!q || !cand_ids || !ids_out || !scores_out || (n > 0 && !base)) return AH_ERR_NULL;
    return hip_status(ah::launch_reorder(q, nq, d, base, base_dtype, n, cand_ids, R, k, ids_out,
                                         scores_out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
