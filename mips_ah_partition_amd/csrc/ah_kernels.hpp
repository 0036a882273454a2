// Host-side launch interface of the kernels behind the C ABI in include/ah.h.
// The C-ABI layer (ah_api.hip) validates arguments, lays out workspaces and
// calls these; each returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define AH_LUT_MAX_BLOCKS 4096

namespace ah {

hipError_t launch_build_lut(const float* q, int64_t nq, int32_t d, const float* cb, int32_t B,
                            int32_t dpb, float* lut_f32, int8_t* lut_i8, float* scale, float* bias,
                            hipStream_t stream);

size_t partition_workspace_bytes(int64_t nq, int32_t L);
hipError_t launch_partition(const float* q, int64_t nq, int32_t d, const float* cent, int32_t L,
                            int32_t nl, int32_t* leaves, float* scores, void* ws, hipStream_t stream);

struct ScanProblem {
    const int8_t* lut;
    int64_t nq;
    int32_t B;
    const uint8_t* codes;
    int32_t stride;
    int64_t n;
    const int32_t* ids;
    const int64_t* leaf_offsets;
    int32_t L;
    const int32_t* leaves;
    int32_t nl;
    int32_t R;
    int32_t* out_ids;
    int32_t* out_scores;
    int64_t tile_bytes;  // tiled code layout: bytes per 64-row tile (stride = padded row bytes); 0 = row-major
    const int32_t* leaf_bias = nullptr;  // residual variant: [nq][nl] added to the sums of the j-th leaf's rows
    int32_t bias_bound = 0;              // every bias is clipped to [-bias_bound, bias_bound]
};
size_t scan_workspace_bytes(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R);
// Offsets of the per-query append counters and the control words inside the scan workspace.
void scan_counter_offsets(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R, size_t* appended,
                          size_t* control);
// Plain-stream HBM read of n16 16-byte words (measurement hook).
hipError_t launch_read_probe(const void* data, int64_t n16, int32_t blocks_per_cu, uint32_t* sink, hipStream_t stream);
hipError_t launch_scan(const ScanProblem& p, void* ws, size_t ws_bytes, hipStream_t stream,
                       hipEvent_t main_start = nullptr, hipEvent_t main_stop = nullptr);

hipError_t launch_rows_topk(const float* S, int64_t rows, int32_t L, int32_t k, int32_t* ids, float* scores,
                            hipStream_t stream);
// Best k of each row of a candidate list: row r holds rowcnt[r] scores S[r * cap
// + j] with ids idmap[r * cap + j]; rows with rowcnt[r] > cap are skipped.
// cap <= 4096, k <= 512.
// k-means update: centroids[l] = float64 mean of the rows with leaf l (float32), kept when empty.
size_t kmeans_workspace_bytes(int32_t L, int32_t d);
hipError_t launch_kmeans_update(const float* x, int64_t n, int32_t d, const int32_t* leaf, int32_t L, float* cent,
                                int32_t* counts, void* ws, hipStream_t stream);
// Residual variant's per-leaf term: clip(rint((s[q][j] - s[q][0]) / step[q]), -bound, bound), 0 when step is 0.
hipError_t launch_residual_bias(const float* scores, const float* step, int64_t nq, int32_t nl, int32_t bound,
                                int32_t* bias, hipStream_t stream);
hipError_t launch_list_topk(const float* S, const int32_t* idmap, const uint32_t* rowcnt, int64_t rows, int32_t cap,
                            int32_t k, int32_t* ids, float* scores, hipStream_t stream);

hipError_t launch_sq8_quantize(const float* x, int64_t n, int32_t d, double pct, int8_t* codes, float* scale,
                               hipStream_t stream);
size_t sq8_workspace_bytes(int64_t nq, int64_t n, int32_t d, int32_t R);
// d4 non-null: the documents are 4-bit codes [n][d/2] standing for the int8
// values levels[16] (host memory), instead of int8 rows d8.
hipError_t launch_sq8_topk(const int8_t* q8, const float* qs, int64_t nq, const int8_t* d8, const float* ds,
                           int64_t n, int32_t d, int32_t R, int32_t* ids, float* scores, void* ws,
                           hipStream_t stream, const uint8_t* d4 = nullptr, const int8_t* levels = nullptr);

// Training-free rotation quantiser: block Hadamard rotation of rows, and the
// nearest-level 4-bit encoding with the norm-restoring row step.
hipError_t launch_rslm_rotate(const float* x, int64_t n, int32_t d, const float* signs, const int32_t* perm,
                              float* y, hipStream_t stream);
hipError_t launch_rslm_encode(const float* y, int64_t n, int32_t d, const float* levels, const float* mids,
                              double lam, uint8_t* codes, float* step, hipStream_t stream);

size_t assign_workspace_bytes(int64_t n, int32_t L);
hipError_t launch_assign(const float* x, int64_t n, int32_t d, const float* cent, int32_t L, int32_t* leaves,
                         float* scores, void* ws, hipStream_t stream);

hipError_t launch_encode(const void* rows, int32_t dtype, int64_t n, int32_t d, const float* cb, int32_t B,
                         int32_t dpb, double eta, int32_t sweeps, uint8_t* codes, int32_t stride,
                         hipStream_t stream, bool from_codes = false);

// Anisotropic codebook training: the block-by-block closed-form center update at fixed codes.
size_t pq_update_workspace_bytes(int64_t n, int32_t B, int32_t dpb);
hipError_t launch_pq_update(const float* x, int64_t n, int32_t d, const uint8_t* codes, int32_t stride, int32_t B,
                            int32_t dpb, double eta, float* cb, void* ws, hipStream_t stream);

size_t tiled_codes_bytes(int64_t n, int32_t B);
hipError_t launch_tile_codes(const uint8_t* codes, int32_t stride, int64_t n, int32_t B, uint8_t* tiled,
                             hipStream_t stream);

hipError_t launch_reorder(const float* q, int64_t nq, int32_t d, const void* base, int32_t dtype,
                          int64_t n, const int32_t* cand, int32_t R, int32_t k, int32_t* ids,
                          float* scores, hipStream_t stream);

}  // namespace ah
