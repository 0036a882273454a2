/*
 * ah.h -- C ABI of the MI355X (gfx950) asymmetric-hashing search path.
 *
 * The four calls follow the query path of the page "ScaNN: Anisotropic Vector
 * Quantization for Maximum Inner Product Search", section "Three stages of a
 * search": a query scores every partition centroid and descends into the best
 * leaves (ah_partition_score); a lookup table of q.center per block of
 * dimensions is built (ah_build_lut); a row's approximate score is the sum of
 * its table entries, and the best candidates are kept (ah_scan_topk); the best
 * few hundred candidates are rescored with exact dot products
 * (ah_reorder_exact).  Codebooks, centroids and codes are trained on the host
 * and passed in.
 *
 * Conventions shared by every call
 *  - Every array pointer is a DEVICE pointer to row-major, contiguous memory
 *    owned by the caller; the library keeps no pointer after a call returns and
 *    holds no global mutable state, so calls on distinct streams are safe (the
 *    one exception, ah_scan_topk_noalloc, keeps its scratch in a static array
 *    per GPU; see there).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns; device faults surface at the
 *    caller's next synchronisation.  The caller keeps inputs, outputs and
 *    workspace alive until the stream has finished the work.
 *  - Return value: AH_OK (0) or a negative AH_ERR_* code, checked on the host
 *    before anything is enqueued (AH_ERR_HIP reports a failed launch).
 *    ah_status_string() describes a code.  nq == 0 is a successful no-op.
 *  - Rankings order by score descending, then by id ascending, so every kept
 *    set is unique.
 *  - Codes: row-major, `code_stride` bytes per row (>= ceil(B/2)); block b of a
 *    row is the nibble (row[b/2] >> 4*(b%2)) & 15 (low nibble = even block).
 *    Or (code_stride == AH_CODES_TILED) the tiled layout of ah_tile_codes: the
 *    same bytes, rearranged so that one 16-byte segment of 64 consecutive rows
 *    is one contiguous 1 KB run.
 */
#ifndef AH_H
#define AH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    AH_OK = 0,
    AH_ERR_NULL = -1,        /* a required pointer is NULL */
    AH_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
    AH_ERR_UNSUPPORTED = -3, /* valid but not supported (dtype, limits below) */
    AH_ERR_WORKSPACE = -4,   /* workspace pointer NULL or smaller than required */
    AH_ERR_HIP = -5          /* a HIP launch failed */
};

enum { AH_F32 = 0, AH_BF16 = 1 };

/* Limits (AH_ERR_UNSUPPORTED beyond them). */
#define AH_MAX_BLOCKS 4096   /* B */
#define AH_MAX_DPB 16        /* dimensions_per_block */
#define AH_MAX_R 4096        /* pre-reorder candidates (also max nl and k) */
#define AH_MAX_DIM 16384     /* d */

#define AH_MAX_ASSIGN_LEAVES 4096 /* L for ah_assign_leaves */
#define AH_MAX_LEAF_BIAS (1 << 24) /* bias_bound of the residual scan */

/* code_stride value selecting the tiled code layout (see ah_tile_codes); a
 * negative sentinel, so that a zero stride is rejected rather than taken as
 * the tiled layout. */
#define AH_CODES_TILED (-1)

const char* ah_status_string(int status);
int ah_version(void);

/* ---------------------------------------------------------------------------
 * Step 1: centroid scoring and leaf choice (ScaNN page, "Three stages of a
 * search": a query scores every centroid and descends into the best
 * num_leaves_to_search; cost on the worked example: 1,000 centroids x 128 dims).
 *
 *   q          float32 [nq][d]   queries
 *   centroids  float32 [L][d]    partition centroids
 *   leaves_out int32   [nq][nl]  best nl leaf ids, best first
 *   leaf_scores_out float32 [nq][nl] their scores q.c (fp32 accumulation), or NULL
 *   workspace  >= ah_partition_workspace_bytes(nq, L) bytes of device memory
 * Errors: AH_ERR_NULL (q, centroids, leaves_out, workspace), AH_ERR_SHAPE
 * (nq < 0, d < 1, L < 1, nl < 1 or nl > L), AH_ERR_UNSUPPORTED (d > AH_MAX_DIM,
 * nl > AH_MAX_R), AH_ERR_WORKSPACE.
 */
size_t ah_partition_workspace_bytes(int64_t nq, int32_t L);
int ah_partition_score(const float* q, int64_t nq, int32_t d, const float* centroids, int32_t L,
                       int32_t nl, int32_t* leaves_out, float* leaf_scores_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Step 2: per-query lookup table (ScaNN page, "Three stages of a search":
 * a table of q.center per block; each vector is split into blocks of
 * dimensions_per_block dims, each replaced by one of 16 centers).
 *
 *   q          float32 [nq][d]
 *   codebooks  float32 [B][16][dpb]   (d == B*dpb)
 *   lut_f32_out float32 [nq][B][16]   T[q][b][c] = sum_t q[b*dpb+t]*cb[b][c][t], or NULL;
 *                                     the sum is taken in float64 in t order and rounded
 *                                     once to float32 (so T is the float32 rounding of a
 *                                     float64 left-to-right sum of exact products)
 *   lut_i8_out  int8    [nq][B][16]   int8 table
 *   scale_out   float32 [nq]          per-query step s
 *   bias_out    float32 [nq]          per-query bias beta
 * int8 table (fp32 arithmetic in this order): lo_b/hi_b = min/max over c of
 * T[q][b][.]; m_b = 0.5f*(lo_b+hi_b); Rng = max_b(hi_b-lo_b); if Rng > 0:
 * T8 = clamp(rint((T - m_b) * (254.0f/Rng)), -127, 127), s = Rng/254.0f, else
 * T8 = 0, s = 0; beta = sum of m_b in block order.  The approximate score of a
 * row is beta + s * sum_b T8[q][b][code_b].
 * Errors: AH_ERR_NULL, AH_ERR_SHAPE (d != B*dpb, B < 1, dpb < 1, nq < 0),
 * AH_ERR_UNSUPPORTED (B > AH_MAX_BLOCKS, dpb > AH_MAX_DPB).
 */
int ah_build_lut(const float* q, int64_t nq, int32_t d, const float* codebooks, int32_t B,
                 int32_t dpb, float* lut_f32_out, int8_t* lut_i8_out, float* scale_out,
                 float* bias_out, void* stream);

/* ---------------------------------------------------------------------------
 * Steps 3+4: code scan and top-R (ScaNN page, "Three stages of a search": a
 * row's approximate score is the sum of its table entries; "Using the library":
 * the best pre_reorder_num_neighbors go on to reorder; worked example: the scan
 * dominates the cost of a query).
 *
 *   lut_i8       int8 [nq][B][16]
 *   codes        uint8 [n][code_stride]  (leaf-sorted when partitioned), or the
 *                tiled layout of ah_tile_codes when code_stride == AH_CODES_TILED
 *                (then 16-byte aligned, else AH_ERR_UNSUPPORTED)
 *   ids          int32 [n] original row id of each code row, or NULL (= row index)
 *   leaf_offsets int64 [L+1] rows of leaf l are [leaf_offsets[l], leaf_offsets[l+1]),
 *                or NULL when leaves == NULL
 *   leaves       int32 [nq][nl] leaves each query scans (distinct per query), or
 *                NULL = every query scans all n rows
 *   cand_ids_out    int32 [nq][R]  original ids, best first
 *   cand_scores_out int32 [nq][R]  their exact integer sums sum_b T8[q][b][code_b]
 *   Slots beyond the number of scanned rows hold (-1, INT32_MIN).
 *   workspace    >= ah_scan_workspace_bytes(nq, B, n, L, nl, R) bytes
 * Sums are exact int32; the kept set is the unique top-R by (sum desc, id asc).
 * Errors: AH_ERR_NULL, AH_ERR_SHAPE (nq < 0, n < 0, B < 1, code_stride neither
 * AH_CODES_TILED nor >= ceil(B/2), R < 1, leaves given with L < 1 or nl < 1 or nl > L or no
 * leaf_offsets), AH_ERR_UNSUPPORTED (B > AH_MAX_BLOCKS, R > AH_MAX_R,
 * n >= 2^31), AH_ERR_WORKSPACE.
 */
size_t ah_scan_workspace_bytes(int64_t nq, int32_t B, int64_t n, int32_t L, int32_t nl, int32_t R);
int ah_scan_topk(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes,
                 int32_t code_stride, int64_t n, const int32_t* ids, const int64_t* leaf_offsets,
                 int32_t L, const int32_t* leaves, int32_t nl, int32_t R, int32_t* cand_ids_out,
                 int32_t* cand_scores_out, void* workspace, size_t workspace_bytes, void* stream);

/* ah_scan_topk without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The scan's scratch (thresholds, counters,
 * histograms, candidate lists, fallback slots, leaf inversion) lives in one
 * static device array of AH_SCAN_SCRATCH_BYTES per GPU, held by every GPU the
 * library runs on until the process ends; its address is looked up once per
 * device on the first call.  The call allocates nothing and clears, with its
 * own kernels, everything the scan needs to start from zero.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and give wrong results; serialise them.
 * Arguments, results and errors are those of ah_scan_topk, plus
 * AH_ERR_UNSUPPORTED when ah_scan_workspace_bytes(nq, B, n, L, nl, R) exceeds
 * AH_SCAN_SCRATCH_BYTES, and AH_ERR_HIP if the array's address cannot be had. */
#define AH_SCAN_SCRATCH_BYTES (128u << 20)
int ah_scan_topk_noalloc(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes,
                         int32_t code_stride, int64_t n, const int32_t* ids, const int64_t* leaf_offsets,
                         int32_t L, const int32_t* leaves, int32_t nl, int32_t R, int32_t* cand_ids_out,
                         int32_t* cand_scores_out, void* stream);

/* ---------------------------------------------------------------------------
 * Int8 scalar-quantised flat search (a second workload; page "Incoherence-Aware
 * Asymmetric Quantization for Retrieval": a robust per-vector int8 scale, and
 * "A Specialized int8 Retrieval Engine": exact integer dots scaled by both
 * steps, best k).  The exact rescore of the kept candidates is
 * ah_reorder_exact.
 *
 * ah_sq8_quantize: per row, P = the pct-th percentile of |x| (linear
 * interpolation between order statistics, every step in float32 as numpy
 * computes it for a float32 vector), step s = max(P, 1e-8) / 127 (float32),
 * codes clip(round_half_even(x / s), -127, 127).
 *   x          float32 [n][d];  pct in [0, 100] (the page uses 99.9)
 *   codes_out  int8 [n][d];  scale_out float32 [n]
 * Errors: AH_ERR_SHAPE (n < 0, d < 1, pct outside [0, 100]),
 * AH_ERR_UNSUPPORTED (d > AH_MAX_DIM), AH_ERR_NULL.
 *
 * ah_sq8_scan_topk: for every query the R best documents by
 * score = ((float)(q8 . d8) * q_scale) * d_scale (float32 products left to
 * right, the integer dot exact), ties to the lower document id.
 *   q8 int8 [nq][d], q_scale float32 [nq], d8 int8 [n][d], d_scale float32 [n]
 *   ids_out int32 [nq][R], scores_out float32 [nq][R] (or NULL)
 *   workspace >= ah_sq8_workspace_bytes(nq, n, d, R) bytes (0 for invalid sizes)
 * Errors: AH_ERR_SHAPE (nq < 0, n < 1, d < 1, R < 1, R > n), AH_ERR_UNSUPPORTED
 * (d % 16 != 0, q8 or d8 not 16-byte aligned, d > AH_MAX_DIM, R > AH_MAX_R,
 * n >= 2^31), AH_ERR_NULL, AH_ERR_WORKSPACE.
 */
int ah_sq8_quantize(const float* x, int64_t n, int32_t d, double pct, int8_t* codes_out, float* scale_out,
                    void* stream);
size_t ah_sq8_workspace_bytes(int64_t nq, int64_t n, int32_t d, int32_t R);
int ah_sq8_scan_topk(const int8_t* q8, const float* q_scale, int64_t nq, const int8_t* d8, const float* d_scale,
                     int64_t n, int32_t d, int32_t R, int32_t* ids_out, float* scores_out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Training-free rotation quantiser (page "RSLM: Training-Free Vector
 * Quantization for Approximate Nearest Neighbor Search", method points: a
 * block-wise cascaded fast Walsh-Hadamard rotation of block size 128 with sign
 * flips and a permutation, the tail dimensions handled by an overlapping block;
 * a fixed Lloyd-Max codebook of at most 16 centroids for the rotated
 * coordinates; a global scale restoring the L2 norm of the final
 * reconstruction), 4 bits per dimension, scored on the int8 matrix cores.
 *
 * ah_rslm_rotate: y = rotation of x, per row: v = x * signs, v'[j] = v[perm[j]],
 * then the orthonormal Sylvester Hadamard H_b / sqrt(b) on the blocks [k b,
 * (k+1) b), k < d / b, and, when b does not divide d, on the tail block
 * [d - b, d) last (b = min(128, largest power of two <= d)).  float32 butterflies.
 *   x, y_out float32 [n][d];  signs float32 [d] (+-1);  perm int32 [d] (a permutation)
 * Errors: AH_ERR_SHAPE (n < 0, d < 1), AH_ERR_UNSUPPORTED (d > AH_MAX_DIM), AH_ERR_NULL.
 *
 * ah_rslm_encode: 4-bit codes of rotated rows against 16 ascending levels
 * (host memory; the Lloyd-Max levels of N(0,1)): f = float32(sqrt(d) / |y|)
 * (0 for a zero row), u = y * f (float32), code = number of midpoints
 * float32((L[c] + L[c+1]) / 2) strictly below u (the nearest level, ties to the
 * lower); step = (|y| / |L[code]|) / Lam with Lam = 127 / L[15] (squares summed
 * in float64), so that step * Lam * L[code] has the row's norm.
 *   y float32 [n][d];  codes_out uint8 [n][ceil(d/2)] (low nibble = even
 *   dimension);  step_out float32 [n]
 * Errors: AH_ERR_SHAPE (n < 0, d < 1, levels not strictly increasing or
 * L[15] <= 0), AH_ERR_UNSUPPORTED (d > AH_MAX_DIM), AH_ERR_NULL.
 *
 * ah_rslm_scan_topk: the int8 flat search (ah_sq8_scan_topk) with each
 * document's int8 values levels_i8[code] (host memory, 16 bytes; usually
 * rint(L[c] * Lam)) read from its 4-bit codes, and step as the document step:
 * score = ((float)(q8 . levels_i8[codes]) * q_scale) * step, top-R by (score
 * desc, id asc).  q8 and q_scale are the rotated queries' int8 codes and steps
 * from ah_sq8_quantize.
 *   codes uint8 [n][d/2], 8-byte aligned;  workspace >= ah_sq8_workspace_bytes(nq, n, d, R)
 * Errors: as ah_sq8_scan_topk (codes not 8-byte aligned: AH_ERR_UNSUPPORTED).
 */
int ah_rslm_rotate(const float* x, int64_t n, int32_t d, const float* signs, const int32_t* perm, float* y_out,
                   void* stream);
int ah_rslm_encode(const float* y, int64_t n, int32_t d, const float* levels, uint8_t* codes_out, float* step_out,
                   void* stream);
int ah_rslm_scan_topk(const int8_t* q8, const float* q_scale, int64_t nq, const uint8_t* codes, const float* step,
                      int64_t n, int32_t d, const int8_t* levels_i8, int32_t R, int32_t* ids_out, float* scores_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Partition assignment (the k-means assignment step behind the partition the
 * first stage searches; ScaNN page, section "Three stages of a search"): each
 * row goes to the centroid nearest to it.
 *
 *   x          float32 [n][d] rows
 *   centroids  float32 [L][d], L <= AH_MAX_ASSIGN_LEAVES
 *   leaf_out   int32 [n]  argmin_l |x - c_l|^2, computed as argmax_l
 *              (x . c_l - |c_l|^2 / 2) in fp32 (MFMA contraction, fp32
 *              accumulation), lowest leaf id on ties
 *   score_out  float32 [n] that maximum, or NULL
 *   workspace  >= ah_assign_workspace_bytes(n, L) bytes
 * Errors: AH_ERR_NULL, AH_ERR_SHAPE (n < 0, d < 1, L < 1),
 * AH_ERR_UNSUPPORTED (L > AH_MAX_ASSIGN_LEAVES, d > AH_MAX_DIM), AH_ERR_WORKSPACE.
 */
size_t ah_assign_workspace_bytes(int64_t n, int32_t L);
int ah_assign_leaves(const float* x, int64_t n, int32_t d, const float* centroids, int32_t L, int32_t* leaf_out,
                     float* score_out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The partition's k-means update step (with ah_assign_leaves, one Lloyd
 * iteration on the GPU; the ScaNN page's partition groups rows under
 * centroids, and a centroid is the mean of its rows): for every leaf l with
 * rows, centroids[l] = float32(sum of its rows in float64 / their number); a
 * leaf without rows keeps its centroid.  The float64 sums are taken by atomic
 * adds in no fixed order, so a result may differ from a row-order sum by one
 * float32 unit.  Rows whose leaf is outside [0, L) are left out.
 *   x float32 [n][d];  leaf_of_row int32 [n];  centroids float32 [L][d] (in:
 *   previous, out: updated);  counts_out int32 [L] rows per leaf, or NULL
 *   workspace >= ah_kmeans_workspace_bytes(L, d) bytes
 * Errors: AH_ERR_SHAPE (n < 0, d < 1, L < 1), AH_ERR_UNSUPPORTED (d >
 * AH_MAX_DIM, n >= 2^32), AH_ERR_NULL, AH_ERR_WORKSPACE.
 */
size_t ah_kmeans_workspace_bytes(int32_t L, int32_t d);
int ah_kmeans_update(const float* x, int64_t n, int32_t d, const int32_t* leaf_of_row, int32_t L, float* centroids,
                     int32_t* counts_out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Encoding: the codes the scan reads (ScaNN page, sections "The loss in one
 * paragraph" and "Training an anisotropic codebook yourself": a row's loss is
 * (eta-1)*(u.r)^2 + |r|^2 for its residual r = x - decode(code) and direction
 * u = x/|x|; the coupled block choices are refined iteratively).  Reading
 * taken: block-coordinate descent from the per-block nearest centers (squared
 * L2), `sweeps` sweeps over b = 0..B-1, each block taking the center that
 * minimises the row's loss with the other blocks fixed; ties to the lowest
 * center index.  Float64 arithmetic in a fixed order, so the codes are
 * reproducible bit for bit.
 *
 *   rows       [n][d] float32 (rows_dtype AH_F32) or bfloat16 (AH_BF16)
 *   codebooks  float32 [B][16][dpb], d == B * dpb
 *   eta        >= 0 (1 = plain nearest-center encoding); sweeps 0..64
 *   codes_out  uint8 [n][code_stride] (code_stride >= ceil(B/2)), nibbles as
 *              described above; bytes past ceil(B/2) are written as zero
 * Errors: AH_ERR_SHAPE (n < 0, B < 1, dpb < 1, d != B*dpb, code_stride <
 * ceil(B/2), sweeps outside 0..64, eta < 0 or not finite), AH_ERR_UNSUPPORTED
 * (dtype, dpb > AH_MAX_DPB, B > AH_MAX_BLOCKS), AH_ERR_NULL.
 */
int ah_encode(const void* rows, int32_t rows_dtype, int64_t n, int32_t d, const float* codebooks, int32_t B,
              int32_t dpb, double eta, int32_t sweeps, uint8_t* codes_out, int32_t code_stride, void* stream);

/* The same descent started from the codes already in codes_inout (no nearest-
 * center start): `sweeps` sweeps, results written back in place.  With
 * ah_pq_update this is one iteration of anisotropic codebook training (ScaNN
 * page, "Training an anisotropic codebook yourself": assign by the loss,
 * update each center in closed form).  Arguments and errors as ah_encode. */
int ah_encode_sweep(const void* rows, int32_t rows_dtype, int64_t n, int32_t d, const float* codebooks, int32_t B,
                    int32_t dpb, double eta, int32_t sweeps, uint8_t* codes_inout, int32_t code_stride, void* stream);

/* Center update of anisotropic codebook training at fixed codes, block by block
 * in order, each with the other blocks' current centers: block b's center c
 * solves  sum_i [(eta-1) u u^T + I] c = sum_i [x_ib + (eta-1)(s_i - p_ib + u.x_ib) u]
 * over the rows coded c (u = x_ib/|x|, p_ib = u.(x_ib - center), s_i = sum_b
 * p_ib at the current centers), by Gaussian elimination with partial pivoting
 * in float64; a center with no rows, or a singular system, keeps its value;
 * block b's p_ib and s_i are refreshed before block b+1.  The float64 sums are
 * taken in no fixed order (results agree with a row-order sum to rounding).
 *   x float32 [n][d] (d == B * dpb);  codes uint8 [n][code_stride];
 *   codebooks float32 [B][16][dpb] (in: current, out: updated)
 *   workspace >= ah_pq_update_workspace_bytes(n, B, dpb) bytes
 * Errors: AH_ERR_SHAPE (n < 0, B < 1, dpb < 1, d != B*dpb, code_stride <
 * ceil(B/2), eta < 0 or not finite), AH_ERR_UNSUPPORTED (dpb > AH_MAX_DPB,
 * B > AH_MAX_BLOCKS), AH_ERR_NULL, AH_ERR_WORKSPACE. */
size_t ah_pq_update_workspace_bytes(int64_t n, int32_t B, int32_t dpb);
int ah_pq_update(const float* x, int64_t n, int32_t d, const uint8_t* codes, int32_t code_stride, int32_t B,
                 int32_t dpb, double eta, float* codebooks, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Code layout for the scan (same page and section as the scan: the codes are
 * read once per query batch, so their layout decides how well the reads
 * coalesce).  Not a step of the method: a rearrangement of the same bytes.
 *
 * ah_tile_codes writes the tiled layout of row-major codes:
 *   codes      uint8 [n][code_stride] row-major (code_stride >= ceil(B/2))
 *   tiled_out  >= ah_tiled_codes_bytes(n, B) bytes, 16-byte aligned
 * With S = ceil(ceil(B/2) / 16) segments of 16 bytes per row (the last padded
 * with zero bytes), byte k of row r goes to
 *   (r / 64) * (64 * S * 16) + (k / 16) * 1024 + (r % 64) * 16 + k % 16;
 * slots of the last tile past row n - 1 are zero.  Pass the result to
 * ah_scan_topk with code_stride = AH_CODES_TILED; ids, leaf_offsets and leaves
 * keep referring to row numbers.
 * Errors: AH_ERR_SHAPE (n < 0, B < 1, code_stride < ceil(B/2), tiled_bytes too
 * small), AH_ERR_UNSUPPORTED (B > AH_MAX_BLOCKS, n >= 2^31, tiled_out not 16-byte
 * aligned), AH_ERR_NULL.  ah_tiled_codes_bytes returns 0 for n < 0 or B < 1.
 */
size_t ah_tiled_codes_bytes(int64_t n, int32_t B);
int ah_tile_codes(const uint8_t* codes, int32_t code_stride, int64_t n, int32_t B, uint8_t* tiled_out,
                  size_t tiled_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Residual (leaf-relative) variant of steps 3+4 (page "RSLM: Training-Free
 * Vector Quantization for Approximate Nearest Neighbor Search", relative mode:
 * a row is coded as its residual from a coarse approximation; here the coarse
 * approximation is the row's leaf centroid, so q.x = q.c_leaf + q.residual and
 * the table, built from the residual codebooks, scores the residual).
 *
 * ah_residual_leaf_bias: the leaf term in table units for each probed leaf:
 *   bias_out[q][j] = clip(rint((leaf_scores[q][j] - leaf_scores[q][0]) / step[q]),
 *                         -bias_bound, bias_bound)
 * in float32 (round half to even), 0 for a query whose step is 0 (a constant
 * table).  leaf_scores float32 [nq][nl] is ah_partition_score's scores_out (the
 * first leaf is the best one), step float32 [nq] is ah_build_lut's scale_out.
 *   bias_out int32 [nq][nl]
 * Errors: AH_ERR_SHAPE (nq < 0, nl < 1, bias_bound < 0), AH_ERR_UNSUPPORTED
 * (bias_bound > AH_MAX_LEAF_BIAS), AH_ERR_NULL.
 *
 * ah_scan_topk_residual: ah_scan_topk over the listed leaves, a row of the
 * query's j-th leaf scoring its sum plus clip(leaf_bias[q][j], -bias_bound,
 * bias_bound); the kept set is the unique top-R by (score desc, id asc) and
 * cand_scores_out holds those int32 scores.  Arguments as ah_scan_topk, plus
 *   leaf_bias   int32 [nq][nl] (device), aligned with leaves
 *   bias_bound  in [0, AH_MAX_LEAF_BIAS]; a larger bound coarsens the scan's
 *               internal score histograms (255 B + 2 bias_bound values over
 *               1,024 bins), so the threshold rises in coarser steps
 *   workspace   >= ah_scan_workspace_bytes(nq, B, n, L, nl, R) bytes
 * Errors: as ah_scan_topk; AH_ERR_SHAPE also when leaves is NULL or
 * bias_bound < 0, AH_ERR_NULL when leaf_bias is NULL, AH_ERR_UNSUPPORTED when
 * bias_bound > AH_MAX_LEAF_BIAS.
 */
int ah_residual_leaf_bias(const float* leaf_scores, const float* step, int64_t nq, int32_t nl, int32_t bias_bound,
                          int32_t* bias_out, void* stream);
int ah_scan_topk_residual(const int8_t* lut_i8, int64_t nq, int32_t B, const uint8_t* codes, int32_t code_stride,
                          int64_t n, const int32_t* ids, const int64_t* leaf_offsets, int32_t L,
                          const int32_t* leaves, int32_t nl, const int32_t* leaf_bias, int32_t bias_bound, int32_t R,
                          int32_t* cand_ids_out, int32_t* cand_scores_out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------
 * Step 5: exact reorder (ScaNN page, "Three stages of a search": the best few
 * hundred candidates are rescored with exact dot products; "Failure modes":
 * reorder must keep more than k).
 *
 *   q         float32 [nq][d]
 *   base      [n][d] stored rows, float32 (AH_F32) or bf16 bits (AH_BF16)
 *   cand_ids  int32 [nq][R]  candidate ids, -1 = empty slot (skipped)
 *   ids_out   int32 [nq][k]  best k by exact score, best first
 *   scores_out float32 [nq][k] exact q.x (bf16 rows widened exactly to fp32,
 *             products and sum in fp64, rounded once to fp32); ranking by
 *             (that fp32 score desc, id asc); empty slots (-1, -inf)
 * Errors: AH_ERR_NULL, AH_ERR_SHAPE (nq < 0, d < 1, n < 0, R < 1, k < 1,
 * k > R), AH_ERR_UNSUPPORTED (dtype, R > AH_MAX_R, d > AH_MAX_DIM).  Candidate
 * ids must lie in [-1, n).
 */
int ah_reorder_exact(const float* q, int64_t nq, int32_t d, const void* base, int32_t base_dtype,
                     int64_t n, const int32_t* cand_ids, int32_t R, int32_t k, int32_t* ids_out,
                     float* scores_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AH_H */
