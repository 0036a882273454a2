/*
 * ah_index.h -- host (CPU) C ABI for building an asymmetric-hashing index:
 * anisotropic product-quantisation codebooks and the coupled encoding of rows.
 *
 * Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
 * Product Search", sections "The loss in one paragraph" (residual split into
 * parts parallel and orthogonal to x, weight ratio eta), "Training an
 * anisotropic codebook yourself" (k-means-like alternation: assignment by the
 * anisotropic loss, closed-form center update; eta = 1 reduces to k-means) and
 * its closing note that per-block codes are coupled through the parallel
 * component and are refined iteratively.
 *
 * Loss of row x with unit direction u = x/|x| and reconstruction x~ (the
 * concatenation of one center per block):  (eta - 1) * (u.r)^2 + |r|^2 with
 * r = x - x~.  Per block b with the other blocks fixed, the loss in the block's
 * center c is (eta-1)*(s_b + u_b.(x_b - c))^2 + |x_b - c|^2 where s_b is the
 * parallel residual of the other blocks; its minimiser over the rows assigned
 * to c solves
 *     sum_i [(eta-1) u_ib u_ib^T + I] c = sum_i [x_ib + (eta-1)(s_ib + u_ib.x_ib) u_ib],
 * which for one block is the page's per-center linear system with right-hand
 * side sum_i eta_i x_i.
 *
 * All arrays are host memory, row-major; results are deterministic for a given
 * input, whatever the number of threads.  Return 0 or -1 (bad arguments).
 */
#ifndef AH_INDEX_H
#define AH_INDEX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Train codebooks float32 [B][16][dpb] on rows X float32 [m][d] (d == B*dpb).
 * init_rows: 16 distinct row indices whose block values seed every block's
 * centers.  Each of `iters` iterations: one assignment sweep over the blocks in
 * order (each block takes the center minimising the loss with the others
 * fixed, lowest index on ties; the first iteration starts from the per-block
 * nearest center), then one center update per block in order (the solve above;
 * a center with no rows keeps its value).  loss_out[iters+1] (or NULL)
 * receives the total loss before the first and after every iteration. */
int ahx_train_pq(const float* X, int64_t m, int32_t d, int32_t B, int32_t dpb, double eta,
                 int32_t iters, const int64_t* init_rows, float* codebooks, double* loss_out);

/* Encode rows X float32 [n][d] with codebooks [B][16][dpb]: per-block nearest
 * center, then `sweeps` coordinate-descent sweeps over the blocks as in
 * training.  codes uint8 [n][stride] (stride >= ceil(B/2)), low nibble = even
 * block; bytes beyond ceil(B/2) are zeroed. */
int ahx_encode(const float* X, int64_t n, int32_t d, int32_t B, int32_t dpb, double eta,
               const float* codebooks, int32_t sweeps, uint8_t* codes, int32_t stride);

/* The same with the anisotropic direction taken from separate rows: u =
 * V_i / |V_i| while X_i is the vector quantised (the residual variant: X holds
 * residuals from the leaf centroids, V the original rows, since the score
 * error of q.x is q.(r - r~) and its parallel part lies along x).  V may be
 * NULL (then V = X, as in the functions above). */
int ahx_train_pq_dir(const float* X, const float* V, int64_t m, int32_t d, int32_t B, int32_t dpb, double eta,
                     int32_t iters, const int64_t* init_rows, float* codebooks, double* loss_out);
int ahx_encode_dir(const float* X, const float* V, int64_t n, int32_t d, int32_t B, int32_t dpb, double eta,
                   const float* codebooks, int32_t sweeps, uint8_t* codes, int32_t stride);

/* Total loss of an encoding (float64). */
double ahx_loss(const float* X, int64_t n, int32_t d, int32_t B, int32_t dpb, double eta,
                const float* codebooks, const uint8_t* codes, int32_t stride);

#ifdef __cplusplus
}
#endif

#endif /* AH_INDEX_H */
