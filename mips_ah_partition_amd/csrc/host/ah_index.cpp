// Host-side index build (include/ah_index.h): anisotropic product-quantisation
// codebooks and coupled encoding, float64 arithmetic, OpenMP over rows.
//
// Source: page "ScaNN: Anisotropic Vector Quantization for Maximum Inner
// Product Search", sections "The loss in one paragraph" and "Training an
// anisotropic codebook yourself" (assignment by the loss (eta-1)(u.r)^2 + |r|^2,
// closed-form center update, iterative refinement of coupled block codes).
//
// Determinism: every reduction over rows is split into a fixed number of
// contiguous chunks whose partial sums are combined in chunk order, so the
// result does not depend on the thread count.
#include "../../../include/ah_index.h"

#include <omp.h>

#include <cmath>
#include <cstring>
#include <limits>
#include <vector>

namespace {

constexpr int kC = 16;          // centers per block
constexpr int64_t kChunks = 512;  // fixed reduction chunks

double inv_norm(const float* x, int d) {
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += (double)x[j] * x[j];
    return s > 0.0 ? 1.0 / std::sqrt(s) : 0.0;
}

// Per-block nearest center (squared L2), lowest index on ties.
void nearest_codes(const float* x, const float* cb, int B, int dpb, uint8_t* code) {
    for (int b = 0; b < B; ++b) {
        const float* xb = x + (int64_t)b * dpb;
        double best = std::numeric_limits<double>::infinity();
        int bc = 0;
        for (int c = 0; c < kC; ++c) {
            const float* cc = cb + ((int64_t)b * kC + c) * dpb;
            double nr = 0.0;
            for (int t = 0; t < dpb; ++t) {
                const double r = (double)xb[t] - cc[t];
                nr += r * r;
            }
            if (nr < best) { best = nr; bc = c; }
        }
        code[b] = (uint8_t)bc;
    }
}

// Parallel residual u_b . r_b of every block and their sum; u = v * invn is the
// row's unit direction (v = x itself, or the original row when x is a residual).
double block_projections(const float* x, const float* v, double invn, const float* cb, int B, int dpb,
                         const uint8_t* code, double* proj) {
    double s = 0.0;
    for (int b = 0; b < B; ++b) {
        const float* xb = x + (int64_t)b * dpb;
        const float* vb = v + (int64_t)b * dpb;
        const float* cc = cb + ((int64_t)b * kC + code[b]) * dpb;
        double pr = 0.0;
        for (int t = 0; t < dpb; ++t) pr += (double)vb[t] * invn * ((double)xb[t] - cc[t]);
        proj[b] = pr;
        s += pr;
    }
    return s;
}

// One coordinate-descent sweep over the blocks in order: each block takes the
// center minimising the row's loss with the other blocks fixed.
void cd_sweep(const float* x, const float* v, double invn, const float* cb, int B, int dpb, double eta,
              uint8_t* code, double* proj) {
    double s = 0.0;
    for (int b = 0; b < B; ++b) s += proj[b];
    for (int b = 0; b < B; ++b) {
        const float* xb = x + (int64_t)b * dpb;
        const float* vb = v + (int64_t)b * dpb;
        const double sm = s - proj[b];
        double best = std::numeric_limits<double>::infinity(), bpr = 0.0;
        int bc = code[b];
        for (int c = 0; c < kC; ++c) {
            const float* cc = cb + ((int64_t)b * kC + c) * dpb;
            double pr = 0.0, nr = 0.0;
            for (int t = 0; t < dpb; ++t) {
                const double r = (double)xb[t] - cc[t];
                pr += (double)vb[t] * invn * r;
                nr += r * r;
            }
            const double par = sm + pr;
            const double L = (eta - 1.0) * par * par + nr;
            if (L < best) { best = L; bc = c; bpr = pr; }
        }
        code[b] = (uint8_t)bc;
        proj[b] = bpr;
        s = sm + bpr;
    }
}

double row_loss(const float* x, const float* v, const float* cb, int B, int dpb, double eta, const uint8_t* code) {
    const int d = B * dpb;
    const double invn = inv_norm(v, d);
    double par = 0.0, nr = 0.0;
    for (int b = 0; b < B; ++b) {
        const float* xb = x + (int64_t)b * dpb;
        const float* vb = v + (int64_t)b * dpb;
        const float* cc = cb + ((int64_t)b * kC + code[b]) * dpb;
        for (int t = 0; t < dpb; ++t) {
            const double r = (double)xb[t] - cc[t];
            par += (double)vb[t] * invn * r;
            nr += r * r;
        }
    }
    return (eta - 1.0) * par * par + nr;
}

// Gaussian elimination with partial pivoting on an n x n system (n <= 16).
bool solve(int n, double* A, double* rhs) {
    for (int i = 0; i < n; ++i) {
        int p = i;
        for (int r = i + 1; r < n; ++r)
            if (std::fabs(A[r * n + i]) > std::fabs(A[p * n + i])) p = r;
        if (A[p * n + i] == 0.0) return false;
        if (p != i) {
            for (int c = 0; c < n; ++c) std::swap(A[i * n + c], A[p * n + c]);
            std::swap(rhs[i], rhs[p]);
        }
        for (int r = i + 1; r < n; ++r) {
            const double f = A[r * n + i] / A[i * n + i];
            for (int c = i; c < n; ++c) A[r * n + c] -= f * A[i * n + c];
            rhs[r] -= f * rhs[i];
        }
    }
    for (int i = n - 1; i >= 0; --i) {
        double v = rhs[i];
        for (int c = i + 1; c < n; ++c) v -= A[i * n + c] * rhs[c];
        rhs[i] = v / A[i * n + i];
    }
    return true;
}

double total_loss(const float* X, const float* V, int64_t m, int d, int B, int dpb, double eta, const float* cb,
                  const uint8_t* codes, int64_t cstride) {
    std::vector<double> part(kChunks, 0.0);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ch = 0; ch < kChunks; ++ch) {
        const int64_t a = m * ch / kChunks, z = m * (ch + 1) / kChunks;
        double s = 0.0;
        for (int64_t i = a; i < z; ++i) s += row_loss(X + i * d, V + i * d, cb, B, dpb, eta, codes + i * cstride);
        part[ch] = s;
    }
    double s = 0.0;
    for (double v : part) s += v;
    return s;
}

}  // namespace

extern "C" {

int ahx_train_pq(const float* X, int64_t m, int32_t d, int32_t B, int32_t dpb, double eta, int32_t iters,
                 const int64_t* init_rows, float* codebooks, double* loss_out) {
    return ahx_train_pq_dir(X, nullptr, m, d, B, dpb, eta, iters, init_rows, codebooks, loss_out);
}

int ahx_train_pq_dir(const float* X, const float* V, int64_t m, int32_t d, int32_t B, int32_t dpb, double eta,
                     int32_t iters, const int64_t* init_rows, float* codebooks, double* loss_out) {
    if (!X || !init_rows || !codebooks || m < 1 || B < 1 || dpb < 1 || dpb > 16 || (int64_t)B * dpb != d ||
        iters < 0)
        return -1;
    if (!V) V = X;
    for (int c = 0; c < kC; ++c)
        if (init_rows[c] < 0 || init_rows[c] >= m) return -1;
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < kC; ++c)
            for (int t = 0; t < dpb; ++t)
                codebooks[((int64_t)b * kC + c) * dpb + t] = X[init_rows[c] * d + (int64_t)b * dpb + t];

    std::vector<uint8_t> codes((size_t)m * B);
    std::vector<double> proj((size_t)m * B), invn((size_t)m);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        invn[i] = inv_norm(V + i * d, d);
        nearest_codes(X + i * d, codebooks, B, dpb, &codes[i * B]);
        block_projections(X + i * d, V + i * d, invn[i], codebooks, B, dpb, &codes[i * B], &proj[i * B]);
    }
    if (loss_out) loss_out[0] = total_loss(X, V, m, d, B, dpb, eta, codebooks, codes.data(), B);

    const int nA = dpb * dpb, nAcc = nA + dpb + 1;
    std::vector<double> acc((size_t)kChunks * kC * nAcc);
    std::vector<double> s((size_t)m);
    for (int it = 0; it < iters; ++it) {
        // assignment: one coordinate-descent sweep per row
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < m; ++i)
            cd_sweep(X + i * d, V + i * d, invn[i], codebooks, B, dpb, eta, &codes[i * B], &proj[i * B]);
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < m; ++i) {
            double t = 0.0;
            for (int b = 0; b < B; ++b) t += proj[i * B + b];
            s[i] = t;
        }
        // update: block by block, each with the other blocks' current centers
        for (int b = 0; b < B; ++b) {
            std::fill(acc.begin(), acc.end(), 0.0);
#pragma omp parallel for schedule(dynamic, 1)
            for (int64_t ch = 0; ch < kChunks; ++ch) {
                const int64_t a = m * ch / kChunks, z = m * (ch + 1) / kChunks;
                double* A0 = &acc[(size_t)ch * kC * nAcc];
                for (int64_t i = a; i < z; ++i) {
                    const float* xb = X + i * d + (int64_t)b * dpb;
                    const float* vb = V + i * d + (int64_t)b * dpb;
                    const int c = codes[i * B + b];
                    double* Ac = A0 + c * nAcc;
                    double* rc = Ac + nA;
                    const double sm = s[i] - proj[i * B + b];
                    double ux = 0.0;
                    double u[16];
                    for (int t = 0; t < dpb; ++t) {
                        u[t] = (double)vb[t] * invn[i];
                        ux += u[t] * xb[t];
                    }
                    const double w = (eta - 1.0) * (sm + ux);
                    for (int r = 0; r < dpb; ++r) {
                        for (int t = 0; t < dpb; ++t) Ac[r * dpb + t] += (eta - 1.0) * u[r] * u[t];
                        Ac[r * dpb + r] += 1.0;
                        rc[r] += (double)xb[r] + w * u[r];
                    }
                    rc[dpb] += 1.0;
                }
            }
            for (int c = 0; c < kC; ++c) {
                std::vector<double> A(nA, 0.0), rhs(dpb + 1, 0.0);
                for (int64_t ch = 0; ch < kChunks; ++ch) {
                    const double* Ac = &acc[((size_t)ch * kC + c) * nAcc];
                    for (int e = 0; e < nA; ++e) A[e] += Ac[e];
                    for (int e = 0; e <= dpb; ++e) rhs[e] += Ac[nA + e];
                }
                if (rhs[dpb] == 0.0) continue;  // no rows: keep the center
                if (!solve(dpb, A.data(), rhs.data())) continue;
                for (int t = 0; t < dpb; ++t) codebooks[((int64_t)b * kC + c) * dpb + t] = (float)rhs[t];
            }
            // refresh this block's parallel residuals with the new centers
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < m; ++i) {
                const float* xb = X + i * d + (int64_t)b * dpb;
                const float* vb = V + i * d + (int64_t)b * dpb;
                const float* cc = codebooks + ((int64_t)b * kC + codes[i * B + b]) * dpb;
                double pr = 0.0;
                for (int t = 0; t < dpb; ++t) pr += (double)vb[t] * invn[i] * ((double)xb[t] - cc[t]);
                s[i] += pr - proj[i * B + b];
                proj[i * B + b] = pr;
            }
        }
        if (loss_out) loss_out[it + 1] = total_loss(X, V, m, d, B, dpb, eta, codebooks, codes.data(), B);
    }
    return 0;
}

int ahx_encode(const float* X, int64_t n, int32_t d, int32_t B, int32_t dpb, double eta, const float* codebooks,
               int32_t sweeps, uint8_t* codes, int32_t stride) {
    return ahx_encode_dir(X, nullptr, n, d, B, dpb, eta, codebooks, sweeps, codes, stride);
}

int ahx_encode_dir(const float* X, const float* V, int64_t n, int32_t d, int32_t B, int32_t dpb, double eta,
                   const float* codebooks, int32_t sweeps, uint8_t* codes, int32_t stride) {
    if ((n > 0 && (!X || !codes)) || !codebooks || B < 1 || dpb < 1 || dpb > 16 || (int64_t)B * dpb != d ||
        stride < (B + 1) / 2 || sweeps < 0)
        return -1;
    if (!V) V = X;
#pragma omp parallel
    {
        std::vector<uint8_t> code(B);
        std::vector<double> proj(B);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            const float* x = X + i * d;
            const float* v = V + i * d;
            const double invn = inv_norm(v, d);
            nearest_codes(x, codebooks, B, dpb, code.data());
            block_projections(x, v, invn, codebooks, B, dpb, code.data(), proj.data());
            for (int sw = 0; sw < sweeps; ++sw) cd_sweep(x, v, invn, codebooks, B, dpb, eta, code.data(), proj.data());
            uint8_t* row = codes + i * (int64_t)stride;
            std::memset(row, 0, (size_t)stride);
            for (int b = 0; b < B; ++b) row[b >> 1] |= (uint8_t)(code[b] << (4 * (b & 1)));
        }
    }
    return 0;
}

double ahx_loss(const float* X, int64_t n, int32_t d, int32_t B, int32_t dpb, double eta, const float* codebooks,
                const uint8_t* codes, int32_t stride) {
    std::vector<double> part(kChunks, 0.0);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ch = 0; ch < kChunks; ++ch) {
        const int64_t a = n * ch / kChunks, z = n * (ch + 1) / kChunks;
        std::vector<uint8_t> code(B);
        double s = 0.0;
        for (int64_t i = a; i < z; ++i) {
            const uint8_t* row = codes + i * (int64_t)stride;
            for (int b = 0; b < B; ++b) code[b] = (row[b >> 1] >> (4 * (b & 1))) & 15;
            s += row_loss(X + i * d, X + i * d, codebooks, B, dpb, eta, code.data());
        }
        part[ch] = s;
    }
    double s = 0.0;
    for (double v : part) s += v;
    return s;
}

}  // extern "C"
