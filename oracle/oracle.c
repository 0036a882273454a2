/*
 * CPU oracle for the asymmetric-hashing (AH) search path -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, deliberately unoptimised C.  Each function writes out the plain
 * definition of one step of the query path described on the page "ScaNN:
 * Anisotropic Vector Quantization for Maximum Inner Product Search", section
 * "Three stages of a search" (partition scoring, per-block lookup table,
 * sum of table entries, keep the best candidates, exact reorder).
 *
 * This file shares no code, header or constant with the GPU library: it is
 * compiled on its own (oracle/build.py) and is used only by tests/, by the
 * smoke check and by the benchmark's CPU-baseline leg.
 *
 * Conventions (readings of what the pages leave open):
 *  - code of row i, block b: (codes[i*stride + b/2] >> (4*(b&1))) & 15, i.e. the
 *    low nibble holds the even block;
 *  - every ranking orders by score descending, then by id ascending, so the
 *    kept set is unique;
 *  - int8 table: per block the centre m_b = 0.5*(lo_b+hi_b), one per-query step
 *    s = Rng/254 with Rng = max_b (hi_b - lo_b), entries rint((v - m_b)*254/Rng)
 *    clamped to [-127,127] (rint = round half to even, as in the int8 lesson's
 *    "ties go to the even mark"), bias = sum_b m_b accumulated in block order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

typedef struct { int32_t score; int32_t id; } ISC;
typedef struct { double score; int32_t id; } DSC;

static int cmp_isc(const void* a, const void* b) {
    const ISC* x = (const ISC*)a; const ISC* y = (const ISC*)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    return (x->id > y->id) - (x->id < y->id);
}
static int cmp_dsc(const void* a, const void* b) {
    const DSC* x = (const DSC*)a; const DSC* y = (const DSC*)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    return (x->id > y->id) - (x->id < y->id);
}

int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int t) { if (t > 0) omp_set_num_threads(t); }

/* Nibble of block b in a row-major code row. */
static inline int code_of(const uint8_t* row, int32_t b) {
    return (row[b >> 1] >> (4 * (b & 1))) & 15;
}

/* Step 3 of the page: approximate score of one row = sum over blocks of that
 * block's table entry at the row's code.  Integer, exact. */
static inline int32_t adc_sum(const int8_t* lut_q, int32_t B, const uint8_t* row) {
    int32_t s = 0;
    for (int32_t b = 0; b < B; ++b) s += (int32_t)lut_q[b * 16 + code_of(row, b)];
    return s;
}

/* All sums of every query against every row: out[q*n + i]. */
void oracle_scan_sums(const int8_t* lut, int64_t nq, int32_t B, const uint8_t* codes,
                      int64_t n, int32_t stride, int32_t* out) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nq; ++q)
        for (int64_t i = 0; i < n; ++i)
            out[q * n + i] = adc_sum(lut + q * (int64_t)B * 16, B, codes + i * (int64_t)stride);
}

/* Steps 3+4: for each query, score every row of the leaves it searches (all rows
 * when leaves == NULL), sort all (sum, id) pairs by (sum desc, id asc) and keep
 * the first R.  Missing slots are (-1, INT32_MIN).
 *
 * Residual (leaf-relative) variant, when bias != NULL (the RSLM summary page:
 * in its relative mode a row is coded as the residual from a coarse
 * approximation; with the leaf centroid as that approximation, q.x = q.c_leaf +
 * q.residual, and the table scores the residual): a row of the query's j-th
 * leaf scores sum + bias[q*nl + j], the bias clamped to [-bound, bound]. */
static inline int32_t clamp_bias(int32_t v, int32_t bound) {
    return v < -bound ? -bound : (v > bound ? bound : v);
}

void oracle_scan_topk(const int8_t* lut, int64_t nq, int32_t B, const uint8_t* codes, int64_t n,
                      int32_t stride, const int32_t* ids, const int64_t* leaf_offsets, int32_t L,
                      const int32_t* leaves, int32_t nl, int32_t R, int32_t* out_ids,
                      int32_t* out_scores, const int32_t* bias, int32_t bound) {
    (void)L;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nq; ++q) {
        int64_t total = 0;
        if (leaves) {
            for (int32_t j = 0; j < nl; ++j) {
                int32_t l = leaves[q * nl + j];
                total += leaf_offsets[l + 1] - leaf_offsets[l];
            }
        } else {
            total = n;
        }
        ISC* all = (ISC*)malloc(sizeof(ISC) * (size_t)(total > 0 ? total : 1));
        int64_t m = 0;
        const int8_t* lq = lut + q * (int64_t)B * 16;
        if (leaves) {
            for (int32_t j = 0; j < nl; ++j) {
                int32_t l = leaves[q * nl + j];
                int32_t add = bias ? clamp_bias(bias[q * nl + j], bound) : 0;
                for (int64_t i = leaf_offsets[l]; i < leaf_offsets[l + 1]; ++i) {
                    all[m].score = adc_sum(lq, B, codes + i * (int64_t)stride) + add;
                    all[m].id = ids ? ids[i] : (int32_t)i;
                    ++m;
                }
            }
        } else {
            for (int64_t i = 0; i < n; ++i) {
                all[m].score = adc_sum(lq, B, codes + i * (int64_t)stride);
                all[m].id = ids ? ids[i] : (int32_t)i;
                ++m;
            }
        }
        qsort(all, (size_t)m, sizeof(ISC), cmp_isc);
        for (int32_t r = 0; r < R; ++r) {
            out_ids[q * R + r] = r < m ? all[r].id : -1;
            out_scores[q * R + r] = r < m ? all[r].score : INT32_MIN;
        }
        free(all);
    }
}

/* Per-block lookup table of q . center in float64:
 * lut[q][b][c] = sum_t q[b*dpb + t] * cb[b][c][t]. */
void oracle_lut_f64(const float* qv, int64_t nq, int32_t d, const float* cb, int32_t B,
                    int32_t dpb, double* out) {
    (void)d;
    #pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nq; ++q)
        for (int32_t b = 0; b < B; ++b)
            for (int32_t c = 0; c < 16; ++c) {
                double s = 0.0;
                for (int32_t t = 0; t < dpb; ++t)
                    s += (double)qv[q * d + b * dpb + t] * (double)cb[((int64_t)b * 16 + c) * dpb + t];
                out[(q * B + b) * 16 + c] = s;
            }
}

/* int8 quantisation of a given float32 table, all arithmetic in float32 in the
 * order stated in the header comment. */
void oracle_quantize_lut(const float* lut, int64_t nq, int32_t B, int8_t* out, float* scale,
                         float* bias) {
    #pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nq; ++q) {
        const float* t = lut + q * (int64_t)B * 16;
        float* mid = (float*)malloc(sizeof(float) * (size_t)(B > 0 ? B : 1));
        float rng = 0.0f;
        for (int32_t b = 0; b < B; ++b) {
            float lo = t[b * 16], hi = t[b * 16];
            for (int32_t c = 1; c < 16; ++c) {
                if (t[b * 16 + c] < lo) lo = t[b * 16 + c];
                if (t[b * 16 + c] > hi) hi = t[b * 16 + c];
            }
            float sum = lo + hi;
            mid[b] = 0.5f * sum;
            float w = hi - lo;
            if (w > rng) rng = w;
        }
        float beta = 0.0f;
        for (int32_t b = 0; b < B; ++b) beta = beta + mid[b];
        int8_t* o = out + q * (int64_t)B * 16;
        if (rng > 0.0f) {
            float inv = 254.0f / rng;
            for (int32_t b = 0; b < B; ++b)
                for (int32_t c = 0; c < 16; ++c) {
                    float diff = t[b * 16 + c] - mid[b];
                    float v = rintf(diff * inv);
                    if (v > 127.0f) v = 127.0f;
                    if (v < -127.0f) v = -127.0f;
                    o[b * 16 + c] = (int8_t)v;
                }
            scale[q] = rng / 254.0f;
        } else {
            memset(o, 0, (size_t)B * 16);
            scale[q] = 0.0f;
        }
        bias[q] = beta;
        free(mid);
    }
}

static inline double load_row_elem(const void* base, int32_t dtype, int64_t idx) {
    if (dtype == 0) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;  /* bf16 -> f32, exact */
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* Step 5: exact float64 dot products of each query with its candidates
 * (id -1 = empty slot, skipped); keep the best k by (score desc, id asc).
 * Missing slots are (-1, -inf). dtype 0 = float32 rows, 1 = bf16 rows. */
void oracle_reorder(const float* qv, int64_t nq, int32_t d, const void* base, int32_t dtype,
                    int64_t n, const int32_t* cand, int32_t R, int32_t k, int32_t* out_ids,
                    double* out_scores) {
    (void)n;
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nq; ++q) {
        DSC* s = (DSC*)malloc(sizeof(DSC) * (size_t)(R > 0 ? R : 1));
        int32_t m = 0;
        for (int32_t r = 0; r < R; ++r) {
            int32_t id = cand[q * R + r];
            if (id < 0) continue;
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j)
                acc += (double)qv[q * d + j] * load_row_elem(base, dtype, (int64_t)id * d + j);
            s[m].score = acc;
            s[m].id = id;
            ++m;
        }
        qsort(s, (size_t)m, sizeof(DSC), cmp_dsc);
        for (int32_t r = 0; r < k; ++r) {
            out_ids[q * k + r] = r < m ? s[r].id : -1;
            out_scores[q * k + r] = r < m ? s[r].score : -INFINITY;
        }
        free(s);
    }
}

/* Step 1: score every centroid in float64 and keep the best nl leaves by
 * (score desc, leaf id asc). */
void oracle_partition(const float* qv, int64_t nq, int32_t d, const float* cent, int32_t L,
                      int32_t nl, int32_t* out_leaves, double* out_scores) {
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nq; ++q) {
        DSC* s = (DSC*)malloc(sizeof(DSC) * (size_t)(L > 0 ? L : 1));
        for (int32_t l = 0; l < L; ++l) {
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j)
                acc += (double)qv[q * d + j] * (double)cent[(int64_t)l * d + j];
            s[l].score = acc;
            s[l].id = l;
        }
        qsort(s, (size_t)L, sizeof(DSC), cmp_dsc);
        for (int32_t r = 0; r < nl; ++r) {
            out_leaves[q * nl + r] = s[r].id;
            out_scores[q * nl + r] = s[r].score;
        }
        free(s);
    }
}

/* Exact ground truth: float64 dot of every query with every row; the best k by
 * (score desc, id asc) are kept in a small list maintained by insertion.
 * dtype as in oracle_reorder. */
static inline int dsc_better(double s, int32_t id, const DSC* o) {
    return s > o->score || (s == o->score && id < o->id);
}
void oracle_brute_force(const float* qv, int64_t nq, int32_t d, const void* base, int32_t dtype,
                        int64_t n, int32_t k, int32_t* out_ids, double* out_scores) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nq; ++q) {
        DSC* best = (DSC*)malloc(sizeof(DSC) * (size_t)(k > 0 ? k : 1));
        int32_t m = 0;
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j)
                acc += (double)qv[q * d + j] * load_row_elem(base, dtype, i * d + j);
            if (m == k && !dsc_better(acc, (int32_t)i, &best[k - 1])) continue;
            int32_t pos = m < k ? m : k - 1;
            while (pos > 0 && dsc_better(acc, (int32_t)i, &best[pos - 1])) {
                best[pos] = best[pos - 1];
                --pos;
            }
            best[pos].score = acc;
            best[pos].id = (int32_t)i;
            if (m < k) ++m;
        }
        for (int32_t r = 0; r < k; ++r) {
            out_ids[q * k + r] = r < m ? best[r].id : -1;
            out_scores[q * k + r] = r < m ? best[r].score : -INFINITY;
        }
        free(best);
    }
}

/* Anisotropic encoding of rows with given per-block codebooks (the next step
 * before the query path: the ScaNN page, sections "The loss in one paragraph"
 * and "Training an anisotropic codebook yourself").  A row x with direction
 * u = x/|x| is scored by the loss (eta-1)*(u.r)^2 + |r|^2 of its residual
 * r = x - decode(code).  The page only says the coupled block choices are
 * refined iteratively; the reading taken here is block-coordinate descent:
 *   - start from the per-block nearest center (squared L2, lowest index on ties);
 *   - a sweep visits b = 0..B-1 and gives block b the center minimising the
 *     loss with every other block fixed (lowest index on ties);
 *   - `sweeps` sweeps.
 * The parallel residual u.r is the sum over blocks of p_b(c) =
 * sum_t (x_t/|x|)(x_t - c_t); the sweep keeps the running total s and, for
 * block b, the total without it, s - p_b(code_b).  All arithmetic in float64,
 * in exactly this order (x_t/|x| formed as x_t * (1/|x|); p_b and |r_b|^2
 * accumulated over t in order; the candidate's loss as
 * ((eta-1)*par)*par + |r_b|^2 with par = (s - p_b(code_b)) + p_b(c)); the
 * decision is an argmin of these float64 values.  Rows: float32 (dtype 0) or
 * bfloat16 (dtype 1, widened exactly).  Codes nibble-packed, low nibble = even
 * block, unused bits zero. */
static double oracle_pb(const double* xv, double invn, const float* cen, int32_t dpb) {
    double p = 0.0;
    for (int32_t t = 0; t < dpb; ++t) p += (xv[t] * invn) * (xv[t] - (double)cen[t]);
    return p;
}

/* init: when non-NULL, the sweeps start from these codes ([n][stride], the
 * training loop's current assignment) instead of the per-block nearest centers. */
void oracle_encode(const void* rows, int32_t dtype, int64_t n, int32_t d, const float* cb, int32_t B,
                   int32_t dpb, double eta, int32_t sweeps, uint8_t* codes, int32_t stride,
                   const uint8_t* init) {
    #pragma omp parallel
    {
        double* xv = (double*)malloc(sizeof(double) * (size_t)d);
        uint8_t* code = (uint8_t*)malloc((size_t)B);
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double ss = 0.0;
            for (int32_t j = 0; j < d; ++j) {
                xv[j] = load_row_elem(rows, dtype, i * d + j);
                ss += xv[j] * xv[j];
            }
            const double invn = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
            for (int32_t b = 0; b < B; ++b) {
                if (init) {
                    code[b] = (init[i * (int64_t)stride + (b >> 1)] >> (4 * (b & 1))) & 15;
                    continue;
                }
                double best = INFINITY;
                int bc = 0;
                for (int c = 0; c < 16; ++c) {
                    const float* cen = cb + ((int64_t)b * 16 + c) * dpb;
                    double nr = 0.0;
                    for (int32_t t = 0; t < dpb; ++t) {
                        const double r = xv[b * dpb + t] - (double)cen[t];
                        nr += r * r;
                    }
                    if (nr < best) { best = nr; bc = c; }
                }
                code[b] = (uint8_t)bc;
            }
            for (int32_t sw = 0; sw < sweeps; ++sw) {
                double s = 0.0;
                for (int32_t b = 0; b < B; ++b)
                    s += oracle_pb(xv + b * dpb, invn, cb + ((int64_t)b * 16 + code[b]) * dpb, dpb);
                for (int32_t b = 0; b < B; ++b) {
                    const double sm = s - oracle_pb(xv + b * dpb, invn, cb + ((int64_t)b * 16 + code[b]) * dpb, dpb);
                    double best = INFINITY, bp = 0.0;
                    int bc = 0;
                    for (int c = 0; c < 16; ++c) {
                        const float* cen = cb + ((int64_t)b * 16 + c) * dpb;
                        const double p = oracle_pb(xv + b * dpb, invn, cen, dpb);
                        double nr = 0.0;
                        for (int32_t t = 0; t < dpb; ++t) {
                            const double r = xv[b * dpb + t] - (double)cen[t];
                            nr += r * r;
                        }
                        const double par = sm + p;
                        const double L = ((eta - 1.0) * par) * par + nr;
                        if (L < best) { best = L; bc = c; bp = p; }
                    }
                    code[b] = (uint8_t)bc;
                    s = sm + bp;
                }
            }
            uint8_t* row = codes + i * (int64_t)stride;
            memset(row, 0, (size_t)stride);
            for (int32_t b = 0; b < B; ++b) row[b >> 1] |= (uint8_t)(code[b] << (4 * (b & 1)));
        }
        free(xv);
        free(code);
    }
}

/* Nearest centroid of each row (the assignment step of the partitioning; the
 * ScaNN page, "Three stages of a search": rows are grouped under centroids):
 * argmin_l |x - c_l|^2 in float64, summed over t in order, lowest l on ties. */
void oracle_nearest(const float* x, int64_t n, int32_t d, const float* cent, int32_t L, int32_t* out,
                    double* dist2) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double best = INFINITY;
        int32_t bl = 0;
        for (int32_t l = 0; l < L; ++l) {
            double s = 0.0;
            for (int32_t t = 0; t < d; ++t) {
                const double r = (double)x[i * d + t] - (double)cent[(int64_t)l * d + t];
                s += r * r;
            }
            if (s < best) { best = s; bl = l; }
        }
        out[i] = bl;
        if (dist2) dist2[i] = best;
    }
}

/* The center update of anisotropic codebook training (the ScaNN page,
 * "Training an anisotropic codebook yourself": a closed-form per-center solve;
 * with the block coupling, block by block in order, each with the other
 * blocks' current centers): for block b and center c over the rows coded c,
 *   sum_i [(eta-1) u_ib u_ib^T + I] c = sum_i [x_ib + (eta-1)(s_i - p_ib + u_ib.x_ib) u_ib]
 * with u = x/|x|, p_ib = u_ib.(x_ib - center) and s_i = sum_b p_ib at the
 * current centers; the solve is Gaussian elimination with partial pivoting in
 * float64; a center with no rows, or a singular system, keeps its value; after
 * block b, its p_ib and s_i are refreshed with the new centers.  Float32 rows;
 * codes [n][stride] nibble-packed; cb [B][16][dpb] updated in place. */
void oracle_pq_update(const float* X, int64_t n, int32_t d, const uint8_t* codes, int32_t stride, int32_t B,
                      int32_t dpb, double eta, float* cb) {
    double* invn = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)B);
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        double ss = 0.0;
        for (int32_t j = 0; j < d; ++j) ss += (double)X[i * d + j] * (double)X[i * d + j];
        invn[i] = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
        s[i] = 0.0;
        for (int32_t b = 0; b < B; ++b) {
            const int c = (codes[i * (int64_t)stride + (b >> 1)] >> (4 * (b & 1))) & 15;
            double pr = 0.0;
            for (int32_t t = 0; t < dpb; ++t) {
                const double x = X[i * d + b * dpb + t];
                pr += (x * invn[i]) * (x - (double)cb[((int64_t)b * 16 + c) * dpb + t]);
            }
            p[i * B + b] = pr;
            s[i] += pr;
        }
    }
    double A[16 * 16], r[16];
    for (int32_t b = 0; b < B; ++b) {
        for (int c = 0; c < 16; ++c) {
            for (int e = 0; e < dpb * dpb; ++e) A[e] = 0.0;
            for (int e = 0; e < dpb; ++e) r[e] = 0.0;
            int64_t cnt = 0;
            for (int64_t i = 0; i < n; ++i) {
                if (((codes[i * (int64_t)stride + (b >> 1)] >> (4 * (b & 1))) & 15) != c) continue;
                ++cnt;
                double u[16], ux = 0.0;
                for (int32_t t = 0; t < dpb; ++t) {
                    u[t] = (double)X[i * d + b * dpb + t] * invn[i];
                    ux += u[t] * (double)X[i * d + b * dpb + t];
                }
                const double w = (eta - 1.0) * (s[i] - p[i * B + b] + ux);
                for (int32_t a = 0; a < dpb; ++a) {
                    for (int32_t t = 0; t < dpb; ++t) A[a * dpb + t] += (eta - 1.0) * u[a] * u[t];
                    A[a * dpb + a] += 1.0;
                    r[a] += (double)X[i * d + b * dpb + a] + w * u[a];
                }
            }
            if (cnt == 0) continue;
            /* Gaussian elimination with partial pivoting */
            int ok = 1;
            for (int32_t k = 0; k < dpb && ok; ++k) {
                int32_t piv = k;
                for (int32_t a = k + 1; a < dpb; ++a)
                    if (fabs(A[a * dpb + k]) > fabs(A[piv * dpb + k])) piv = a;
                if (A[piv * dpb + k] == 0.0) { ok = 0; break; }
                if (piv != k) {
                    for (int32_t t = 0; t < dpb; ++t) { double tmp = A[k * dpb + t]; A[k * dpb + t] = A[piv * dpb + t]; A[piv * dpb + t] = tmp; }
                    double tmp = r[k]; r[k] = r[piv]; r[piv] = tmp;
                }
                for (int32_t a = k + 1; a < dpb; ++a) {
                    const double f = A[a * dpb + k] / A[k * dpb + k];
                    for (int32_t t = k; t < dpb; ++t) A[a * dpb + t] -= f * A[k * dpb + t];
                    r[a] -= f * r[k];
                }
            }
            if (!ok) continue;
            for (int32_t k = dpb - 1; k >= 0; --k) {
                double v = r[k];
                for (int32_t t = k + 1; t < dpb; ++t) v -= A[k * dpb + t] * r[t];
                r[k] = v / A[k * dpb + k];
            }
            for (int32_t t = 0; t < dpb; ++t) cb[((int64_t)b * 16 + c) * dpb + t] = (float)r[t];
        }
        for (int64_t i = 0; i < n; ++i) {
            const int c = (codes[i * (int64_t)stride + (b >> 1)] >> (4 * (b & 1))) & 15;
            double pr = 0.0;
            for (int32_t t = 0; t < dpb; ++t) {
                const double x = X[i * d + b * dpb + t];
                pr += (x * invn[i]) * (x - (double)cb[((int64_t)b * 16 + c) * dpb + t]);
            }
            s[i] += pr - p[i * B + b];
            p[i * B + b] = pr;
        }
    }
    free(invn);
    free(p);
    free(s);
}

/* The update step of the partitioning's k-means (the ScaNN page's partition
 * groups rows under centroids; a centroid is the mean of its rows, the
 * textbook Lloyd step the anisotropic trainer reduces to at eta = 1): per leaf,
 * the float64 sum of its rows in row order divided by their count, rounded to
 * float32; a leaf with no rows keeps its previous centroid.  counts may be NULL. */
void oracle_kmeans_update(const float* x, int64_t n, int32_t d, const int32_t* leaf, int32_t L,
                          float* cent, int32_t* counts) {
    double* sum = (double*)calloc((size_t)L * (size_t)d, sizeof(double));
    int64_t* cnt = (int64_t*)calloc((size_t)L, sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) {
        const int32_t l = leaf[i];
        cnt[l] += 1;
        for (int32_t t = 0; t < d; ++t) sum[(int64_t)l * d + t] += (double)x[i * d + t];
    }
    for (int32_t l = 0; l < L; ++l) {
        if (counts) counts[l] = (int32_t)cnt[l];
        if (cnt[l] == 0) continue;
        for (int32_t t = 0; t < d; ++t) cent[(int64_t)l * d + t] = (float)(sum[(int64_t)l * d + t] / (double)cnt[l]);
    }
    free(sum);
    free(cnt);
}

/* ----------------------------------------------------------------------------
 * Int8 scalar-quantised flat search (the page "Incoherence-Aware Asymmetric
 * Quantization for Retrieval", sections "A Specialized int8 Retrieval Engine"
 * and the robust int8 scale): every vector gets its own step
 * s = max(P, 1e-8) / 127 with P the pct-th percentile of its absolute values,
 * codes clip(round(x / s), -127, 127) (round half to even), and a query/document
 * pair scores (float)(q8 . d8) * s_q * s_d with the integer dot exact.
 * Readings: P by linear interpolation between order statistics (position
 * pct/100 * (d-1); fraction t; a + (b-a)*t when t < 0.5, else b - (b-a)*(1-t),
 * with b-a in float32 and the rest in float64, as numpy's linear percentile); s in float32 (the float32 P, then / 127);
 * x / s in float32; the score's multiplications left to right in float32;
 * ranking by (score desc, document id asc). */
static int cmp_f32(const void* a, const void* b) {
    const float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

void oracle_sq8_quantize(const float* x, int64_t n, int32_t d, double pct, int8_t* codes, float* scale) {
    #pragma omp parallel
    {
        float* a = (float*)malloc(sizeof(float) * (size_t)(d > 0 ? d : 1));
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            for (int32_t t = 0; t < d; ++t) a[t] = fabsf(x[i * d + t]);
            qsort(a, (size_t)d, sizeof(float), cmp_f32);
            const float pos = (float)(d - 1) * (float)(pct / 100.0);
            int64_t lo = (int64_t)floorf(pos);
            if (lo > d - 1) lo = d - 1;
            const int64_t hi = lo + 1 < d ? lo + 1 : d - 1;
            const float t = pos - (float)lo;
            const float diff = a[hi] - a[lo];
            const float P = t < 0.5f ? a[lo] + diff * t : a[hi] - diff * (1.0f - t);
            const float s = (P > 1e-8f ? P : 1e-8f) / 127.0f;
            scale[i] = s;
            for (int32_t k = 0; k < d; ++k) {
                float v = rintf(x[i * d + k] / s);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                codes[i * d + k] = (int8_t)v;
            }
        }
        free(a);
    }
}

typedef struct { float score; int32_t id; } FSC;
static int cmp_fsc(const void* a, const void* b) {
    const FSC* x = (const FSC*)a; const FSC* y = (const FSC*)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    return (x->id > y->id) - (x->id < y->id);
}

void oracle_sq8_topk(const int8_t* q8, const float* qs, int64_t nq, const int8_t* d8, const float* ds, int64_t n,
                     int32_t d, int32_t R, int32_t* out_ids, float* out_scores) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nq; ++q) {
        FSC* all = (FSC*)malloc(sizeof(FSC) * (size_t)(n > 0 ? n : 1));
        for (int64_t j = 0; j < n; ++j) {
            int64_t dot = 0;
            for (int32_t t = 0; t < d; ++t) dot += (int64_t)q8[q * d + t] * (int64_t)d8[j * d + t];
            const float f = (float)(int32_t)dot;
            all[j].score = (f * qs[q]) * ds[j];
            all[j].id = (int32_t)j;
        }
        qsort(all, (size_t)n, sizeof(FSC), cmp_fsc);
        for (int32_t r = 0; r < R; ++r) {
            out_ids[q * R + r] = r < n ? all[r].id : -1;
            out_scores[q * R + r] = r < n ? all[r].score : -INFINITY;
        }
        free(all);
    }
}
