/*
 * tt_oracle.c -- plain, slow, obviously-correct CPU oracle for TT-EmbeddingBag.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no source, header, table or helper with the HIP path.
 *
 * What it computes (all arithmetic in IEEE double, inputs are the fp32 values):
 *
 *  - The implicit table.  "FBTT-Embedding" README, section "Initialization": core k
 *    has shape  ranks[k-1] x p[k] x q[k] x ranks[k]  with ranks = [1] + tt_ranks + [1];
 *    prod(p) >= num_embeddings, prod(q) == embedding_dim ("Parameters").  The row
 *    index i is split over p and the column index j over q.  The pages do not fix
 *    the order of the split; this oracle takes row-major mixed radix for both
 *    (i = (i1*p2 + i2)*p3 + i3, j = (j1*q2 + j2)*q3 + j3).  Then
 *        W[i][j] = sum_{r1,r2} G1[0][i1][j1][r1] * G2[r1][i2][j2][r2] * G3[r2][i3][j3][0]
 *    written out literally below as a double loop over (r1, r2) for every j.
 *    Cores are passed in the pages' logical layout [R_{k-1}][p_k][q_k][R_k].
 *
 *  - EmbeddingBag pooling.  README intro: same forward/backward as PyTorch's
 *    EmbeddingBag except that the table is compressed; "EmbeddingBag and
 *    Product-Key Memory Layers" (tensorflow/addons #2201), first post: a gather
 *    followed by a (weighted) sum.  Bag b covers positions [off[b], off[b+1]);
 *    the offsets array carries the terminal entry off[nbags] = nnz.  Sum pooling,
 *    optional per-sample weights, an empty bag gives a zero row.
 *
 *  - Mean pooling (PyTorch EmbeddingBag's mode "mean", named as a variant in the survey
 *    of the pages): the bag's (weighted) sum divided by its number of elements; an
 *    empty bag gives a zero row.
 *
 *  - TableBatched layout ("TableBatchedTTEmbeddingBag" section: T tables of one
 *    shape).  Bags are numbered table-major, bag b belongs to table b / B.
 *
 *  - Software cache ("Software Cache" section): an element whose slot >= 0 reads
 *    the decompressed row cache[slot] instead of the TT row, and its gradient goes
 *    to that cache row, not to the cores.
 *
 *  - Backward.  With L = sum_b <dY[b], Y[b]>, the product rule on the definition
 *    of W gives, for each element n with g = w_n * dY[bag(n)]:
 *        dG1[0][i1][j1][r1]  += g[j] * G2[r1][i2][j2][r2] * G3[r2][i3][j3][0]
 *        dG2[r1][i2][j2][r2] += g[j] * G1[0][i1][j1][r1] * G3[r2][i3][j3][0]
 *        dG3[r2][i3][j3][0]  += g[j] * G1[0][i1][j1][r1] * G2[r1][i2][j2][r2]
 *    summed over j, r1, r2 -- again a literal loop.  Duplicated indices add up.
 *    No gradient with respect to the per-sample weights is formed.
 *
 *  - Fused SGD ("Parameters" entry for `sparse`, "Fused Kernel" section): the
 *    weights are updated in the backward pass instead of returning gradients.
 *    Reading taken: identical to one plain SGD step G <- G - lr * dG at the
 *    pre-update cores; slices that received no contribution are left untouched.
 *    Without the fused update (`sparse` False) the gradients above are the result.
 *
 *  - Fused Adagrad ("Parameters": `optimizer`, `eps` for Adagrad only): the
 *    diagonal Adagrad step of Duchi, Hazan and Singer (2011) on the touched slices,
 *    one running sum of squared gradients per parameter, eps added to its root.
 *
 * Error behaviour: returns 0 on success, -1 if an index is outside [0, E), an
 * offsets array is not a valid CSR over [0, nnz], or a cache slot is outside
 * [0, cache_size).  Nothing is written on error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t num_tables;      /* T >= 1 */
    int64_t num_embeddings;  /* E */
    int32_t p[3];
    int32_t q[3];
    int32_t r[2];            /* tt_ranks; full ranks are {1, r[0], r[1], 1} */
    int32_t pooling;         /* 0: sum, 1: mean (sum divided by the bag's length) */
} oracle_shape;

static int64_t prod3(const int32_t *v) { return (int64_t)v[0] * v[1] * v[2]; }

/* number of floats in core k of one table */
int64_t oracle_core_numel(const oracle_shape *s, int k)
{
    const int64_t rk0 = (k == 0) ? 1 : s->r[k - 1];
    const int64_t rk1 = (k == 2) ? 1 : s->r[k];
    return rk0 * s->p[k] * s->q[k] * rk1;
}

/* element of core k in the pages' logical layout [R_{k-1}][p_k][q_k][R_k] */
static double core_at(const oracle_shape *s, const float *G, int k,
                      int64_t ra, int64_t ik, int64_t jk, int64_t rb)
{
    const int64_t rk1 = (k == 2) ? 1 : s->r[k];
    const int64_t pk = s->p[k], qk = s->q[k];
    return (double)G[((ra * pk + ik) * qk + jk) * rk1 + rb];
}

static int64_t core_index(const oracle_shape *s, int k,
                          int64_t ra, int64_t ik, int64_t jk, int64_t rb)
{
    const int64_t rk1 = (k == 2) ? 1 : s->r[k];
    return ((ra * s->p[k] + ik) * s->q[k] + jk) * rk1 + rb;
}

/* row-major mixed-radix split of i over p */
void oracle_split_index(const int32_t p[3], int64_t i, int64_t out[3])
{
    out[2] = i % p[2];
    out[1] = (i / p[2]) % p[1];
    out[0] = i / ((int64_t)p[1] * p[2]);
}

/* W[i][:] of one table, straight from the definition */
void oracle_tt_row(const oracle_shape *s, const float *G1, const float *G2,
                   const float *G3, int64_t i, double *row)
{
    int64_t ii[3];
    oracle_split_index(s->p, i, ii);
    const int32_t *q = s->q;
    for (int64_t j1 = 0; j1 < q[0]; ++j1)
        for (int64_t j2 = 0; j2 < q[1]; ++j2)
            for (int64_t j3 = 0; j3 < q[2]; ++j3) {
                double acc = 0.0;
                for (int64_t r1 = 0; r1 < s->r[0]; ++r1)
                    for (int64_t r2 = 0; r2 < s->r[1]; ++r2)
                        acc += core_at(s, G1, 0, 0, ii[0], j1, r1)
                             * core_at(s, G2, 1, r1, ii[1], j2, r2)
                             * core_at(s, G3, 2, r2, ii[2], j3, 0);
                row[(j1 * q[1] + j2) * q[2] + j3] = acc;
            }
}

static int check_inputs(const oracle_shape *s, const int64_t *idx, int64_t nnz,
                        const int64_t *off, int64_t nbags_total,
                        const int32_t *slot, int64_t cache_size)
{
    if (off[0] != 0 || off[nbags_total] != nnz) return -1;
    for (int64_t b = 0; b < nbags_total; ++b)
        if (off[b + 1] < off[b]) return -1;
    for (int64_t n = 0; n < nnz; ++n) {
        if (slot && slot[n] >= 0) {
            if (slot[n] >= cache_size) return -1;
            continue;
        }
        if (idx[n] < 0 || idx[n] >= s->num_embeddings) return -1;
    }
    if (prod3(s->p) < s->num_embeddings) return -1;
    return 0;
}

/*
 * Forward.  cores: 3*T pointers, table t's cores at cores[3t+0..2] in the
 * logical layout.  off has T*B+1 entries.  psw may be NULL (all weights 1).
 * slot may be NULL (no cache); otherwise slot[n] >= 0 selects cache row slot[n]
 * of `cache` ([cache_size][D]).  Y is [T*B][D] doubles, fully overwritten.
 */
int oracle_forward(const oracle_shape *s, const float *const *cores,
                   const int64_t *idx, int64_t nnz, const int64_t *off, int64_t B,
                   const float *psw, const int32_t *slot, const float *cache,
                   int64_t cache_size, double *Y)
{
    const int64_t T = s->num_tables, D = prod3(s->q), NB = T * B;
    if (check_inputs(s, idx, nnz, off, NB, slot, cache_size)) return -1;
    double *row = (double *)malloc(sizeof(double) * D);
    memset(Y, 0, sizeof(double) * NB * D);
    for (int64_t b = 0; b < NB; ++b) {
        const int64_t t = b / B;
        for (int64_t n = off[b]; n < off[b + 1]; ++n) {
            const double w = psw ? (double)psw[n] : 1.0;
            if (slot && slot[n] >= 0) {
                for (int64_t j = 0; j < D; ++j) row[j] = (double)cache[slot[n] * D + j];
            } else {
                oracle_tt_row(s, cores[3 * t], cores[3 * t + 1], cores[3 * t + 2], idx[n], row);
            }
            for (int64_t j = 0; j < D; ++j) Y[b * D + j] += w * row[j];
        }
        if (s->pooling == 1 && off[b + 1] > off[b])
            for (int64_t j = 0; j < D; ++j) Y[b * D + j] /= (double)(off[b + 1] - off[b]);
    }
    free(row);
    return 0;
}

/*
 * Backward.  dY is [T*B][D] fp32.  grad_w (may be NULL) receives dL/dw_n for every
 * element, the gradient with respect to its per-sample weight: <dY[bag], row_n>, times
 * 1/len with mean pooling (row_n from cache_rows for a hit).  grad[3t+k] are double buffers in the logical
 * layout of core k of table t, fully overwritten.  touched[3t+k] (may be NULL)
 * are byte arrays of length p_k set to 1 for every slice i_k that received a
 * contribution.  grad_cache ([cache_size][D], may be NULL when slot is NULL) and
 * touched_cache ([cache_size]) collect the cache-row gradients.
 */
int oracle_backward(const oracle_shape *s, const float *const *cores,
                    const int64_t *idx, int64_t nnz, const int64_t *off, int64_t B,
                    const float *psw, const int32_t *slot, int64_t cache_size,
                    const float *dY, double *const *grad, uint8_t *const *touched,
                    double *grad_cache, uint8_t *touched_cache, double *grad_w,
                    const float *cache_rows)
{
    const int64_t T = s->num_tables, D = prod3(s->q), NB = T * B;
    if (check_inputs(s, idx, nnz, off, NB, slot, cache_size)) return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < 3; ++k) {
            memset(grad[3 * t + k], 0, sizeof(double) * oracle_core_numel(s, k));
            if (touched) memset(touched[3 * t + k], 0, (size_t)s->p[k]);
        }
    if (grad_cache) memset(grad_cache, 0, sizeof(double) * cache_size * D);
    if (touched_cache) memset(touched_cache, 0, (size_t)cache_size);
    const int32_t *q = s->q;
    const int64_t R1 = s->r[0], R2 = s->r[1];
    for (int64_t b = 0; b < NB; ++b) {
        const int64_t t = b / B;
        const float *G1 = cores[3 * t], *G2 = cores[3 * t + 1], *G3 = cores[3 * t + 2];
        double *d1 = grad[3 * t], *d2 = grad[3 * t + 1], *d3 = grad[3 * t + 2];
        /* mean pooling: out[b] = (sum) / len, so each element's gradient carries 1 / len */
        const double inv = (s->pooling == 1) ? 1.0 / (double)(off[b + 1] - off[b]) : 1.0;
        for (int64_t n = off[b]; n < off[b + 1]; ++n) {
            const double w = (psw ? (double)psw[n] : 1.0) * inv;
            if (slot && slot[n] >= 0) {
                for (int64_t j = 0; j < D; ++j)
                    grad_cache[slot[n] * D + j] += w * (double)dY[b * D + j];
                if (touched_cache) touched_cache[slot[n]] = 1;
                if (grad_w) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < D; ++j)
                        acc += (double)dY[b * D + j] * (double)cache_rows[slot[n] * D + j];
                    grad_w[n] = acc * inv;
                }
                continue;
            }
            int64_t ii[3];
            oracle_split_index(s->p, idx[n], ii);
            if (grad_w) {
                /* dL/dw_n = <dY[b], W[idx_n]> (times 1/len with mean pooling) */
                double *row = (double *)malloc(sizeof(double) * D);
                oracle_tt_row(s, G1, G2, G3, idx[n], row);
                double acc = 0.0;
                for (int64_t j = 0; j < D; ++j) acc += (double)dY[b * D + j] * row[j];
                grad_w[n] = acc * inv;
                free(row);
            }
            if (touched)
                for (int k = 0; k < 3; ++k) touched[3 * t + k][ii[k]] = 1;
            for (int64_t j1 = 0; j1 < q[0]; ++j1)
                for (int64_t j2 = 0; j2 < q[1]; ++j2)
                    for (int64_t j3 = 0; j3 < q[2]; ++j3) {
                        const double g = w * (double)dY[b * D + (j1 * q[1] + j2) * q[2] + j3];
                        for (int64_t r1 = 0; r1 < R1; ++r1)
                            for (int64_t r2 = 0; r2 < R2; ++r2) {
                                const double a = core_at(s, G1, 0, 0, ii[0], j1, r1);
                                const double m = core_at(s, G2, 1, r1, ii[1], j2, r2);
                                const double c = core_at(s, G3, 2, r2, ii[2], j3, 0);
                                d1[core_index(s, 0, 0, ii[0], j1, r1)] += g * m * c;
                                d2[core_index(s, 1, r1, ii[1], j2, r2)] += g * a * c;
                                d3[core_index(s, 2, r2, ii[2], j3, 0)] += g * a * m;
                            }
                    }
        }
    }
    return 0;
}

/*
 * Plain SGD on the slices of one core that received a contribution:
 * G <- fp32( double(G) - lr * dG ).  Untouched slices keep their bits.
 * `core` and `grad` are in the logical layout of core k of one table.
 */
void oracle_sgd_core(const oracle_shape *s, int k, float *core, const double *grad,
                     const uint8_t *touched, double lr)
{
    const int64_t ra = (k == 0) ? 1 : s->r[k - 1];
    const int64_t rb = (k == 2) ? 1 : s->r[k];
    for (int64_t a = 0; a < ra; ++a)
        for (int64_t ik = 0; ik < s->p[k]; ++ik) {
            if (!touched[ik]) continue;
            for (int64_t jk = 0; jk < s->q[k]; ++jk)
                for (int64_t c = 0; c < rb; ++c) {
                    const int64_t e = core_index(s, k, a, ik, jk, c);
                    core[e] = (float)((double)core[e] - lr * grad[e]);
                }
        }
}

/* the same step for cache rows: rows[s] <- fp32(rows[s] - lr * grad[s]) for touched s */
void oracle_sgd_rows(float *rows, const double *grad, const uint8_t *touched,
                     int64_t nrows, int64_t D, double lr)
{
    for (int64_t sl = 0; sl < nrows; ++sl) {
        if (!touched[sl]) continue;
        for (int64_t j = 0; j < D; ++j)
            rows[sl * D + j] = (float)((double)rows[sl * D + j] - lr * grad[sl * D + j]);
    }
}

/*
 * Adagrad, the other optimizer of the fused update ("Parameters": `optimizer`, and
 * `eps` added to the denominator): the diagonal method of Duchi, Hazan and Singer
 * (2011).  Each parameter x keeps a running sum S of its squared gradients:
 *     S <- fp32( double(S) + g^2 );   x <- fp32( double(x) - lr * g / (sqrt(S) + eps) )
 * with the S just stored.  `state` has the layout of `core`; untouched slices keep
 * the bits of both.
 */
void oracle_adagrad_core(const oracle_shape *s, int k, float *core, float *state,
                         const double *grad, const uint8_t *touched, double lr, double eps)
{
    const int64_t ra = (k == 0) ? 1 : s->r[k - 1];
    const int64_t rb = (k == 2) ? 1 : s->r[k];
    for (int64_t a = 0; a < ra; ++a)
        for (int64_t ik = 0; ik < s->p[k]; ++ik) {
            if (!touched[ik]) continue;
            for (int64_t jk = 0; jk < s->q[k]; ++jk)
                for (int64_t c = 0; c < rb; ++c) {
                    const int64_t e = core_index(s, k, a, ik, jk, c);
                    const double g = grad[e];
                    state[e] = (float)((double)state[e] + g * g);
                    core[e] = (float)((double)core[e] - lr * g / (sqrt((double)state[e]) + eps));
                }
        }
}

/* the same step for cache rows, state [nrows][D] */
void oracle_adagrad_rows(float *rows, float *state, const double *grad, const uint8_t *touched,
                         int64_t nrows, int64_t D, double lr, double eps)
{
    for (int64_t sl = 0; sl < nrows; ++sl) {
        if (!touched[sl]) continue;
        for (int64_t j = 0; j < D; ++j) {
            const int64_t e = sl * D + j;
            const double g = grad[e];
            state[e] = (float)((double)state[e] + g * g);
            rows[e] = (float)((double)rows[e] - lr * g / (sqrt((double)state[e]) + eps));
        }
    }
}

/* ------------------------------------------------------------------------------------
 * General number of cores d ("FBTT-Embedding" README, "Parameters": tt_p_shapes,
 * tt_q_shapes and tt_ranks are lists of one length d, ranks padded to {1, ..., 1}).
 * Core k (k = 0 .. d-1) has shape R(k) x p_k x q_k x R(k+1) in the logical layout,
 * with R(0) = R(d) = 1 and R(k) = r[k-1] otherwise.  The row index i and the column
 * index j are split over p and q row-major, as above, and W[i][j] is the product of
 * the d slice matrices G_k[:, i_k, j_k, :] (a 1 x 1 result), evaluated left to right.
 * The gradient of core k at (a, i_k, j_k, b) is g[j] times the product of the slices
 * before k (entry a of that row vector) times the product of the slices after k
 * (entry b of that column vector).
 * ------------------------------------------------------------------------------------ */
#define ORACLE_MAX_D 8

typedef struct {
    int32_t num_tables;      /* T >= 1 */
    int32_t d;               /* 1 <= d <= ORACLE_MAX_D */
    int64_t num_embeddings;  /* E */
    int32_t p[ORACLE_MAX_D];
    int32_t q[ORACLE_MAX_D];
    int32_t r[ORACLE_MAX_D - 1];
    int32_t pooling;         /* 0: sum, 1: mean */
} oracle_shape_d;

static int64_t rank_d(const oracle_shape_d *s, int k)
{
    return (k == 0 || k == s->d) ? 1 : s->r[k - 1];
}

int64_t oracle_core_numel_d(const oracle_shape_d *s, int k)
{
    return rank_d(s, k) * s->p[k] * s->q[k] * rank_d(s, k + 1);
}

static int64_t core_index_d(const oracle_shape_d *s, int k, int64_t a, int64_t ik, int64_t jk,
                            int64_t b)
{
    return ((a * s->p[k] + ik) * s->q[k] + jk) * rank_d(s, k + 1) + b;
}

/* row-major mixed-radix split of v over the d extents e */
static void split_d(const int32_t *e, int d, int64_t v, int64_t *out)
{
    for (int k = d - 1; k >= 0; --k) {
        out[k] = v % e[k];
        v /= e[k];
    }
}

static int check_inputs_d(const oracle_shape_d *s, const int64_t *idx, int64_t nnz,
                          const int64_t *off, int64_t nbags_total)
{
    if (s->d < 1 || s->d > ORACLE_MAX_D) return -1;
    double prodp = 1.0;
    for (int k = 0; k < s->d; ++k) prodp *= s->p[k];
    if (prodp < (double)s->num_embeddings) return -1;
    if (off[0] != 0 || off[nbags_total] != nnz) return -1;
    for (int64_t b = 0; b < nbags_total; ++b)
        if (off[b + 1] < off[b]) return -1;
    for (int64_t n = 0; n < nnz; ++n)
        if (idx[n] < 0 || idx[n] >= s->num_embeddings) return -1;
    return 0;
}

static int64_t dim_d(const oracle_shape_d *s)
{
    int64_t D = 1;
    for (int k = 0; k < s->d; ++k) D *= s->q[k];
    return D;
}

static int64_t max_rank_d(const oracle_shape_d *s)
{
    int64_t m = 1;
    for (int k = 1; k < s->d; ++k)
        if (rank_d(s, k) > m) m = rank_d(s, k);
    return m;
}

/* prefix vectors L[k] (length R(k)) of one (i, j): L[0] = 1, L[k+1] = L[k] * G_k slice */
static void prefix_d(const oracle_shape_d *s, const float *const *G, const int64_t *ii,
                     const int64_t *jj, int64_t M, double *L)
{
    L[0] = 1.0;
    for (int k = 0; k < s->d; ++k) {
        const int64_t ra = rank_d(s, k), rb = rank_d(s, k + 1);
        for (int64_t b = 0; b < rb; ++b) {
            double acc = 0.0;
            for (int64_t a = 0; a < ra; ++a)
                acc += L[k * M + a] * (double)G[k][core_index_d(s, k, a, ii[k], jj[k], b)];
            L[(k + 1) * M + b] = acc;
        }
    }
}

/* suffix vectors S[k] (length R(k)): S[d] = 1, S[k] = G_k slice * S[k+1] */
static void suffix_d(const oracle_shape_d *s, const float *const *G, const int64_t *ii,
                     const int64_t *jj, int64_t M, double *S)
{
    S[s->d * M] = 1.0;
    for (int k = s->d - 1; k >= 0; --k) {
        const int64_t ra = rank_d(s, k), rb = rank_d(s, k + 1);
        for (int64_t a = 0; a < ra; ++a) {
            double acc = 0.0;
            for (int64_t b = 0; b < rb; ++b)
                acc += (double)G[k][core_index_d(s, k, a, ii[k], jj[k], b)] * S[(k + 1) * M + b];
            S[k * M + a] = acc;
        }
    }
}

/* W[i][:] of one table (G: its d cores) */
void oracle_tt_row_d(const oracle_shape_d *s, const float *const *G, int64_t i, double *row)
{
    const int64_t D = dim_d(s), M = max_rank_d(s);
    int64_t ii[ORACLE_MAX_D], jj[ORACLE_MAX_D];
    double *L = (double *)malloc(sizeof(double) * (s->d + 1) * M);
    split_d(s->p, s->d, i, ii);
    for (int64_t j = 0; j < D; ++j) {
        split_d(s->q, s->d, j, jj);
        prefix_d(s, G, ii, jj, M, L);
        row[j] = L[s->d * M];
    }
    free(L);
}

/* Forward over d-core tables: cores holds d*T pointers, table t's at [d*t .. d*t+d). */
int oracle_forward_d(const oracle_shape_d *s, const float *const *cores, const int64_t *idx,
                     int64_t nnz, const int64_t *off, int64_t B, const float *psw, double *Y)
{
    const int64_t T = s->num_tables, NB = T * B;
    if (check_inputs_d(s, idx, nnz, off, NB)) return -1;
    const int64_t D = dim_d(s);
    double *row = (double *)malloc(sizeof(double) * D);
    memset(Y, 0, sizeof(double) * NB * D);
    for (int64_t b = 0; b < NB; ++b) {
        const int64_t t = b / B;
        for (int64_t n = off[b]; n < off[b + 1]; ++n) {
            const double w = psw ? (double)psw[n] : 1.0;
            oracle_tt_row_d(s, cores + s->d * t, idx[n], row);
            for (int64_t j = 0; j < D; ++j) Y[b * D + j] += w * row[j];
        }
        if (s->pooling == 1 && off[b + 1] > off[b])
            for (int64_t j = 0; j < D; ++j) Y[b * D + j] /= (double)(off[b + 1] - off[b]);
    }
    free(row);
    return 0;
}

/* Backward over d-core tables: grad[d*t + k] (double, logical layout) fully overwritten;
 * touched[d*t + k] (may be NULL) marks the slices that received a contribution. */
int oracle_backward_d(const oracle_shape_d *s, const float *const *cores, const int64_t *idx,
                      int64_t nnz, const int64_t *off, int64_t B, const float *psw,
                      const float *dY, double *const *grad, uint8_t *const *touched)
{
    const int64_t T = s->num_tables, NB = T * B;
    if (check_inputs_d(s, idx, nnz, off, NB)) return -1;
    const int d = s->d;
    const int64_t D = dim_d(s), M = max_rank_d(s);
    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < d; ++k) {
            memset(grad[d * t + k], 0, sizeof(double) * oracle_core_numel_d(s, k));
            if (touched) memset(touched[d * t + k], 0, (size_t)s->p[k]);
        }
    double *L = (double *)malloc(sizeof(double) * (d + 1) * M);
    double *S = (double *)malloc(sizeof(double) * (d + 1) * M);
    int64_t ii[ORACLE_MAX_D], jj[ORACLE_MAX_D];
    for (int64_t b = 0; b < NB; ++b) {
        const int64_t t = b / B;
        const float *const *G = cores + d * t;
        const double inv = (s->pooling == 1) ? 1.0 / (double)(off[b + 1] - off[b]) : 1.0;
        for (int64_t n = off[b]; n < off[b + 1]; ++n) {
            const double w = (psw ? (double)psw[n] : 1.0) * inv;
            split_d(s->p, d, idx[n], ii);
            if (touched)
                for (int k = 0; k < d; ++k) touched[d * t + k][ii[k]] = 1;
            for (int64_t j = 0; j < D; ++j) {
                const double g = w * (double)dY[b * D + j];
                split_d(s->q, d, j, jj);
                prefix_d(s, G, ii, jj, M, L);
                suffix_d(s, G, ii, jj, M, S);
                for (int k = 0; k < d; ++k) {
                    const int64_t ra = rank_d(s, k), rb = rank_d(s, k + 1);
                    for (int64_t a = 0; a < ra; ++a)
                        for (int64_t c = 0; c < rb; ++c)
                            grad[d * t + k][core_index_d(s, k, a, ii[k], jj[k], c)] +=
                                g * L[k * M + a] * S[(k + 1) * M + c];
                }
            }
        }
    }
    free(L);
    free(S);
    return 0;
}
