/*
 * Plain CPU oracle for exact Lloyd k-means.  TEST INFRASTRUCTURE ONLY: it is
 * called by the tests, by the smoke check and by the CPU-baseline leg of the
 * benchmark, never by the library.  It shares no code with the GPU path.
 *
 * What it computes (one Lloyd iteration = assignment stage, then update
 * stage), as described on the pages:
 *   - technologypulse.uk "Flash-KMeans" article, section "math unchanged,
 *     dataflow changed": the assignment stage computes the distance of every
 *     point to every centroid and picks the nearest; the update stage averages
 *     the points of each cluster into its new centroid.  The accelerated
 *     kernels claim a result identical to standard Lloyd, so this file is
 *     standard Lloyd written out with explicit loops.
 *   - daily.steinslab.io "e-means" article, section "Breaking 70 Years of
 *     Full-Batch Inertia": each cluster keeps a sum vector S_j and a count
 *     N_j, the centroid is S_j / N_j, and the accumulators are reset and the
 *     whole dataset is streamed every round.
 *   - github LeanModels/LeanQuant issue #1 "1D k-means", the kmeans_fit diff:
 *     per-point sample weights; the weighted centroid is sum(w x) / sum(w).
 *
 * Readings where the pages are silent:
 *   - distance is the squared Euclidean distance, summed in fp64 as
 *     sum_k (x_k - c_k)^2 with k ascending;
 *   - ties go to the smallest centroid index (j ascending, strict '<');
 *   - a cluster with no points keeps its previous centroid;
 *   - the distances of iteration t use C_t rounded (IEEE round-to-nearest-
 *     even) to the storage type of the points, because that is the operand
 *     the accelerated assignment multiplies; the fp32 centroids are the state;
 *   - the assignment ignores weights; the update and the objective use them;
 *     counts are unweighted integers; "empty" means count 0;
 *   - the objective of iteration t is J_t = sum_i w_i * min_j D_ij.
 *
 * Everything is fp64 except the fp32 centroid state and the conversions,
 * which follow the IEEE 754 binary16 / bfloat16 formats bit by bit.
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ----------------------------------------------------------------------- *
 * IEEE conversions.  A small binary format is (man_bits stored mantissa bits,
 * exponent bias, emin = 1 - bias).  binary16: 10 / 15; bfloat16: 7 / 127.
 * ----------------------------------------------------------------------- */

static void format_of(int dtype, int *man_bits, int *bias, int *exp_bits)
{
    if (dtype == ORC_F16) { *man_bits = 10; *bias = 15; *exp_bits = 5; }
    else                  { *man_bits = 7;  *bias = 127; *exp_bits = 8; }
}

/* Exact value of a stored element, as a double. */
double oracle_decode_one(uint32_t bits, int dtype)
{
    if (dtype == ORC_F32) {
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    int man_bits, bias, exp_bits;
    format_of(dtype, &man_bits, &bias, &exp_bits);
    uint32_t total = 1u + (uint32_t)exp_bits + (uint32_t)man_bits;
    uint32_t sign = (bits >> (total - 1)) & 1u;
    uint32_t e = (bits >> man_bits) & ((1u << exp_bits) - 1u);
    uint32_t m = bits & ((1u << man_bits) - 1u);
    double v;
    if (e == (1u << exp_bits) - 1u)
        v = m ? NAN : INFINITY;
    else if (e == 0) /* zero or subnormal: m * 2^(emin - man_bits) */
        v = ldexp((double)m, (1 - bias) - man_bits);
    else             /* normal: (2^man_bits + m) * 2^(e - bias - man_bits) */
        v = ldexp((double)((1u << man_bits) + m), (int)e - bias - man_bits);
    return sign ? -v : v;
}

/* Round a float32 to the small format with round-to-nearest, ties to even. */
uint32_t oracle_round_one(float f, int dtype)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (dtype == ORC_F32) return u;
    int man_bits, bias, exp_bits;
    format_of(dtype, &man_bits, &bias, &exp_bits);
    uint32_t total = 1u + (uint32_t)exp_bits + (uint32_t)man_bits;
    uint32_t sign = (u >> 31) << (total - 1);
    uint32_t emax_field = (1u << exp_bits) - 1u;
    uint32_t fe = (u >> 23) & 0xffu;
    uint32_t fm = u & 0x7fffffu;
    if (fe == 0xffu) /* inf or nan */
        return sign | (emax_field << man_bits) | (fm ? (1u << (man_bits - 1)) : 0u);
    if (fe == 0 && fm == 0) return sign;
    /* |f| = sig * 2^p2 exactly */
    uint64_t sig = fe ? (fm | 0x800000u) : fm;
    int p2 = fe ? (int)fe - 150 : -149;
    int msb = 63 - __builtin_clzll(sig);
    int E = p2 + msb;                       /* floor(log2 |f|) */
    int emin = 1 - bias;
    int qexp = (E < emin ? emin : E) - man_bits; /* log2 of the quantum at |f| */
    int sh = qexp - p2;                     /* |f| / quantum = sig / 2^sh */
    uint64_t n;
    if (sh <= 0) {
        n = sig << (-sh);
    } else if (sh > 62) {
        n = 0;                              /* far below half a quantum */
    } else {
        uint64_t q = sig >> sh, r = sig & ((1ull << sh) - 1ull), half = 1ull << (sh - 1);
        if (r > half || (r == half && (q & 1ull))) q += 1ull;
        n = q;
    }
    /* value = n * 2^qexp */
    if (E < emin) {
        /* subnormal range: n <= 2^man_bits; n == 2^man_bits is the smallest normal,
         * whose encoding (exponent field 1, mantissa 0) equals n. */
        return sign | (uint32_t)n;
    }
    int Eo = E;
    if (n == (2ull << man_bits)) { n >>= 1; Eo += 1; } /* rounding carried into the next binade */
    if (Eo + bias >= (int)emax_field)
        return sign | (emax_field << man_bits);        /* overflow to infinity */
    return sign | ((uint32_t)(Eo + bias) << man_bits) | (uint32_t)(n - (1ull << man_bits));
}

/* Element-wise helpers over arrays. `bits` is uint16 for fp16/bf16, uint32 for fp32. */
void oracle_decode(const void *bits, int dtype, int64_t n, double *out)
{
    if (dtype == ORC_F32) {
        const float *p = (const float *)bits;
        for (int64_t i = 0; i < n; ++i) out[i] = (double)p[i];
    } else {
        const uint16_t *p = (const uint16_t *)bits;
        for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode_one(p[i], dtype);
    }
}

void oracle_round(const float *in, int64_t n, int dtype, void *bits_out)
{
    if (dtype == ORC_F32) {
        memcpy(bits_out, in, (size_t)n * 4);
    } else {
        uint16_t *p = (uint16_t *)bits_out;
        for (int64_t i = 0; i < n; ++i) p[i] = (uint16_t)oracle_round_one(in[i], dtype);
    }
}

/* ----------------------------------------------------------------------- *
 * Assignment stage: for each point, the squared distance to every centroid,
 * and the nearest one.  X [B,N,d], C [B,K,d] (fp64, C already rounded to the
 * point dtype).  Outputs: labels [B,N]; d1 = nearest distance; d2 = second
 * nearest (INFINITY when K == 1), both [B,N].
 * ----------------------------------------------------------------------- */
void oracle_assign(const double *X, int64_t B, int64_t N, int64_t d,
                   const double *C, int64_t K,
                   int32_t *labels, double *d1, double *d2)
{
    int64_t total = B * N;
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < total; ++bi) {
        int64_t b = bi / N;
        const double *x = X + bi * d;
        const double *Cb = C + b * K * d;
        double best = INFINITY, second = INFINITY;
        int32_t arg = -1;
        for (int64_t j = 0; j < K; ++j) {
            const double *c = Cb + j * d;
            double D = 0.0;
            for (int64_t k = 0; k < d; ++k) {
                double t = x[k] - c[k];
                D += t * t;
            }
            if (D < best) {            /* strict: the smallest index wins a tie */
                second = best;
                best = D;
                arg = (int32_t)j;
            } else if (D < second) {
                second = D;
            }
        }
        labels[bi] = arg;
        d1[bi] = best;
        d2[bi] = second;
    }
}

/* ----------------------------------------------------------------------- *
 * Update stage: per cluster j the sum S_j = sum w_i x_i, the weight
 * W_j = sum w_i and the count N_j = #{i : l_i = j}, all accumulated in
 * point order; the new centroid is S_j / W_j, or the old one when N_j == 0.
 * w may be NULL (all weights 1).  S_out [B,K,d] and W_out [B,K] may be NULL.
 * c_new may alias c_old.
 * ----------------------------------------------------------------------- */
void oracle_update(const double *X, const double *w, const int32_t *labels,
                   int64_t B, int64_t N, int64_t d, int64_t K,
                   const float *c_old, float *c_new, int32_t *counts,
                   double *S_out, double *W_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        double *S = (double *)calloc((size_t)(K * d), sizeof(double));
        double *W = (double *)calloc((size_t)K, sizeof(double));
        int64_t *Nj = (int64_t *)calloc((size_t)K, sizeof(int64_t));
        for (int64_t i = 0; i < N; ++i) {
            int64_t j = labels[b * N + i];
            double wi = w ? w[b * N + i] : 1.0;
            const double *x = X + (b * N + i) * d;
            Nj[j] += 1;
            W[j] += wi;
            for (int64_t k = 0; k < d; ++k) S[j * d + k] += wi * x[k];
        }
        for (int64_t j = 0; j < K; ++j) {
            const float *co = c_old + (b * K + j) * d;
            float *cn = c_new + (b * K + j) * d;
            for (int64_t k = 0; k < d; ++k)
                cn[k] = Nj[j] > 0 ? (float)(S[j * d + k] / W[j]) : co[k];
            counts[b * K + j] = (int32_t)Nj[j];
            if (W_out) W_out[b * K + j] = W[j];
            if (S_out)
                for (int64_t k = 0; k < d; ++k) S_out[(b * K + j) * d + k] = S[j * d + k];
        }
        free(S);
        free(W);
        free(Nj);
    }
}

/* ----------------------------------------------------------------------- *
 * Objective of given labels: J_b = sum_i w_i * sum_k (x_ik - c_{l_i,k})^2,
 * i ascending, fp64.  With the labels of the assignment stage this is the
 * objective of that iteration.  C [B,K,d] fp64 (centroids in the point
 * dtype), w may be NULL.  Labels outside [0, K) contribute nothing.
 * ----------------------------------------------------------------------- */
void oracle_objective(const double *X, const double *w, const int32_t *labels,
                      int64_t B, int64_t N, int64_t d, const double *C, int64_t K,
                      double *J)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        double s = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            const int64_t j = labels[b * N + i];
            if (j < 0 || j >= K) continue;
            const double *x = X + (b * N + i) * d;
            const double *c = C + (b * K + j) * d;
            double D = 0.0;
            for (int64_t k = 0; k < d; ++k) {
                const double t = x[k] - c[k];
                D += t * t;
            }
            s += (w ? w[b * N + i] : 1.0) * D;
        }
        J[b] = s;
    }
}

/* ----------------------------------------------------------------------- *
 * The update stage and the objective of given labels, read straight from
 * the stored bits of the points (each element decoded exactly to fp64 where
 * it is used), for point sets too large to hold decoded in fp64.  The
 * arithmetic is that of oracle_update and oracle_objective, term for term
 * and in the same order, so the results are identical:
 *   - update: for every (b, k) the sum S_jk = sum_i w_i x_ik runs over i
 *     ascending, as in oracle_update; the work is divided over coordinates
 *     (one (b, k) pair per task), which does not change any sum.  W_j and
 *     the counts are accumulated by the task of coordinate 0.
 *   - objective: the per-point terms w_i * sum_k (x_ik - c_{l_i,k})^2 are
 *     computed in parallel into a buffer, then added in point order.
 * x: float32 bits, or uint16 bits of fp16 / bf16.  w [B,N] fp32 or NULL.
 * Returns 0, or -1 when memory runs out (objective) or a label is out of
 * range (update).
 * ----------------------------------------------------------------------- */
static double orc_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == ORC_F32) return (double)((const float *)x)[idx];
    return oracle_decode_one(((const uint16_t *)x)[idx], dtype);
}

int oracle_update_bits(const void *x, int dtype, const float *w, const int32_t *labels,
                       int64_t B, int64_t N, int64_t d, int64_t K,
                       const float *c_old, float *c_new, int32_t *counts,
                       double *S_out, double *W_out)
{
    for (int64_t i = 0; i < B * N; ++i)
        if (labels[i] < 0 || labels[i] >= K) return -1;
    double *S = (double *)calloc((size_t)(B * K * d), sizeof(double));
    double *W = (double *)calloc((size_t)(B * K), sizeof(double));
    int64_t *Nj = (int64_t *)calloc((size_t)(B * K), sizeof(int64_t));
    if (!S || !W || !Nj) {
        free(S); free(W); free(Nj);
        return -1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bk = 0; bk < B * d; ++bk) {
        const int64_t b = bk / d, k = bk % d;
        for (int64_t i = 0; i < N; ++i) {
            const int64_t j = labels[b * N + i];
            const double wi = w ? (double)w[b * N + i] : 1.0;
            if (k == 0) {
                Nj[b * K + j] += 1;
                W[b * K + j] += wi;
            }
            S[(b * K + j) * d + k] += wi * orc_elem(x, dtype, (b * N + i) * d + k);
        }
    }
    for (int64_t bj = 0; bj < B * K; ++bj) {
        for (int64_t k = 0; k < d; ++k)
            c_new[bj * d + k] = Nj[bj] > 0 ? (float)(S[bj * d + k] / W[bj]) : c_old[bj * d + k];
        counts[bj] = (int32_t)Nj[bj];
        if (W_out) W_out[bj] = W[bj];
        if (S_out)
            for (int64_t k = 0; k < d; ++k) S_out[bj * d + k] = S[bj * d + k];
    }
    free(S);
    free(W);
    free(Nj);
    return 0;
}

int oracle_objective_bits(const void *x, int dtype, const float *w, const int32_t *labels,
                          int64_t B, int64_t N, int64_t d, const double *C, int64_t K, double *J)
{
    double *term = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    if (!term) return -1;
    for (int64_t b = 0; b < B; ++b) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < N; ++i) {
            const int64_t j = labels[b * N + i];
            if (j < 0 || j >= K) {
                term[i] = 0.0;
                continue;
            }
            const double *c = C + (b * K + j) * d;
            double D = 0.0;
            for (int64_t k = 0; k < d; ++k) {
                const double t = orc_elem(x, dtype, (b * N + i) * d + k) - c[k];
                D += t * t;
            }
            term[i] = (w ? (double)w[b * N + i] : 1.0) * D;
        }
        double s = 0.0;
        for (int64_t i = 0; i < N; ++i) s += term[i];
        J[b] = s;
    }
    free(term);
    return 0;
}

/* ----------------------------------------------------------------------- *
 * n_iter Lloyd iterations from init [B,K,d] fp32.  x holds the stored bits
 * (float32, or uint16 for fp16/bf16).  w [B,N] fp32 or NULL.
 * Outputs: C_out [B,K,d] (centroids after the last update), labels_out and
 * d1_out / d2_out [B,N] (last assignment), counts_out [B,K] (last update),
 * J_out [B, n_iter] (objective of each assignment).  Returns 0, or -1 when
 * memory runs out.
 * ----------------------------------------------------------------------- */
int oracle_fit(const void *x, int dtype, const float *w,
               int64_t B, int64_t N, int64_t d, int64_t K,
               const float *init, int32_t n_iter,
               float *C_out, int32_t *labels_out, int32_t *counts_out,
               double *J_out, double *d1_out, double *d2_out)
{
    int64_t nx = B * N * d, nc = B * K * d;
    double *X = (double *)malloc((size_t)nx * sizeof(double));
    double *Wd = w ? (double *)malloc((size_t)(B * N) * sizeof(double)) : NULL;
    double *Ch = (double *)malloc((size_t)nc * sizeof(double));
    uint32_t *cbits = (uint32_t *)malloc((size_t)nc * sizeof(uint32_t));
    int ok = X && Ch && cbits && (!w || Wd);
    if (ok) {
        oracle_decode(x, dtype, nx, X);
        if (w)
            for (int64_t i = 0; i < B * N; ++i) Wd[i] = (double)w[i];
        memcpy(C_out, init, (size_t)nc * sizeof(float));
        for (int32_t t = 0; t < n_iter; ++t) {
            /* centroids as the assignment sees them: rounded to the point dtype */
            for (int64_t i = 0; i < nc; ++i) {
                cbits[i] = oracle_round_one(C_out[i], dtype);
                Ch[i] = oracle_decode_one(cbits[i], dtype);
            }
            oracle_assign(X, B, N, d, Ch, K, labels_out, d1_out, d2_out);
            for (int64_t b = 0; b < B; ++b) {
                double J = 0.0;
                for (int64_t i = 0; i < N; ++i)
                    J += (Wd ? Wd[b * N + i] : 1.0) * d1_out[b * N + i];
                J_out[b * n_iter + t] = J;
            }
            oracle_update(X, Wd, labels_out, B, N, d, K, C_out, C_out, counts_out, NULL, NULL);
        }
    }
    free(X);
    free(Wd);
    free(Ch);
    free(cbits);
    return ok ? 0 : -1;
}

/* ----------------------------------------------------------------------- *
 * Globally optimal weighted 1D k-means of every row (github LeanModels/
 * LeanQuant issue #1 "1D k-means": for scalar data the globally optimal
 * centroids can be found, and the diff swaps Lloyd for such a 1D clustering
 * with per-point sample weights that returns the centroids).
 *
 * Definition: among all partitions of a row's N points into K non-empty
 * groups, one with the least J = sum_g sum_{i in g} w_i (x_i - mean_g)^2,
 * mean_g = sum_g w_i x_i / sum_g w_i.  For scalars some optimal partition
 * consists of runs of consecutive values in ascending order, so J* is the
 * least cost over the ways to cut the sorted row into K non-empty runs.
 * That minimum is taken by dynamic programming over prefixes of the sorted
 * row:
 *     D[1][j] = SSE(0, j),
 *     D[k][j] = min over k-1 <= i < j of D[k-1][i] + SSE(i, j),
 * where SSE(i, j) is the weighted sum of squared deviations of sorted points
 * i .. j-1 from their weighted mean.  For fixed j, SSE(i, j) is accumulated
 * point by point as i moves down (running weight, weighted mean and sum of
 * squares, fp64).  The first minimizing i (smallest) is kept; points are
 * sorted by (value, original index).
 *
 * X [B,N] fp64 values, w [B,N] fp64 weights or NULL (all 1), 1 <= K <= N.
 * Outputs: J_out [B] = D[K][N]; means_out [B,K] the run means in ascending
 * order (fp64, each a fresh weighted average of its run); labels_out [B,N]
 * the run of every point (in the row's original order); counts_out [B,K] the
 * run sizes.  Returns 0, or -1 when memory runs out or K is out of range.
 * ----------------------------------------------------------------------- */
typedef struct { double v; int64_t i; } orc_vi;

static int orc_vi_cmp(const void *a, const void *b)
{
    const orc_vi *p = (const orc_vi *)a, *q = (const orc_vi *)b;
    if (p->v < q->v) return -1;
    if (p->v > q->v) return 1;
    return (p->i > q->i) - (p->i < q->i);
}

int oracle_optimal_1d(const double *X, const double *w, int64_t B, int64_t N, int64_t K,
                      double *J_out, double *means_out, int32_t *labels_out, int32_t *counts_out)
{
    if (K < 1 || K > N) return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t b = 0; b < B; ++b) {
        orc_vi *s = (orc_vi *)malloc((size_t)N * sizeof(orc_vi));
        double *xs = (double *)malloc((size_t)N * sizeof(double));
        double *ws = (double *)malloc((size_t)N * sizeof(double));
        double *D = (double *)malloc((size_t)((K + 1) * (N + 1)) * sizeof(double));
        int64_t *cut = (int64_t *)malloc((size_t)((K + 1) * (N + 1)) * sizeof(int64_t));
        int64_t *bound = (int64_t *)malloc((size_t)(K + 1) * sizeof(int64_t));
        if (!s || !xs || !ws || !D || !cut || !bound) {
            failed = 1;
        } else {
            for (int64_t i = 0; i < N; ++i) {
                s[i].v = X[b * N + i];
                s[i].i = i;
            }
            qsort(s, (size_t)N, sizeof(orc_vi), orc_vi_cmp);
            for (int64_t p = 0; p < N; ++p) {
                xs[p] = s[p].v;
                ws[p] = w ? w[b * N + s[p].i] : 1.0;
            }
            for (int64_t k = 0; k <= K; ++k)
                for (int64_t j = 0; j <= N; ++j) {
                    D[k * (N + 1) + j] = INFINITY;
                    cut[k * (N + 1) + j] = -1;
                }
            D[0] = 0.0; /* no points in no runs */
            for (int64_t k = 1; k <= K; ++k) {
                for (int64_t j = k; j <= N; ++j) {
                    double best = INFINITY;
                    int64_t arg = -1;
                    /* the last run is sorted points i .. j-1; grow it downwards */
                    double W = 0.0, mean = 0.0, sse = 0.0;
                    for (int64_t i = j - 1; i >= k - 1; --i) {
                        const double wi = ws[i], xi = xs[i];
                        const double Wn = W + wi;
                        const double delta = xi - mean;
                        const double mean_n = mean + wi * delta / Wn;
                        sse += wi * delta * (xi - mean_n);
                        W = Wn;
                        mean = mean_n;
                        const double cand = D[(k - 1) * (N + 1) + i] + sse;
                        /* i descends, so '<=' keeps the smallest i among equal costs */
                        if (cand <= best) {
                            best = cand;
                            arg = i;
                        }
                    }
                    D[k * (N + 1) + j] = best;
                    cut[k * (N + 1) + j] = arg;
                }
            }
            J_out[b] = D[K * (N + 1) + N];
            /* runs from the cuts: run k-1 is sorted points bound[k-1] .. bound[k]-1 */
            bound[K] = N;
            for (int64_t k = K; k >= 1; --k) bound[k - 1] = cut[k * (N + 1) + bound[k]];
            for (int64_t k = 0; k < K; ++k) {
                double sw = 0.0, swx = 0.0;
                for (int64_t p = bound[k]; p < bound[k + 1]; ++p) {
                    sw += ws[p];
                    swx += ws[p] * xs[p];
                    labels_out[b * N + s[p].i] = (int32_t)k;
                }
                means_out[b * K + k] = swx / sw;
                counts_out[b * K + k] = (int32_t)(bound[k + 1] - bound[k]);
            }
        }
        free(s);
        free(xs);
        free(ws);
        free(D);
        free(cut);
        free(bound);
    }
    return failed ? -1 : 0;
}

/* ----------------------------------------------------------------------- *
 * e-means (daily.steinslab.io "e-means" article): mini-batch k-means whose
 * cluster statistics are exponential moving averages.
 *   - "Breaking 70 Years of Full-Batch Inertia": each cluster keeps a sum
 *     S_j and a count N_j, the centroid is their quotient, and every batch
 *     updates S_j <- (1 - a) S_j + a s_j (s_j the batch's sum of cluster j;
 *     the same for N_j with the batch count n_j).  After the last epoch the
 *     centroids move to the plain mean of that epoch's assignments.
 *   - "Mini-Batch Stochastic Noise...": the step a follows a cosine decay
 *     from a0 down to 0.1 a0 (floor = 0.1 is the page's; it is a parameter).
 *   - "Proportional Splitting Resurrects Thousands of Dead Centers": a dead
 *     cluster takes over half of a live cluster drawn with probability
 *     proportional to its size, and the two are split apart.
 * Readings where the article is silent: batches are
 * consecutive slices of `batch` points in storage order (the caller fixes
 * the order); S and N start at zero and a centroid moves only once its N
 * is positive; a step t of T = epochs * ceil(N / batch) uses
 * a_t = a0 floor + a0 (1 - floor) (1 + cos(pi t / (T - 1))) / 2 (a0 when
 * T = 1); after a batch's update (before any of its splits), cluster j is
 * dead when N_j < dead_frac * min(batch, N) / K; dead clusters are handled
 * in ascending order, each with the uniform u = uniforms[t * K + j],
 * choosing the donor k as the first index whose prefix of N (taken after
 * the update, before any split of this batch) exceeds u * sum(N), skipping
 * k = j and a donor whose N is zero at its turn; the donor's S and N
 * halve, the dead cluster gets the same S and N, and their centroids
 * become c_k (1 + eps s_c) and c_k (1 - eps s_c), s_c = +1 for even and -1
 * for odd coordinates (S rescaled to match).  Assignments use the
 * centroids rounded to the point dtype, as in oracle_fit.
 *
 * x: stored bits [N, d]; init [K, d] fp32.  Outputs: C_out [K, d] fp32;
 * J_out [T] (sum of each batch's nearest distances at assignment time);
 * labels_out [N] (every point's assignment in the last epoch); counts_out
 * [K] (points per cluster in the last epoch).  Returns 0, or -1 when memory
 * runs out or an argument is out of range.
 * ----------------------------------------------------------------------- */
int oracle_emeans(const void *x, int dtype, int64_t N, int64_t d, int64_t K, const float *init,
                  int64_t batch, int32_t epochs, double alpha0, double floor_frac, double dead_frac,
                  double eps, const float *uniforms, float *C_out, double *J_out, int32_t *labels_out,
                  int32_t *counts_out)
{
    if (N < 1 || d < 1 || K < 1 || batch < 1 || epochs < 1) return -1;
    const int64_t nb = (N + batch - 1) / batch, T = (int64_t)epochs * nb;
    const int64_t mfull = batch < N ? batch : N;
    double *X = (double *)malloc((size_t)(N * d) * sizeof(double));
    double *S = (double *)calloc((size_t)(K * d), sizeof(double));
    double *Nc = (double *)calloc((size_t)K, sizeof(double));
    double *s = (double *)malloc((size_t)(K * d) * sizeof(double));
    double *n = (double *)malloc((size_t)K * sizeof(double));
    double *F = (double *)calloc((size_t)(K * d), sizeof(double));
    double *G = (double *)calloc((size_t)K, sizeof(double));
    double *Ch = (double *)malloc((size_t)(K * d) * sizeof(double));
    double *P = (double *)malloc((size_t)(K + 1) * sizeof(double));
    char *dead = (char *)malloc((size_t)K);
    int32_t *lab = (int32_t *)malloc((size_t)mfull * sizeof(int32_t));
    double *d1 = (double *)malloc((size_t)mfull * sizeof(double));
    double *d2 = (double *)malloc((size_t)mfull * sizeof(double));
    int ok = X && S && Nc && s && n && F && G && Ch && P && dead && lab && d1 && d2;
    if (ok) {
        oracle_decode(x, dtype, N * d, X);
        memcpy(C_out, init, (size_t)(K * d) * sizeof(float));
        for (int64_t t = 0; t < T; ++t) {
            const int64_t e = t / nb, i0 = (t % nb) * batch;
            const int64_t m = (i0 + batch <= N) ? batch : N - i0;
            const double a = T > 1 ? alpha0 * floor_frac +
                                         alpha0 * (1.0 - floor_frac) * 0.5 * (1.0 + cos(acos(-1.0) * (double)t / (double)(T - 1)))
                                   : alpha0;
            for (int64_t q = 0; q < K * d; ++q) Ch[q] = oracle_decode_one(oracle_round_one(C_out[q], dtype), dtype);
            oracle_assign(X + i0 * d, 1, m, d, Ch, K, lab, d1, d2);
            double J = 0.0;
            for (int64_t i = 0; i < m; ++i) J += d1[i];
            J_out[t] = J;
            for (int64_t q = 0; q < K * d; ++q) s[q] = 0.0;
            for (int64_t j = 0; j < K; ++j) n[j] = 0.0;
            for (int64_t i = 0; i < m; ++i) {
                const int64_t j = lab[i];
                n[j] += 1.0;
                for (int64_t c = 0; c < d; ++c) s[j * d + c] += X[(i0 + i) * d + c];
            }
            if (e == epochs - 1) {
                for (int64_t q = 0; q < K * d; ++q) F[q] += s[q];
                for (int64_t j = 0; j < K; ++j) G[j] += n[j];
                for (int64_t i = 0; i < m; ++i) labels_out[i0 + i] = lab[i];
            }
            for (int64_t j = 0; j < K; ++j) {
                Nc[j] = (1.0 - a) * Nc[j] + a * n[j];
                for (int64_t c = 0; c < d; ++c) {
                    S[j * d + c] = (1.0 - a) * S[j * d + c] + a * s[j * d + c];
                    if (Nc[j] > 0.0) C_out[j * d + c] = (float)(S[j * d + c] / Nc[j]);
                }
            }
            /* proportional splitting of dead clusters */
            P[0] = 0.0;
            for (int64_t j = 0; j < K; ++j) P[j + 1] = P[j] + Nc[j];
            const double dead_below = dead_frac * (double)mfull / (double)K;
            for (int64_t j = 0; j < K; ++j) dead[j] = Nc[j] < dead_below;
            for (int64_t j = 0; j < K; ++j) {
                if (!dead[j]) continue;
                const double target = (double)uniforms[t * K + j] * P[K];
                int64_t k = 0;
                while (k < K - 1 && !(P[k + 1] > target)) ++k;
                if (k == j || !(Nc[k] > 0.0)) continue;
                Nc[k] *= 0.5;
                Nc[j] = Nc[k];
                for (int64_t c = 0; c < d; ++c) {
                    const double ck = S[k * d + c] * 0.5 / Nc[k];
                    const double sgn = (c % 2 == 0) ? 1.0 : -1.0;
                    const float cj = (float)(ck * (1.0 + eps * sgn));
                    const float ckn = (float)(ck * (1.0 - eps * sgn));
                    C_out[j * d + c] = cj;
                    C_out[k * d + c] = ckn;
                    S[j * d + c] = (double)cj * Nc[j];
                    S[k * d + c] = (double)ckn * Nc[k];
                }
            }
        }
        for (int64_t j = 0; j < K; ++j) {
            counts_out[j] = (int32_t)G[j];
            if (G[j] > 0.0)
                for (int64_t c = 0; c < d; ++c) C_out[j * d + c] = (float)(F[j * d + c] / G[j]);
        }
    }
    free(X); free(S); free(Nc); free(s); free(n); free(F); free(G); free(Ch); free(P); free(dead); free(lab);
    free(d1); free(d2);
    return ok ? 0 : -1;
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
