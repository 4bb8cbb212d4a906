/*
 * tbe_oracle.c -- plain, single-threaded CPU oracle of the Table Batched
 * Embedding (TBE) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  The product (the HIP
 * library under table_embedding_amd/) never calls it, and the two share no
 * code, header, constant or helper: every value below is derived here from the
 * method's definition.
 *
 * Sources (pages as published; sections named, no line numbers):
 *  - "Modernizing Table Batched Embeddings with FBTriton" (English summary at
 *    yuxiaoba.github.io/tech/en/fbtriton-tbe), sections "Why redesign a sparse
 *    operator?", "Forward", "Backward", "Fusion boundaries", "Read results".
 *  - "NVIDIA HugeCTR ... DistributedSlotSparseEmbeddingHash backward" walkthrough
 *    (eqicode.com QuestionAnswer 2236): CSR input example, sample-id
 *    expansion (step 1), radix sort by row (step 3), run counting (step 4),
 *    gradient accumulation and the Adagrad kernel (step 5).
 *
 * Conventions (plain readings of the pages, listed with the other readings of
 * the design notes):
 *  - T tables; table t has R_t rows of width D_t, pooling sum or mean.
 *  - B bags per table, table-major: bag j = t*B + b, CSR offsets O[0..T*B].
 *  - Lookups p in [O[j], O[j+1]) belong to bag j; I[p] is a row of table t.
 *  - Output / grad rows are [B, Dtot] FP32 with table t at columns
 *    [c_t, c_t + D_t), c_t = sum of earlier widths.
 *  - Everything real is accumulated in double; results are rounded to the
 *    stored type with round-to-nearest-even.
 *  - Linear row key of a lookup = base_t + I[p], base_t = sum of earlier R_t
 *    (table order).
 *
 * Every function validates its inputs and returns a negative code on a
 * violation (index outside [0, R_t), offsets not monotone).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* storage codes used by this oracle's Python wrapper */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_I32 = 0, OR_I64 = 1 };
enum { OR_SUM = 0, OR_MEAN = 1 };
/* run-length threshold and chunk size of the backward ("Backward": runs
 * shorter than 256 lookups are updated by one owner; longer runs are cut
 * into chunks of 256 lookups). */
enum { OR_LONG_RUN = 256, OR_CHUNK = 256 };

/* ------------------------------------------------------------------------
 * Number formats.  IEEE 754 binary16 (1/5/10) and bfloat16 (1/8/7, the upper
 * half of binary32).  Decoding follows the format definition; rounding is
 * roundTiesToEven with gradual underflow and overflow to infinity.
 * ---------------------------------------------------------------------- */

/* Round x to p significand bits (hidden bit included), minimum normal
 * exponent emin, maximum exponent emax. */
static double round_format(double x, int p, int emin, int emax)
{
    if (x != x || x == 0.0 || isinf(x))
        return x;
    int e;
    frexp(x, &e);            /* |x| in [2^(e-1), 2^e) */
    int lead = e - 1;
    if (lead < emin)
        lead = emin;         /* subnormal range: the quantum stops shrinking */
    double q = ldexp(1.0, lead - (p - 1));
    double r = nearbyint(x / q) * q; /* default rounding mode: ties to even */
    double maxf = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxf)
        return copysign(INFINITY, x);
    return r;
}

double oracle_round(int32_t wdtype, double x)
{
    switch (wdtype) {
    case OR_F32: return (double)(float)x;
    case OR_F16: return round_format(x, 11, -14, 15);
    case OR_BF16: return round_format(x, 8, -126, 127);
    }
    return NAN;
}

static double decode_small(uint16_t h, int mbits, int ebits)
{
    int bias = (1 << (ebits - 1)) - 1;
    int s = h >> 15;
    int e = (h >> mbits) & ((1 << ebits) - 1);
    int m = h & ((1 << mbits) - 1);
    double v;
    if (e == 0)
        v = ldexp((double)m, 1 - bias - mbits);
    else if (e == (1 << ebits) - 1)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)((1 << mbits) + m), e - bias - mbits);
    return s ? -v : v;
}

/* x must already be representable (output of round_format) */
static uint16_t encode_small(double x, int mbits, int ebits)
{
    int bias = (1 << (ebits - 1)) - 1;
    uint16_t s = signbit(x) ? 0x8000u : 0u;
    uint16_t emax_field = (uint16_t)((1 << ebits) - 1);
    if (x != x)
        return (uint16_t)(s | (emax_field << mbits) | (1u << (mbits - 1)));
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(s | (emax_field << mbits));
    if (a == 0.0)
        return s;
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < 1 - bias) /* subnormal: value = m * 2^(1-bias-mbits) */
        return (uint16_t)(s | (uint16_t)ldexp(a, -(1 - bias - mbits)));
    uint16_t m = (uint16_t)(ldexp(a, mbits - lead) - (double)(1 << mbits));
    return (uint16_t)(s | ((uint16_t)(lead + bias) << mbits) | m);
}

double oracle_decode(int32_t wdtype, const void *w, int64_t i)
{
    switch (wdtype) {
    case OR_F32: return (double)((const float *)w)[i];
    case OR_F16: return decode_small(((const uint16_t *)w)[i], 10, 5);
    case OR_BF16: return decode_small(((const uint16_t *)w)[i], 7, 8);
    }
    return NAN;
}

/* store round-to-nearest-even(x) at element i */
void oracle_store(int32_t wdtype, void *w, int64_t i, double x)
{
    double r = oracle_round(wdtype, x);
    switch (wdtype) {
    case OR_F32: ((float *)w)[i] = (float)r; break;
    case OR_F16: ((uint16_t *)w)[i] = encode_small(r, 10, 5); break;
    case OR_BF16: ((uint16_t *)w)[i] = encode_small(r, 7, 8); break;
    }
}

static int64_t load_index(int32_t itype, const void *a, int64_t i)
{
    return itype == OR_I32 ? (int64_t)((const int32_t *)a)[i] : ((const int64_t *)a)[i];
}

/* Offsets: O[0] = 0, non-decreasing, O[T*B] = N; every index inside its table. */
static int validate(int32_t T, const int64_t *rows, int64_t B, int32_t itype,
                    const void *indices, const void *offsets)
{
    if (T < 0 || B < 0)
        return -1;
    if (load_index(itype, offsets, 0) != 0)
        return -2;
    for (int64_t j = 0; j < (int64_t)T * B; ++j) {
        int64_t lo = load_index(itype, offsets, j), hi = load_index(itype, offsets, j + 1);
        if (hi < lo)
            return -2;
        int64_t t = j / B;
        for (int64_t p = lo; p < hi; ++p) {
            int64_t r = load_index(itype, indices, p);
            if (r < 0 || r >= rows[t])
                return -3;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Forward ("Forward": each bag gathers its indexed rows and pools them; mean
 * pooling = sum then scale by 1/L, HugeCTR forward_sum + forward_scale):
 *   out[b, c_t + d] = (1/L if mean) * sum_{p in bag(t,b)} S[p] * W_t[I[p], d]
 * an empty bag gives 0.
 * ---------------------------------------------------------------------- */
int oracle_forward(int32_t T, const int64_t *rows, const int32_t *dims, const int32_t *pooling,
                   int32_t wdtype, const void *const *weights, int64_t B, int32_t itype,
                   const void *indices, const void *offsets, const float *psw,
                   float *out, int64_t out_stride)
{
    int rc = validate(T, rows, B, itype, indices, offsets);
    if (rc)
        return rc;
    int64_t dmax = 1;
    for (int32_t t = 0; t < T; ++t)
        if (dims[t] > dmax)
            dmax = dims[t];
    double *acc = (double *)malloc(sizeof(double) * (size_t)dmax);
    if (!acc)
        return -9;
    int64_t col = 0;
    for (int32_t t = 0; t < T; ++t) {
        int64_t D = dims[t];
        for (int64_t b = 0; b < B; ++b) {
            int64_t j = (int64_t)t * B + b;
            int64_t lo = load_index(itype, offsets, j), hi = load_index(itype, offsets, j + 1);
            for (int64_t d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t p = lo; p < hi; ++p) {
                int64_t r = load_index(itype, indices, p);
                double s = psw ? (double)psw[p] : 1.0;
                for (int64_t d = 0; d < D; ++d)
                    acc[d] += s * oracle_decode(wdtype, weights[t], r * D + d);
            }
            if (pooling[t] == OR_MEAN && hi > lo)
                for (int64_t d = 0; d < D; ++d)
                    acc[d] /= (double)(hi - lo);
            for (int64_t d = 0; d < D; ++d)
                out[b * out_stride + col + d] = (float)acc[d];
        }
        col += D;
    }
    free(acc);
    return 0;
}

/* ------------------------------------------------------------------------
 * Preprocessing ("Backward": transposition, sorting and run-length encoding
 * turn "rows a sample used" into "samples that used a row"; HugeCTR steps 1,
 * 3 and 4 print the same pipeline with every intermediate array):
 *   P1  key[p] = base_t + I[p], bag[p] = j                 (transposition)
 *   P2  positions stably sorted by key                     (sort)
 *   P3  maximal blocks of equal key -> runs                (run-length encoding)
 *   P4  runs shorter than 256 -> short list, others -> long list and chunks
 *       of 256 lookups, the last chunk possibly shorter    (classification)
 * Outputs (caller allocates: N for per-lookup arrays, N+1 for run_start,
 * N for per-run arrays, N/256 + N for chunk arrays is always enough):
 *   counts = {U, n_short, n_long, n_chunks}.
 * ---------------------------------------------------------------------- */
typedef struct {
    uint64_t key;
    int64_t pos;
} kp_t;

static int cmp_kp(const void *a, const void *b)
{
    const kp_t *x = (const kp_t *)a, *y = (const kp_t *)b;
    if (x->key != y->key)
        return x->key < y->key ? -1 : 1;
    /* equal keys keep ascending position: a stable sort */
    return x->pos < y->pos ? -1 : (x->pos > y->pos ? 1 : 0);
}

int oracle_preprocess(int32_t T, const int64_t *rows, int64_t B, int32_t itype,
                      const void *indices, const void *offsets,
                      uint64_t *key, int64_t *bag, uint64_t *sorted_key, int64_t *sorted_pos,
                      int64_t *run_start, uint64_t *run_key, int64_t *short_list,
                      int64_t *long_list, int64_t *chunk_long, int64_t *chunk_start,
                      int64_t *chunk_len, int64_t *counts)
{
    int rc = validate(T, rows, B, itype, indices, offsets);
    if (rc)
        return rc;
    int64_t N = load_index(itype, offsets, (int64_t)T * B);
    /* P1 transposition */
    int64_t base = 0;
    for (int32_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < B; ++b) {
            int64_t j = (int64_t)t * B + b;
            int64_t lo = load_index(itype, offsets, j), hi = load_index(itype, offsets, j + 1);
            for (int64_t p = lo; p < hi; ++p) {
                key[p] = (uint64_t)(base + load_index(itype, indices, p));
                bag[p] = j;
            }
        }
        base += rows[t];
    }
    /* P2 stable sort of positions by key */
    kp_t *kp = (kp_t *)malloc(sizeof(kp_t) * (size_t)(N ? N : 1));
    if (!kp)
        return -9;
    for (int64_t p = 0; p < N; ++p) {
        kp[p].key = key[p];
        kp[p].pos = p;
    }
    qsort(kp, (size_t)N, sizeof(kp_t), cmp_kp);
    for (int64_t i = 0; i < N; ++i) {
        sorted_key[i] = kp[i].key;
        sorted_pos[i] = kp[i].pos;
    }
    free(kp);
    /* P3 run-length encoding */
    int64_t U = 0;
    for (int64_t i = 0; i < N; ++i) {
        if (i == 0 || sorted_key[i] != sorted_key[i - 1]) {
            run_start[U] = i;
            run_key[U] = sorted_key[i];
            ++U;
        }
    }
    run_start[U] = N;
    /* P4 classification and chunk tasks, ascending run order */
    int64_t ns = 0, nl = 0, nc = 0;
    for (int64_t u = 0; u < U; ++u) {
        int64_t len = run_start[u + 1] - run_start[u];
        if (len < OR_LONG_RUN) {
            short_list[ns++] = u;
            continue;
        }
        for (int64_t k = 0; k * OR_CHUNK < len; ++k) {
            chunk_long[nc] = nl;
            chunk_start[nc] = run_start[u] + k * OR_CHUNK;
            chunk_len[nc] = (len - k * OR_CHUNK) < OR_CHUNK ? (len - k * OR_CHUNK) : OR_CHUNK;
            ++nc;
        }
        long_list[nl++] = u;
    }
    counts[0] = U;
    counts[1] = ns;
    counts[2] = nl;
    counts[3] = nc;
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward with exact row-wise Adagrad, applied once per touched row
 * ("Backward"; "Fusion boundaries": per-sample weights scale each gradient
 * contribution before grouping; HugeCTR step 5: the run's gradient is the sum
 * of the gradient rows of its samples; mean pooling scales by 1/L).
 * For each run u of table t and row r:
 *   g[d]  = sum_i S[p_i] * G[b(p_i), c_t + d] * (1/L_bag if mean)   (ascending i)
 *   m     = M_t[r] + (sum_d g[d]^2) / D_t ;  M_t[r] <- float(m)
 *   W_t[r,d] <- rne(W_t[r,d] - lr * g[d] / (sqrt(M_t[r]) + eps))
 * The momentum is updated first and the new value is used; eps is outside
 * the square root.  Rows no lookup touched are left as they are.
 * ---------------------------------------------------------------------- */
/* Optimizer epilogues applied once per touched row r of table t to its
 * gradient g[0..D) (accumulated in double):
 *  OR_OPT_ROWWISE_ADAGRAD  (FBTriton page, "Backward"; HugeCTR step 5 as the
 *      row-wise variant): state M[r] += mean_d g[d]^2, stored as float; then
 *      w[d] -= lr * g[d] / (sqrt(M[r]) + eps).
 *  OR_OPT_ADAGRAD  (HugeCTR walkthrough, step 5, the element-wise Adagrad
 *      kernel): state A[r*D + d] += g[d]^2, stored as float; then
 *      w[d] -= lr * g[d] / (sqrt(A[r*D + d]) + eps).
 *  OR_OPT_SGD: w[d] -= lr * g[d]; no state.
 * The square root and the step use the stored (float) state, as the row-wise
 * case does. */
enum { OR_OPT_ROWWISE_ADAGRAD = 0, OR_OPT_ADAGRAD = 1, OR_OPT_SGD = 2 };

int oracle_backward(int32_t T, const int64_t *rows, const int32_t *dims,
                    const int32_t *pooling, int32_t wdtype, void *const *weights,
                    float *const *state, int64_t B, int32_t itype, const void *indices,
                    const void *offsets, const float *psw, const float *grad,
                    int64_t grad_stride, int32_t optimizer, float lr, float eps)
{
    if (optimizer < OR_OPT_ROWWISE_ADAGRAD || optimizer > OR_OPT_SGD)
        return -8;
    int rc = validate(T, rows, B, itype, indices, offsets);
    if (rc)
        return rc;
    int64_t N = load_index(itype, offsets, (int64_t)T * B);
    size_t n1 = (size_t)(N ? N : 1);
    uint64_t *key = malloc(sizeof(uint64_t) * n1), *skey = malloc(sizeof(uint64_t) * n1),
             *rkey = malloc(sizeof(uint64_t) * n1);
    int64_t *bag = malloc(sizeof(int64_t) * n1), *spos = malloc(sizeof(int64_t) * n1),
            *rstart = malloc(sizeof(int64_t) * (n1 + 1)), *sl = malloc(sizeof(int64_t) * n1),
            *ll = malloc(sizeof(int64_t) * n1), *cl = malloc(sizeof(int64_t) * (n1 + 1)),
            *cs = malloc(sizeof(int64_t) * (n1 + 1)), *cn = malloc(sizeof(int64_t) * (n1 + 1));
    int64_t counts[4];
    int64_t *base = malloc(sizeof(int64_t) * (size_t)(T + 1));
    int64_t *col = malloc(sizeof(int64_t) * (size_t)(T + 1));
    int64_t dmax = 1;
    double *g = NULL;
    rc = -9;
    if (!key || !skey || !rkey || !bag || !spos || !rstart || !sl || !ll || !cl || !cs || !cn ||
        !base || !col)
        goto done;
    rc = oracle_preprocess(T, rows, B, itype, indices, offsets, key, bag, skey, spos, rstart,
                           rkey, sl, ll, cl, cs, cn, counts);
    if (rc)
        goto done;
    base[0] = 0;
    col[0] = 0;
    for (int32_t t = 0; t < T; ++t) {
        base[t + 1] = base[t] + rows[t];
        col[t + 1] = col[t] + dims[t];
        if (dims[t] > dmax)
            dmax = dims[t];
    }
    g = (double *)malloc(sizeof(double) * (size_t)dmax);
    if (!g) {
        rc = -9;
        goto done;
    }
    int32_t t = 0;
    for (int64_t u = 0; u < counts[0]; ++u) {
        /* table of the run: base_t <= key < base_{t+1} (keys ascend with u) */
        while ((int64_t)rkey[u] >= base[t + 1])
            ++t;
        int64_t r = (int64_t)rkey[u] - base[t];
        int64_t D = dims[t];
        for (int64_t d = 0; d < D; ++d)
            g[d] = 0.0;
        for (int64_t i = rstart[u]; i < rstart[u + 1]; ++i) {
            int64_t p = spos[i];
            int64_t j = bag[p];
            int64_t b = j - (int64_t)t * B;
            double s = psw ? (double)psw[p] : 1.0;
            if (pooling[t] == OR_MEAN) {
                int64_t L = load_index(itype, offsets, j + 1) - load_index(itype, offsets, j);
                s *= 1.0 / (double)L;
            }
            for (int64_t d = 0; d < D; ++d)
                g[d] += s * (double)grad[b * grad_stride + col[t] + d];
        }
        if (optimizer == OR_OPT_ROWWISE_ADAGRAD) {
            double sq = 0.0;
            for (int64_t d = 0; d < D; ++d)
                sq += g[d] * g[d];
            float *M = state[t];
            M[r] = (float)((double)M[r] + sq / (double)D);
            double denom = sqrt((double)M[r]) + (double)eps;
            for (int64_t d = 0; d < D; ++d) {
                double w = oracle_decode(wdtype, weights[t], r * D + d);
                oracle_store(wdtype, weights[t], r * D + d, w - (double)lr * g[d] / denom);
            }
        } else if (optimizer == OR_OPT_ADAGRAD) {
            float *A = state[t];
            for (int64_t d = 0; d < D; ++d) {
                A[r * D + d] = (float)((double)A[r * D + d] + g[d] * g[d]);
                double denom = sqrt((double)A[r * D + d]) + (double)eps;
                double w = oracle_decode(wdtype, weights[t], r * D + d);
                oracle_store(wdtype, weights[t], r * D + d, w - (double)lr * g[d] / denom);
            }
        } else {
            for (int64_t d = 0; d < D; ++d) {
                double w = oracle_decode(wdtype, weights[t], r * D + d);
                oracle_store(wdtype, weights[t], r * D + d, w - (double)lr * g[d]);
            }
        }
    }
    rc = 0;
done:
    free(key); free(skey); free(rkey); free(bag); free(spos); free(rstart); free(sl);
    free(ll); free(cl); free(cs); free(cn); free(base); free(col); free(g);
    return rc;
}

int oracle_backward_rowwise_adagrad(int32_t T, const int64_t *rows, const int32_t *dims,
                                    const int32_t *pooling, int32_t wdtype,
                                    void *const *weights, float *const *momentum, int64_t B,
                                    int32_t itype, const void *indices, const void *offsets,
                                    const float *psw, const float *grad, int64_t grad_stride,
                                    float lr, float eps)
{
    return oracle_backward(T, rows, dims, pooling, wdtype, weights, momentum, B, itype, indices,
                           offsets, psw, grad, grad_stride, OR_OPT_ROWWISE_ADAGRAD, lr, eps);
}
