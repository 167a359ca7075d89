/*
 * oracle.c -- plain fp64 CPU reference for one tensor-parallel rank's Transformer-block shard.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
 * CPU-baseline leg of the benchmark load this library. The HIP product path never calls it,
 * and it shares no source, header or constant with that path.
 *
 * What it computes, and where the pages define it:
 *   - A linear layer Y = X W (+ b), with W in R^{H_in x H_out} stored row-major
 *     (llms.blog, "The Core Primitives", the definition of X, W and Y).
 *   - The MLP block GeLU(X A) B and its tensor-parallel split: A split by columns,
 *     B split by rows, rank r computing GeLU(X A_r) B_r, the block output being the sum
 *     over ranks (ai360xpert.com, "How It Works", steps 1-3; llms.blog, "Partitioning the
 *     Multi-Layer Perceptron (MLP) Block"). The column bias a is split with its columns.
 *   - GeLU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), the exact form. The pages name
 *     GeLU without a formula; the exact-erf form is the reading taken here.
 *   - Attention of the rank's heads (llms.blog, "Partitioning Multi-Head and Grouped-Query
 *     Attention", steps 1-3): Q, K, V projections on the columns of the rank's heads,
 *     Head = softmax(Q K^T / sqrt(d_k)) V per head, heads concatenated locally, times the
 *     matching row slice of W_O. Causal masking (key k visible to query i iff k <= i in
 *     the same sequence) is the configured variant; causal = 0 is the unmasked formula.
 *   - The partial sum Y = sum_r Y_r that the all-reduce computes (llms.blog, "Row-Parallel
 *     Linear Layer", output and communication bullets).
 *
 * Conventions: activations are passed as fp64 (exact copies of the fp32/bf16 inputs),
 * weights and biases as fp32 and widened to fp64 for every product; every sum is fp64.
 * Rank r owns the contiguous column range [r*F/N, (r+1)*F/N) of A and the same row range
 * of B; for attention it owns heads r*H/N ... (r+1)*H/N - 1, i.e. the columns
 * [r*h/N, (r+1)*h/N) of W_Q, W_K, W_V and the same rows of W_O. Token row t = b*seq + s.
 * Unequal splits are rejected (return -1), as the pages only ever use exact shards.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* GeLU, exact erf form                                                                   */
/* ------------------------------------------------------------------------------------ */
double oracle_gelu(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

void oracle_gelu_array(const double* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_gelu(x[i]);
}

/* ------------------------------------------------------------------------------------ */
/* Linear layer on a column range of W:                                                    */
/*   Y[t, o - col_lo] = bias[o] + sum_k X[t, k] * W[k, o],  o in [col_lo, col_hi)          */
/* X is [rows, in] with row stride ldx, W is [in, ldw] row-major, Y is [rows, ldy].        */
/* ------------------------------------------------------------------------------------ */
static void linear_cols(const double* X, int64_t ldx, const float* W, int64_t ldw,
                        const float* bias, double* Y, int64_t ldy, int64_t rows, int64_t in,
                        int64_t col_lo, int64_t col_hi)
{
    const int64_t width = col_hi - col_lo;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < rows; ++t) {
        double* y = Y + t * ldy;
        for (int64_t j = 0; j < width; ++j) y[j] = bias ? (double)bias[col_lo + j] : 0.0;
        const double* x = X + t * ldx;
        for (int64_t k = 0; k < in; ++k) {
            const double xk = x[k];
            const float* w = W + k * ldw + col_lo;
            for (int64_t j = 0; j < width; ++j) y[j] += xk * (double)w[j];
        }
    }
}

/* Y = X W (+ bias) for a contiguous W [in, out]. */
void oracle_linear(const double* X, const float* W, const float* bias, double* Y,
                   int64_t rows, int64_t in, int64_t out)
{
    linear_cols(X, in, W, out, bias, Y, out, rows, in, 0, out);
}

/* Same with an fp64 weight (used for products of two fp64 intermediates). */
static void linear_dd(const double* X, int64_t ldx, const double* W, int64_t ldw,
                      double* Y, int64_t ldy, int64_t rows, int64_t in, int64_t out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < rows; ++t) {
        double* y = Y + t * ldy;
        for (int64_t j = 0; j < out; ++j) y[j] = 0.0;
        for (int64_t k = 0; k < in; ++k) {
            const double xk = X[t * ldx + k];
            const double* w = W + k * ldw;
            for (int64_t j = 0; j < out; ++j) y[j] += xk * w[j];
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* MLP block                                                                             */
/* ------------------------------------------------------------------------------------ */

/* Column-parallel half of rank r: Y_r = GeLU(X A_r + a_r), Y_r is [T, F/N]. */
int oracle_mlp_column(const double* X, const float* A, const float* a, double* Y_r,
                      int64_t T, int64_t h, int64_t F, int N, int r)
{
    if (N < 1 || r < 0 || r >= N || F % N != 0) return -1;
    const int64_t Fl = F / N, lo = (int64_t)r * Fl;
    linear_cols(X, h, A, F, a, Y_r, Fl, T, h, lo, lo + Fl);
    oracle_gelu_array(Y_r, Y_r, T * Fl);
    return 0;
}

/* Row-parallel half of rank r: Z_r = Y_r B_r with B_r = B[r*F/N : (r+1)*F/N, :]. */
int oracle_mlp_row(const double* Y_r, const float* B, double* Z_r,
                   int64_t T, int64_t h, int64_t F, int N, int r)
{
    if (N < 1 || r < 0 || r >= N || F % N != 0) return -1;
    const int64_t Fl = F / N;
    const float* B_r = B + (int64_t)r * Fl * h;   /* rows of B are contiguous */
    linear_cols(Y_r, Fl, B_r, h, NULL, Z_r, h, T, Fl, 0, h);
    return 0;
}

/* Rank r's MLP partial Z_r = GeLU(X A_r + a_r) B_r. With N = 1 this is the unsharded block. */
int oracle_mlp_shard(const double* X, const float* A, const float* a, const float* B,
                     double* Z_r, int64_t T, int64_t h, int64_t F, int N, int r)
{
    if (N < 1 || r < 0 || r >= N || F % N != 0) return -1;
    double* Y = (double*)malloc(sizeof(double) * (size_t)(T * (F / N)));
    if (!Y) return -2;
    int rc = oracle_mlp_column(X, A, a, Y, T, h, F, N, r);
    if (rc == 0) rc = oracle_mlp_row(Y, B, Z_r, T, h, F, N, r);
    free(Y);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* Attention block                                                                         */
/* ------------------------------------------------------------------------------------ */

/* Projections of rank r: Q_r = X W_Q[:, C_r] + b_Q[C_r] (and K, V alike), each [T, h/N],
   C_r = columns of heads r*H/N ... (r+1)*H/N - 1. Any bias pointer may be NULL. */
int oracle_qkv_shard(const double* X, const float* Wq, const float* Wk, const float* Wv,
                     const float* bq, const float* bk, const float* bv,
                     double* Q, double* K, double* V, int64_t T, int64_t h, int H, int N, int r)
{
    if (N < 1 || r < 0 || r >= N || H < 1 || h % H != 0 || H % N != 0) return -1;
    const int64_t w = h / N, lo = (int64_t)r * w;
    if (Q) linear_cols(X, h, Wq, h, bq, Q, w, T, h, lo, lo + w);
    if (K) linear_cols(X, h, Wk, h, bk, K, w, T, h, lo, lo + w);
    if (V) linear_cols(X, h, Wv, h, bv, V, w, T, h, lo, lo + w);
    return 0;
}

/* Softmax attention of n_heads heads of width d on token rows laid out t = b*seq + s.
   Q, K, V are [T, n_heads*d] (head j in columns j*d ... j*d+d-1). For each requested query
   row t (all T rows if rows == NULL) and each head, with s_k = <Q[t], K[b*seq+k]> / sqrt(d)
   over visible keys k (k <= s if causal, else all k < seq):
       O[t] = sum_k exp(s_k - m) V[b*seq+k] / sum_k exp(s_k - m),  m = max_k s_k.
   O is [n_rows, n_heads*d] in the order of `rows`: heads concatenated locally. */
int oracle_attention(const double* Q, const double* K, const double* V, double* O,
                     int64_t batch, int64_t seq, int n_heads, int64_t d, int causal,
                     const int64_t* rows, int64_t n_rows)
{
    if (batch < 1 || seq < 1 || n_heads < 1 || d < 1) return -1;
    const int64_t T = batch * seq, ld = (int64_t)n_heads * d;
    const int64_t nq = rows ? n_rows : T;
    const double scale = 1.0 / sqrt((double)d);
    for (int64_t i = 0; i < nq; ++i) {
        const int64_t t = rows ? rows[i] : i;
        if (t < 0 || t >= T) return -1;
    }
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t i = 0; i < nq; ++i) {
        for (int j = 0; j < n_heads; ++j) {
            const int64_t t = rows ? rows[i] : i;
            const int64_t b = t / seq, s = t % seq;
            const int64_t n_keys = causal ? s + 1 : seq;
            const double* q = Q + t * ld + (int64_t)j * d;
            double* score = (double*)malloc(sizeof(double) * (size_t)n_keys);
            double m = -INFINITY;
            for (int64_t k = 0; k < n_keys; ++k) {
                const double* kk = K + (b * seq + k) * ld + (int64_t)j * d;
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c) dot += q[c] * kk[c];
                score[k] = dot * scale;
                if (score[k] > m) m = score[k];
            }
            double denom = 0.0;
            for (int64_t k = 0; k < n_keys; ++k) {
                score[k] = exp(score[k] - m);
                denom += score[k];
            }
            double* o = O + i * ld + (int64_t)j * d;
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            for (int64_t k = 0; k < n_keys; ++k) {
                const double* vv = V + (b * seq + k) * ld + (int64_t)j * d;
                const double p = score[k] / denom;
                for (int64_t c = 0; c < d; ++c) o[c] += p * vv[c];
            }
            free(score);
        }
    }
    return 0;
}

/* Row-parallel output projection of rank r: Z_r = O_r W_O[C_r, :], O_r is [n_rows, h/N]. */
int oracle_out_proj_shard(const double* O_r, const float* Wo, double* Z_r,
                          int64_t n_rows, int64_t h, int H, int N, int r)
{
    if (N < 1 || r < 0 || r >= N || H < 1 || h % H != 0 || H % N != 0) return -1;
    const int64_t w = h / N;
    const float* Wo_r = Wo + (int64_t)r * w * h;  /* rows C_r of W_O are contiguous */
    linear_cols(O_r, w, Wo_r, h, NULL, Z_r, h, n_rows, w, 0, h);
    return 0;
}

/* Rank r's attention partial Z_r on the requested token rows (all rows if rows == NULL):
   projections, attention of the rank's heads, output projection. Only the keys a requested
   query can see are projected (causal: positions up to the latest requested one in its
   sequence). Optional outputs O_r [n_rows, h/N] (attention output before W_O). */
int oracle_attn_shard(const double* X, const float* Wq, const float* Wk, const float* Wv,
                      const float* bq, const float* bk, const float* bv, const float* Wo,
                      double* Z_r, double* O_r_out, int64_t batch, int64_t seq, int64_t h,
                      int H, int N, int r, int causal, const int64_t* rows, int64_t n_rows)
{
    if (N < 1 || r < 0 || r >= N || H < 1 || h % H != 0 || H % N != 0) return -1;
    if (batch < 1 || seq < 1) return -1;
    const int64_t T = batch * seq, w = h / N, d = h / H, lo = (int64_t)r * w;
    const int Hl = H / N;
    const int64_t nq = rows ? n_rows : T;
    /* Which key positions of each sequence are needed. */
    int64_t* need = (int64_t*)calloc((size_t)batch, sizeof(int64_t));   /* keys [0, need[b]) */
    for (int64_t i = 0; i < nq; ++i) {
        const int64_t t = rows ? rows[i] : i;
        if (t < 0 || t >= T) { free(need); return -1; }
        const int64_t b = t / seq, s = t % seq;
        const int64_t n = causal ? s + 1 : seq;
        if (n > need[b]) need[b] = n;
    }
    /* K and V of the needed positions, Q of the requested rows, laid out in full [T, w]. */
    double* Q = (double*)calloc((size_t)(T * w), sizeof(double));
    double* K = (double*)calloc((size_t)(T * w), sizeof(double));
    double* V = (double*)calloc((size_t)(T * w), sizeof(double));
    double* O = (double*)malloc(sizeof(double) * (size_t)(nq * w));
    if (!Q || !K || !V || !O) { free(need); free(Q); free(K); free(V); free(O); return -2; }
    for (int64_t b = 0; b < batch; ++b) {
        if (need[b] == 0) continue;
        const double* Xb = X + b * seq * h;
        linear_cols(Xb, h, Wk, h, bk, K + b * seq * w, w, need[b], h, lo, lo + w);
        linear_cols(Xb, h, Wv, h, bv, V + b * seq * w, w, need[b], h, lo, lo + w);
    }
    for (int64_t i = 0; i < nq; ++i) {
        const int64_t t = rows ? rows[i] : i;
        linear_cols(X + t * h, h, Wq, h, bq, Q + t * w, w, 1, h, lo, lo + w);
    }
    int rc = oracle_attention(Q, K, V, O, batch, seq, Hl, d, causal, rows, nq);
    if (rc == 0 && Z_r) rc = oracle_out_proj_shard(O, Wo, Z_r, nq, h, H, N, r);
    if (rc == 0 && O_r_out) memcpy(O_r_out, O, sizeof(double) * (size_t)(nq * w));
    free(need); free(Q); free(K); free(V); free(O);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* Partial sum (what the all-reduce computes): Z = sum_r Z_r, in fp64.                      */
/* ------------------------------------------------------------------------------------ */
int oracle_sum_partials(const float* parts, int n_parts, int64_t numel, double* Z)
{
    if (n_parts < 1 || numel < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < numel; ++i) {
        double s = 0.0;
        for (int p = 0; p < n_parts; ++p) s += (double)parts[(int64_t)p * numel + i];
        Z[i] = s;
    }
    return 0;
}

/* Product of two fp64 matrices (used by tests to compare projections). */
void oracle_matmul_dd(const double* X, const double* W, double* Y,
                      int64_t rows, int64_t in, int64_t out)
{
    linear_dd(X, in, W, out, Y, out, rows, in, out);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
