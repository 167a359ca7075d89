/*
 * oracle.c -- plain fp64 CPU reference for one tensor-parallel rank's Transformer-block shard.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and the
 * CPU-baseline leg of the benchmark load this library. The HIP product path never calls it,
 * and it shares no source, header or constant with that path.
 *
 * This file holds the oracle's element-wise and per-row steps; the linear layers (matrix
 * products, a library primitive) and the tensor-parallel slicing are in oracle/__init__.py.
 *   - GeLU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), the exact form. The pages name
 *     GeLU without a formula; the exact-erf form is the reading taken here.
 *   - Head = softmax(Q K^T / sqrt(d_k)) V for each head, query by query (llms.blog,
 *     "Partitioning Multi-Head and Grouped-Query Attention", step 2). Causal masking (key k
 *     visible to query i iff k <= i in the same sequence) is the configured variant;
 *     causal = 0 is the unmasked formula of that step.
 *   - The partial sum Y = sum_r Y_r that the all-reduce computes (llms.blog, "Row-Parallel
 *     Linear Layer", output and communication bullets).
 *   - GeLU'(x) = Phi(x) + x phi(x), the derivative of the exact form, for the backward pass
 *     of the MLP shard (llms.blog, "Partitioning the MLP Block": one all-reduce in the
 *     backward pass too).
 *   - SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x)), the gate of SwiGLU (llms.blog, MLP
 *     step 2: SiLU(X W_gate,i) * (X W_up,i)); the pages name SiLU without a formula.
 *   - LayerNorm of a row: (x - mean) / sqrt(var + eps) * gamma + beta, var the biased
 *     (1/n) variance (llms.blog, "Sequence Parallelism": LayerNorm runs on the s/N slice).
 *   - Grouped-query attention: query head j reads key/value head j / (H / H_kv) (llms.blog,
 *     "Grouped-Query Attention (GQA) Constraints").
 * All arithmetic is fp64. Token row t = b*seq + s.
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

/* d/dx [x Phi(x)] = Phi(x) + x phi(x), phi the standard normal density. */
double oracle_gelu_grad(double x)
{
    const double inv_sqrt_2pi = 0.39894228040143267794;
    return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * inv_sqrt_2pi * exp(-0.5 * x * x);
}

void oracle_gelu_grad_array(const double* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_gelu_grad(x[i]);
}

/* ------------------------------------------------------------------------------------ */
/* SiLU (the gate of SwiGLU) and LayerNorm                                                */
/* ------------------------------------------------------------------------------------ */
double oracle_silu(double x)
{
    return x / (1.0 + exp(-x));   /* x -> -inf: exp(-x) = inf and the quotient is -0 */
}

void oracle_silu_array(const double* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_silu(x[i]);
}

/* y[r] = (x[r] - mean) / sqrt(var + eps) * gamma + beta for each of `rows` rows of `cols`
   values; mean and the biased variance are taken over the row. */
int oracle_layernorm(const double* x, const double* gamma, const double* beta, double eps,
                     int64_t rows, int64_t cols, double* y)
{
    if (rows < 0 || cols < 1 || eps < 0.0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * cols;
        double mean = 0.0;
        for (int64_t c = 0; c < cols; ++c) mean += xr[c];
        mean /= (double)cols;
        double var = 0.0;
        for (int64_t c = 0; c < cols; ++c) var += (xr[c] - mean) * (xr[c] - mean);
        var /= (double)cols;
        const double inv = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < cols; ++c) y[r * cols + c] = (xr[c] - mean) * inv * gamma[c] + beta[c];
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Attention block                                                                         */
/* ------------------------------------------------------------------------------------ */

/* Softmax attention of n_heads heads of width d on token rows laid out t = b*seq + s.
   Q, K, V are [T, n_heads*d] (head j in columns j*d ... j*d+d-1). For each requested query
   row t (all T rows if rows == NULL) and each head, with s_k = <Q[t], K[b*seq+k]> / sqrt(d)
   over visible keys k (k <= s if causal, else all k < seq):
       O[t] = sum_k exp(s_k - m) V[b*seq+k] / sum_k exp(s_k - m),  m = max_k s_k.
   O is [n_rows, n_heads*d] in the order of `rows`: heads concatenated locally. */
/* Grouped-query form: K and V hold n_kv_heads heads ([T, n_kv_heads*d]); query head j reads
   key/value head j / (n_heads / n_kv_heads). n_kv_heads = n_heads is the multi-head case. */
int oracle_attention_gqa(const double* Q, const double* K, const double* V, double* O,
                         int64_t batch, int64_t seq, int n_heads, int n_kv_heads, int64_t d,
                         int causal, const int64_t* rows, int64_t n_rows)
{
    if (batch < 1 || seq < 1 || n_heads < 1 || d < 1) return -1;
    if (n_kv_heads < 1 || n_heads % n_kv_heads != 0) return -1;
    const int group = n_heads / n_kv_heads;
    const int64_t T = batch * seq, ld = (int64_t)n_heads * d, ldkv = (int64_t)n_kv_heads * d;
    int failed = 0;
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
            const int64_t kv = j / group;
            double* score = (double*)malloc(sizeof(double) * (size_t)n_keys);
            if (!score) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            double m = -INFINITY;
            for (int64_t k = 0; k < n_keys; ++k) {
                const double* kk = K + (b * seq + k) * ldkv + kv * d;
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
                const double* vv = V + (b * seq + k) * ldkv + kv * d;
                const double p = score[k] / denom;
                for (int64_t c = 0; c < d; ++c) o[c] += p * vv[c];
            }
            free(score);
        }
    }
    return failed ? -1 : 0;
}

int oracle_attention(const double* Q, const double* K, const double* V, double* O,
                     int64_t batch, int64_t seq, int n_heads, int64_t d, int causal,
                     const int64_t* rows, int64_t n_rows)
{
    return oracle_attention_gqa(Q, K, V, O, batch, seq, n_heads, n_heads, d, causal, rows,
                                n_rows);
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

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
