/*
 * CPU ORACLE for the DSA lightning indexer forward pass -- test
 * infrastructure only.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path never does.
 *
 * It is a plain, slow, obviously-correct restatement of the method, written
 * from the archdiff.com compare pages for Kimi K3.1 Pro (page "Qwen3.5 vs
 * Kimi K3.1 Pro", component table):
 *   - sparse/compressed-attention row: per MLA layer, H = 32, D = 128;
 *     q = c_q W_q with W_q [1536][4096]; one key vector per token,
 *     k = LayerNorm(x W_k) with W_k [7168][128], common to all heads;
 *     w = x W_w with W_w [7168][32]; I = sum_h w_h * ReLU(q_h . k); each
 *     query keeps 2,048 tokens;
 *   - QK-norm row: the LayerNorm is applied to k;
 *   - RoPE row of the "Kimi K3.1 Pro vs Gemma 4 31B" page: index_rope_dim = 0,
 *     so q and k are not rotated;
 *   - long-context row of that page: every key s <= t of the prefix is scored.
 *
 * Arithmetic: inputs are bf16 bit patterns widened exactly to double; every
 * sum runs in double in a fixed ascending order; the projected q, k, w are
 * rounded once, from double, to bf16 with round-to-nearest-even (own bit
 * level routine, no trip through float).  Top-k is a full sort of the row by
 * (score descending, index ascending) -- ties go to the lower token index --
 * after which the kept indices are listed in ascending order.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 * causal boundary s <= t (a query scores itself); short rows keep all t+1
 * tokens and pad with -1 / -inf; no score scale; no projection biases; the
 * LayerNorm is mean-centred with biased variance over the 128 key dims,
 * applied to the unrounded projection, with gain and bias; w has no
 * activation and may be negative; head h of q is columns [128h, 128h+128).
 *
 * FP8 key cache (a next step on the same pages: serving engines cache the
 * indexer keys in FP8, "Kimi K3.1 Pro vs GLM-5" page, low-precision row; the
 * pages give no FP8 format or scale, so the reading is stated here): OCP
 * E4M3 codes (bias 7, no infinities, 448 the largest finite value) with one
 * power-of-two scale per cached key (per query head for the query), the
 * smallest 2^e with max|x| <= 448 * 2^e, so that x / 2^e is exact and the
 * only rounding is round-to-nearest-even onto E4M3.  The score of the FP8
 * path is the same formula on the dequantised q and k, in double.
 *
 * Sparse MLA over the selected tokens (the consumer of the selection, a next step on the
 * same pages: "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page, gated-MLA row -- H = 96; cache row
 * = 512 latent + 64 position-key values = 576 per token; q/k head dim 192, v head dim 128;
 * query t attends to the <= 2,048 rows picked for it; no rotary step, RoPE row of the
 * "Kimi K3.1 Pro vs Gemma 4 31B" page).  The
 * reading: queries come in the absorbed latent form (the key up-projection folded into the
 * 128 no-position dims of each head, the 64 key-slot dims as they are), so head h's logit
 * for token s is scale * q~_h . kv[s] over the 576 cached values, the softmax runs over the
 * selected tokens only, and the head's output is the softmax-weighted sum of the 512-dim
 * latents (the value up-projection, the output gate and the output projection follow as
 * dense products).
 *
 * Shares no code, header or table with the HIP implementation.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- shapes of one indexer layer (sparse-attention row of the table) ---- */
enum {
    OR_HEADS = 32,     /* "32 heads" */
    OR_DIM = 128,      /* "x 128 dims" */
    OR_QLAT = 1536,    /* query latent width */
    OR_QOUT = 4096,    /* 1,536 -> 4,096 = 32 x 128 */
    OR_HIDDEN = 7168,  /* hidden width, 7,168 -> 32 for the head weights */
    OR_TOPK = 2048     /* "top 2,048 tokens per query" */
};

/* Number of weight elements one indexer layer holds under the readings above
 * (W_q, W_k, W_w, LayerNorm gain and bias; no projection biases). */
int64_t oracle_param_count(void) {
    return (int64_t)OR_QLAT * OR_QOUT      /* W_q */
         + (int64_t)OR_HIDDEN * OR_DIM     /* W_k */
         + (int64_t)OR_HIDDEN * OR_HEADS   /* W_w */
         + 2 * (int64_t)OR_DIM;            /* LayerNorm gain and bias */
}

/* Threads the OpenMP loops of this library use. */
int oracle_num_threads(void) { return omp_get_max_threads(); }

int oracle_dims(int32_t *out6) {
    out6[0] = OR_HEADS; out6[1] = OR_DIM; out6[2] = OR_QLAT;
    out6[3] = OR_QOUT; out6[4] = OR_HIDDEN; out6[5] = OR_TOPK;
    return 6;
}

/* ---------------- bf16 <-> double ---------------- */

/* Exact widening: a bf16 pattern is the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits, binary32 exponent
 * range, subnormals included), ties to even, in one step from the double.
 * Overflow goes to infinity.  NaN maps to the canonical quiet NaN. */
uint16_t oracle_f64_to_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    frexp(a, &e);                          /* a = m * 2^e, 0.5 <= m < 1 */
    int qexp = e - 8;                      /* 8 significant bits -> quantum 2^(e-8) */
    if (qexp < -133) qexp = -133;          /* bf16 subnormal quantum is 2^-133 */
    double scaled = ldexp(a, -qexp);       /* exact: power-of-two scaling */
    double r = floor(scaled);
    double frac = scaled - r;              /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double v = ldexp(r, qexp);             /* exactly representable in bf16 (or 2^128) */
    if (v >= 0x1p128) return sign | 0x7F80;
    float f = (float)v;                    /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

void oracle_f64_to_bf16_array(const double *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(x[i]);
}

/* ---------------- projections ---------------- */

/* out[r][j] = sum_{i < n_in, ascending} A[r][i] * W[i][j]  in double,
 * for r < rows.  A is bf16 [rows][lda], W is bf16 [n_in][n_out] row-major. */
void oracle_linear_f64(const uint16_t *A, int64_t lda, const uint16_t *W, int64_t n_in,
                       int64_t n_out, int64_t rows, double *out) {
    double *Wd = (double *)malloc(sizeof(double) * (size_t)(n_in * n_out));
    for (int64_t e = 0; e < n_in * n_out; ++e) Wd[e] = oracle_bf16_to_f64(W[e]);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        double *o = out + r * n_out;
        for (int64_t j = 0; j < n_out; ++j) o[j] = 0.0;
        for (int64_t i = 0; i < n_in; ++i) {
            double a = oracle_bf16_to_f64(A[r * lda + i]);
            const double *wr = Wd + i * n_out;
            for (int64_t j = 0; j < n_out; ++j) o[j] += a * wr[j];
        }
    }
    free(Wd);
}

/* LayerNorm over n values (the QK-norm row: a LayerNorm on the indexer key).
 * mu = mean(a), var = mean((a - mu)^2) (biased), out = (a - mu)/sqrt(var + eps)*g + b. */
void oracle_layernorm_f64(const double *a, int64_t n, const uint16_t *gamma,
                          const uint16_t *beta, double eps, double *out) {
    double mu = 0.0;
    for (int64_t j = 0; j < n; ++j) mu += a[j];
    mu /= (double)n;
    double var = 0.0;
    for (int64_t j = 0; j < n; ++j) var += (a[j] - mu) * (a[j] - mu);
    var /= (double)n;
    double inv = 1.0 / sqrt(var + eps);
    for (int64_t j = 0; j < n; ++j)
        out[j] = (a[j] - mu) * inv * oracle_bf16_to_f64(gamma[j]) + oracle_bf16_to_f64(beta[j]);
}

/* One indexer layer's projections for rows [0, rows):
 *   q[r]  = bf16( c_q[r] . W_q )                       [rows][4096]
 *   k[r]  = bf16( LayerNorm( x[r] . W_k ) )            [rows][128]
 *   w[r]  = bf16( x[r] . W_w )                         [rows][32]
 * Any of q/k/w may be NULL to skip it (c_q / x may then be NULL too). */
void oracle_project(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                    const uint16_t *Wq, const uint16_t *Wk, const uint16_t *Ww,
                    const uint16_t *gamma, const uint16_t *beta, double eps, int64_t rows,
                    uint16_t *q, uint16_t *k, uint16_t *w) {
    const int64_t chunk = 256;
    double *buf = (double *)malloc(sizeof(double) * (size_t)chunk * OR_QOUT);
    for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
        int64_t n = rows - r0 < chunk ? rows - r0 : chunk;
        if (q) {
            oracle_linear_f64(c_q + r0 * ldc, ldc, Wq, OR_QLAT, OR_QOUT, n, buf);
            oracle_f64_to_bf16_array(buf, n * OR_QOUT, q + r0 * OR_QOUT);
        }
        if (k) {
            oracle_linear_f64(x + r0 * ldx, ldx, Wk, OR_HIDDEN, OR_DIM, n, buf);
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < n; ++r) {
                double ln[OR_DIM];
                oracle_layernorm_f64(buf + r * OR_DIM, OR_DIM, gamma, beta, eps, ln);
                oracle_f64_to_bf16_array(ln, OR_DIM, k + (r0 + r) * OR_DIM);
            }
        }
        if (w) {
            oracle_linear_f64(x + r0 * ldx, ldx, Ww, OR_HIDDEN, OR_HEADS, n, buf);
            oracle_f64_to_bf16_array(buf, n * OR_HEADS, w + r0 * OR_HEADS);
        }
    }
    free(buf);
}

/* ---------------- scores ---------------- */

/* I[s] = sum_{h < H} w[h] * max(0, sum_{d < D} q[h][d] * k[s][d]),  s in [0, n).
 * q is bf16 [H][D] (head-major), w bf16 [H], k bf16 [n][D]; sums in double,
 * h and d ascending.  No rotary step (index_rope_dim = 0), no scale. */
void oracle_scores(const uint16_t *q, const uint16_t *w, const uint16_t *k, int64_t n,
                   int H, int D, double *I) {
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *wd = (double *)malloc(sizeof(double) * (size_t)H);
    double *kd = (double *)malloc(sizeof(double) * (size_t)D);
    for (int i = 0; i < H * D; ++i) qd[i] = oracle_bf16_to_f64(q[i]);
    for (int h = 0; h < H; ++h) wd[h] = oracle_bf16_to_f64(w[h]);
    for (int64_t s = 0; s < n; ++s) {
        for (int d = 0; d < D; ++d) kd[d] = oracle_bf16_to_f64(k[s * D + d]);
        double acc = 0.0;
        for (int h = 0; h < H; ++h) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qd[h * D + d] * kd[d];
            acc += wd[h] * (dot > 0.0 ? dot : 0.0);
        }
        I[s] = acc;
    }
    free(qd); free(wd); free(kd);
}

/* ---------------- selection ---------------- */

typedef struct { double v; int64_t i; } or_item;

/* Score descending, then index ascending: a strict total order, so the sort
 * result is the unique "stable" order the method's tie rule asks for.
 * -0.0 and +0.0 compare equal here (IEEE ==), so they tie. */
static int or_cmp_desc(const void *a, const void *b) {
    const or_item *x = (const or_item *)a, *y = (const or_item *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return x->i < y->i ? -1 : (x->i > y->i ? 1 : 0);
}

static int or_cmp_idx(const void *a, const void *b) {
    const or_item *x = (const or_item *)a, *y = (const or_item *)b;
    return x->i < y->i ? -1 : (x->i > y->i ? 1 : 0);
}

/* Top-k of I[0..n): keep the first min(topk, n) items of the full sort by
 * (score desc, index asc); list them by ascending index into idx/score,
 * padding with -1 / -inf up to topk.  tau = score of the topk-th item when
 * n > topk (else -inf); maxabs = max |I|. */
void oracle_topk(const double *I, int64_t n, int topk, int32_t *idx, double *score,
                 double *tau, double *maxabs) {
    or_item *it = (or_item *)malloc(sizeof(or_item) * (size_t)(n > 0 ? n : 1));
    double m = 0.0;
    for (int64_t s = 0; s < n; ++s) {
        it[s].v = I[s];
        it[s].i = s;
        if (fabs(I[s]) > m) m = fabs(I[s]);
    }
    qsort(it, (size_t)n, sizeof(or_item), or_cmp_desc);
    int64_t keep = n < topk ? n : topk;
    if (tau) *tau = n > topk ? it[topk - 1].v : -INFINITY;
    if (maxabs) *maxabs = m;
    qsort(it, (size_t)keep, sizeof(or_item), or_cmp_idx);
    for (int64_t j = 0; j < topk; ++j) {
        idx[j] = j < keep ? (int32_t)it[j].i : -1;
        score[j] = j < keep ? it[j].v : -INFINITY;
    }
    free(it);
}

/* ---------------- rows ---------------- */

/* For each listed row r (OpenMP over rows, caller orders them longest first):
 * query q_rows[r] ([H][D] bf16), weights w_rows[r] ([H] bf16), keys
 * k_base + k_off[r]*D .. (t[r] + 1 keys: the whole causal prefix, self
 * included).  Writes idx/score [nrows][topk], tau/maxabs [nrows], and, when
 * full is not NULL, the row's full score vector at full + full_off[r]. */
void oracle_rows(const uint16_t *q_rows, const uint16_t *w_rows, const uint16_t *k_base,
                 const int64_t *k_off, const int64_t *t, int64_t nrows, int H, int D, int topk,
                 int32_t *idx, double *score, double *tau, double *maxabs, double *full,
                 const int64_t *full_off) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t n = t[r] + 1;
        double *I = full ? full + full_off[r] : (double *)malloc(sizeof(double) * (size_t)n);
        oracle_scores(q_rows + r * (int64_t)H * D, w_rows + r * (int64_t)H, k_base + k_off[r] * D,
                      n, H, D, I);
        oracle_topk(I, n, topk, idx + r * (int64_t)topk, score + r * (int64_t)topk, tau + r,
                    maxabs + r);
        if (!full) free(I);
    }
}

/* ---------------- FP8 (OCP E4M3) key cache ---------------- */

/* Value of an E4M3 code: sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 holds the subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN. */
double oracle_e4m3_to_f64(uint8_t c) {
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e ? ldexp(8.0 + m, e - 10) : ldexp((double)m, -9);
    return sgn ? -mag : mag;
}

/* Nearest E4M3 code to x (ties to the even code), for |x| <= 448.  The codes
 * of one sign are in value order, so the magnitude is located by walking the
 * binades: in binade [2^E, 2^(E+1)), E >= -6, the 8 codes are spaced 2^(E-3);
 * below 2^-6 the subnormals are spaced 2^-9.  x/spacing is exact in double. */
uint8_t oracle_f64_to_e4m3(double x) {
    const uint8_t sgn = (signbit(x) ? 0x80 : 0x00);
    const double a = fabs(x);
    int E = -6;                       /* binade of a, at least the subnormal one */
    while (E < 8 && a >= ldexp(1.0, E + 1)) ++E;
    const double unit = ldexp(1.0, E - 3);
    const double n = a / unit;        /* in [0, 16) */
    double r = floor(n);
    const double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    /* code magnitude: codes below 8 are the subnormals (n < 8 when E = -6 and
     * a < 2^-6); in binade E the codes are 8 (E + 6) + r, r in [8, 16] */
    int mag;
    if (a < ldexp(1.0, -6)) mag = (int)r;              /* r in [0, 8]: 8 is 2^-6 */
    else mag = 8 * (E + 6) + (int)r;
    return (uint8_t)(sgn | mag);
}

/* Smallest integer e with amax <= 448 * 2^e (amax > 0; 0 for amax = 0). */
int oracle_pow2_scale_exp(double amax) {
    if (!(amax > 0.0)) return 0;
    int e = 0;
    while (amax > 448.0 * ldexp(1.0, e)) ++e;
    while (amax <= 448.0 * ldexp(1.0, e - 1)) --e;
    return e;
}

/* Quantise n vectors of d bf16 values: codes[i][j] = E4M3(x[i][j] / 2^e_i),
 * e_i = oracle_pow2_scale_exp(max_j |x[i][j]|). */
void oracle_quantize_e4m3(const uint16_t *x, int64_t n, int d, uint8_t *codes, int32_t *exps) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double amax = 0.0;
        for (int j = 0; j < d; ++j) {
            const double v = fabs(oracle_bf16_to_f64(x[i * d + j]));
            if (v > amax) amax = v;
        }
        const int e = oracle_pow2_scale_exp(amax);
        exps[i] = e;
        for (int j = 0; j < d; ++j)
            codes[i * d + j] = oracle_f64_to_e4m3(ldexp(oracle_bf16_to_f64(x[i * d + j]), -e));
    }
}

/* FP8 decode rows: row r has query codes qc [H][D] with per-head exponents qe [H], bf16
 * weights w [H], and scores the cached keys kc[(k_off[r] + s) * D ..] (exponent ke[..]) for
 * s <= t[r]:  I[s] = 2^ke[s] * sum_h w[h] 2^qe[h] max(0, sum_d dq[h][d] dk[s][d]), with
 * dq, dk the E4M3 values, in double.  Selection as oracle_rows. */
void oracle_rows_fp8(const uint8_t *qc, const int32_t *qe, const uint16_t *w_rows,
                     const uint8_t *kc, const int32_t *ke, const int64_t *k_off, const int64_t *t,
                     int64_t nrows, int H, int D, int topk, int32_t *idx, double *score,
                     double *tau, double *maxabs, double *full, const int64_t *full_off) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t n = t[r] + 1;
        double *I = full ? full + full_off[r] : (double *)malloc(sizeof(double) * (size_t)n);
        double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
        double *kd = (double *)malloc(sizeof(double) * (size_t)D);
        double *wq = (double *)malloc(sizeof(double) * (size_t)H);
        for (int i = 0; i < H * D; ++i) qd[i] = oracle_e4m3_to_f64(qc[r * (int64_t)H * D + i]);
        for (int h = 0; h < H; ++h)
            wq[h] = oracle_bf16_to_f64(w_rows[r * (int64_t)H + h]) * ldexp(1.0, qe[r * (int64_t)H + h]);
        for (int64_t s = 0; s < n; ++s) {
            const int64_t row = k_off[r] + s;
            for (int d = 0; d < D; ++d) kd[d] = oracle_e4m3_to_f64(kc[row * D + d]);
            double acc = 0.0;
            for (int h = 0; h < H; ++h) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qd[h * D + d] * kd[d];
                acc += wq[h] * (dot > 0.0 ? dot : 0.0);
            }
            I[s] = ldexp(acc, ke[row]);
        }
        oracle_topk(I, n, topk, idx + r * (int64_t)topk, score + r * (int64_t)topk, tau + r,
                    maxabs + r);
        free(qd); free(kd); free(wq);
        if (!full) free(I);
    }
}

/* ---- sparse MLA over the selected tokens ----
 * q [T][H][576] bf16 (absorbed queries), kv [*][576] bf16 (cache rows: 512-dim latent, then
 * the 64-dim key slot), idx [T][K] int32 (selected rows relative to row0[t]; -1 = no token),
 * row0 [T] (NULL: 0).  For query t and head h, over the valid selections j:
 *   z_j = scale * sum_d q[t][h][d] kv[r_j][d]
 *   o[t][h][:] = sum_j exp(z_j - m) kv[r_j][0:512] / sum_j exp(z_j - m),   m = max_j z_j
 *   lse[t][h] = m + log(sum_j exp(z_j - m))
 * in double, j ascending.  No valid selection: o = 0, lse = -inf. */
enum { OR_MLA_KV = 576, OR_MLA_V = 512 };
void oracle_sparse_mla(const uint16_t *q, const uint16_t *kv, const int32_t *idx, const int64_t *row0,
                       int64_t T, int H, int K, double scale, double *o, double *lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        double *z = (double *)malloc(sizeof(double) * (size_t)K);
        double *qd = (double *)malloc(sizeof(double) * OR_MLA_KV);
        for (int h = 0; h < H; ++h) {
            const uint16_t *qh = q + ((size_t)t * H + h) * OR_MLA_KV;
            for (int d = 0; d < OR_MLA_KV; ++d) qd[d] = oracle_bf16_to_f64(qh[d]);
            double m = -INFINITY;
            for (int j = 0; j < K; ++j) {
                const int32_t s = idx[t * (int64_t)K + j];
                if (s < 0) continue;
                const uint16_t *kr = kv + (size_t)((row0 ? row0[t] : 0) + s) * OR_MLA_KV;
                double dot = 0.0;
                for (int d = 0; d < OR_MLA_KV; ++d) dot += qd[d] * oracle_bf16_to_f64(kr[d]);
                z[j] = scale * dot;
                if (z[j] > m) m = z[j];
            }
            double *oh = o + ((size_t)t * H + h) * OR_MLA_V;
            for (int d = 0; d < OR_MLA_V; ++d) oh[d] = 0.0;
            if (m == -INFINITY) {
                lse[t * H + h] = -INFINITY;
                continue;
            }
            double l = 0.0;
            for (int j = 0; j < K; ++j) {
                const int32_t s = idx[t * (int64_t)K + j];
                if (s < 0) continue;
                const double p = exp(z[j] - m);
                const uint16_t *kr = kv + (size_t)((row0 ? row0[t] : 0) + s) * OR_MLA_KV;
                for (int d = 0; d < OR_MLA_V; ++d) oh[d] += p * oracle_bf16_to_f64(kr[d]);
                l += p;
            }
            for (int d = 0; d < OR_MLA_V; ++d) oh[d] /= l;
            lse[t * H + h] = m + log(l);
        }
        free(z);
        free(qd);
    }
}
