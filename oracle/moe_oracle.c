/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle of the fused MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, table or constant with the HIP path.
 *
 * Sources (web pages; cited by title and section):
 *   [P3] "Mixture-of-Experts kernel engineering on Amazon SageMaker AI"
 *        (summary text): a fused MoE merges token routing, data shuffling
 *        and the expert network computations into one batched GPU op in
 *        place of sequential per-expert loops; the expert GEMM is
 *        C = A.B with A the tokens [M,K] and B the expert weights [K,N];
 *        the Swap-AB passage (Figure 1) states C^T[N,M] = B^T[N,K].A^T[K,M],
 *        so weights are held output-major as B^T[N,K]; the FP8 passage
 *        names FP8 tensor scaling, matrix multiplication and expert
 *        aggregation as the steps a one-pass backend fuses, for FP8
 *        tensor-quantized (per-tensor scale) models.
 *   [P2] "«До 10% пропускной способности и 9% к TTFT»: AWS раскрыла
 *        оптимизации ядер MoE на SageMaker AI", sections "Зачем
 *        оптимизировать ядра MoE" (same definition of fused MoE) and
 *        "Triton вместо CUTLASS для FP8-квантования".
 *   [P4] "AI混合专家模型性能优化全链路解析", chapter 1, dynamic expert load
 *        balancing: experts are picked by top-k over router logits.
 *
 * What the oracle computes is the per-token expert loop that the fusion
 * only reorders ([P3] summary, fused-MoE definition):
 *
 *   out[t] = sum_{j<k} w[t,j] * W2[e_tj] . ( silu(W1[e_tj][0:N] . x_t)
 *                                            * (W1[e_tj][N:2N] . x_t) )
 *
 * The pages leave open the expert MLP's form, the gating details and the
 * FP8 quantisation points.  The readings taken here (each one also listed
 * in the design notes) are:
 *   R1 logits are the fp32 rounding of the fp64 dot product x_t . W_r[e]
 *      (+ bias[e] when a bias is given); every bf16*bf16 product is exact
 *      in fp64.
 *   R2 top-k selects the k largest fp32 logits, ties to the lower expert id,
 *      slots in descending-logit order; selecting on logits equals selecting
 *      on softmax probabilities since softmax is strictly increasing.
 *   R3 routing weights are the softmax over all E renormalised over the k
 *      selected, i.e. w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0).
 *   R4 W1[e] rows [0,N) are the gate, rows [N,2N) the up projection;
 *      silu(z) = z / (1 + exp(-z)).
 *   R5 the permutation is a stable counting sort of p = t*k + j by expert,
 *      each expert's segment padded to a multiple of the block size with
 *      the sentinel M*k.
 *   R6 FP8 is OCP E4M3FN (bias 7, max 448, no infinities, NaN 0x7F/0xFF),
 *      encoded round-to-nearest-even after clamping to +-448.
 *   R7 FP8 activations are quantised per token (x) and per token-slot (the
 *      SiLU*up activation), each with scale s = fp32(amax)/448 (1 if
 *      amax = 0), code = E4M3(fp32(v) / s) with one correctly-rounded fp32
 *      division; weight scales are per expert tensor.
 *   R8 (a scheme the pages do not describe; the per-tensor one generalised)
 *      per-channel weight scales: one fp32 scale per output row of each
 *      expert's W1 (2N rows, gate then up) and W2 (K rows), multiplying that
 *      row's dot products where R7 multiplies by the tensor's scale.
 *   R9 (also beyond the pages) MXFP4 weights, OCP microscaling: e2m1
 *      elements (sign, 2 exponent bits with bias 1, 1 mantissa bit; exponent
 *      0 is subnormal: 0 or 0.5) packed two per byte, the even element of a
 *      row in the low nibble, and one E8M0 scale 2^(e-127) (e = 255: NaN) per
 *      32 consecutive elements of a row along the reduction dimension; a
 *      weight is its element times its block's scale.  Activations as R7.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_MISSING_EXPERT 2
#define ORC_ERR_NOMEM 3

/* ---------------------------------------------------------------------- */
/* Number formats                                                          */
/* ---------------------------------------------------------------------- */

/* bf16 is the top half of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP E4M3FN decode (R6): sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: m/8 * 2^-6.  S.1111.111 is NaN. */
double orc_e4m3_to_f64(uint8_t c)
{
    int s = c >> 7;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP E4M3FN encode of an fp32 value (R6): nearest representable value,
 * ties to the even mantissa, magnitudes clamped to 448 first.  All the
 * arithmetic below is exact in double (power-of-two scalings of a float,
 * then rint in the default round-half-even mode). */
uint8_t orc_f32_to_e4m3(float f)
{
    double a;
    int sign, ex;
    double q;
    if (isnan(f))
        return 0x7F;
    sign = signbit(f) ? 0x80 : 0;
    a = fabs((double)f);
    if (a > 448.0)
        a = 448.0;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: grid step 2^-9; q == 8 is the smallest normal,
         * whose code is also 8. */
        q = rint(a * 512.0);
        return (uint8_t)(sign | (int)q);
    }
    frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
    ex -= 1;                /* a in [2^ex, 2^(ex+1)), ex in [-6, 8] */
    q = rint(ldexp(a, 3 - ex)); /* mantissa incl. hidden bit, in [8, 16] */
    if (q == 16.0) {
        q = 8.0;
        ex += 1;
    }
    return (uint8_t)(sign | ((ex + 7) << 3) | ((int)q - 8));
}

/* Decode table of the 256 codes, filled once from orc_e4m3_to_f64 so the
 * expert loops do not re-derive every code. */
static double e4m3_table[256];
static int e4m3_table_ready = 0;

static void init_e4m3_table(void)
{
    int c;
    if (e4m3_table_ready)
        return;
    for (c = 0; c < 256; ++c)
        e4m3_table[c] = orc_e4m3_to_f64((uint8_t)c);
    e4m3_table_ready = 1;
}

/* Per-row dynamic quantisation (R7) of n fp32 values. */
static void quant_row_f32(const float *v, int64_t n, uint8_t *q, float *scale)
{
    float amax = 0.0f, s;
    int64_t i;
    for (i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    for (i = 0; i < n; ++i) {
        float r = v[i] / s;
        q[i] = orc_f32_to_e4m3(r);
    }
    *scale = s;
}

/* ---------------------------------------------------------------------- */
/* Gating                                                                  */
/* ---------------------------------------------------------------------- */

/* R1: logits[t,e] = fp32( sum_k x[t,k]*wr[e,k] + bias[e] ), k ascending. */
int orc_logits(const uint16_t *x, const uint16_t *wr, const float *bias,
               int64_t M, int64_t K, int64_t E, float *logits)
{
    int64_t t;
    if (M < 0 || K <= 0 || E <= 0 || (M > 0 && (!x || !wr || !logits)))
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (t = 0; t < M; ++t) {
        int64_t e, k;
        for (e = 0; e < E; ++e) {
            double acc = 0.0;
            for (k = 0; k < K; ++k)
                acc += orc_bf16_to_f64(x[t * K + k]) * orc_bf16_to_f64(wr[e * K + k]);
            if (bias)
                acc += (double)bias[e];
            logits[t * E + e] = (float)acc;
        }
    }
    return ORC_OK;
}

/* R2 + R3 on given fp32 logits: ids[t,j] int32 and weights[t,j] fp64. */
int orc_topk(const float *logits, int64_t M, int64_t E, int64_t k,
             int32_t *ids, double *weights)
{
    int64_t t;
    if (M < 0 || E <= 0 || k < 1 || k > E || (M > 0 && (!logits || !ids)))
        return ORC_ERR_ARG;
    for (t = 0; t < M; ++t) {
        const float *l = logits + t * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        double den = 0.0, l0;
        int64_t j, e;
        if (!taken)
            return ORC_ERR_NOMEM;
        for (j = 0; j < k; ++j) {
            int64_t best = -1;
            for (e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                /* strict '>' keeps the lower id on equal logits */
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
        }
        free(taken);
        if (weights) {
            l0 = (double)l[ids[t * k]];
            for (j = 0; j < k; ++j)
                den += exp((double)l[ids[t * k + j]] - l0);
            for (j = 0; j < k; ++j)
                weights[t * k + j] = exp((double)l[ids[t * k + j]] - l0) / den;
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* Expert-sorted permutation (R5)                                           */
/* ---------------------------------------------------------------------- */

/* Capacity of sorted_ids: M*k + E*(B-1); of block_expert: capacity / B.
 * Positions past num_padded hold the sentinel M*k and blocks past the last
 * used one hold -1. */
int orc_align(const int32_t *ids, int64_t M, int64_t k, int64_t E, int64_t B,
              int32_t *sorted_ids, int32_t *block_expert,
              int32_t *expert_offsets, int32_t *num_padded)
{
    int64_t n = M * k, cap, nblk, e, p, i;
    int64_t *count, *fill;
    if (M < 0 || k < 1 || E <= 0 || B < 1)
        return ORC_ERR_ARG;
    cap = n + E * (B - 1);
    nblk = cap / B;
    count = (int64_t *)calloc((size_t)E, sizeof *count);
    fill = (int64_t *)calloc((size_t)E, sizeof *fill);
    if (!count || !fill) {
        free(count);
        free(fill);
        return ORC_ERR_NOMEM;
    }
    for (p = 0; p < n; ++p) {
        if (ids[p] < 0 || ids[p] >= E) {
            free(count);
            free(fill);
            return ORC_ERR_ARG;
        }
        count[ids[p]]++;
    }
    expert_offsets[0] = 0;
    for (e = 0; e < E; ++e) {
        int64_t padded = (count[e] + B - 1) / B * B;
        expert_offsets[e + 1] = (int32_t)(expert_offsets[e] + padded);
    }
    *num_padded = expert_offsets[E];
    for (i = 0; i < cap; ++i)
        sorted_ids[i] = (int32_t)n;
    for (p = 0; p < n; ++p) {     /* ascending p: stable within an expert */
        e = ids[p];
        sorted_ids[expert_offsets[e] + fill[e]] = (int32_t)p;
        fill[e]++;
    }
    for (i = 0; i < nblk; ++i)
        block_expert[i] = -1;
    for (e = 0; e < E; ++e)
        for (i = expert_offsets[e] / B; i < expert_offsets[e + 1] / B; ++i)
            block_expert[i] = (int32_t)e;
    free(count);
    free(fill);
    return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* Expert MLP and combine                                                   */
/* ---------------------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* The expert MLP of one token-slot is written as two steps, so that the
 * host's threads can share the work of a single slot: the activation
 * element n (a function of the token row and two W1 rows) and the output
 * element c (a function of the whole activation row and one W2 row).  Each
 * element is one fixed-order fp64 sum, computed by one thread. */

/* bf16 weights: act[n] = silu(W1g[n].x) * (W1u[n].x). */
static double act_bf16(const uint16_t *xt, const uint16_t *w1, int64_t K, int64_t N, int64_t n)
{
    const uint16_t *g = w1 + n * K;
    const uint16_t *u = w1 + (N + n) * K;
    double hg = 0.0, hu = 0.0;
    int64_t kk;
    for (kk = 0; kk < K; ++kk) {
        double xv = orc_bf16_to_f64(xt[kk]);
        hg += orc_bf16_to_f64(g[kk]) * xv;
        hu += orc_bf16_to_f64(u[kk]) * xv;
    }
    return silu(hg) * hu;
}

/* bf16 weights: y[c] = W2[c] . act. */
static double out_bf16(const double *act, const uint16_t *w2, int64_t N, int64_t c)
{
    const uint16_t *r = w2 + c * N;
    double acc = 0.0;
    int64_t n;
    for (n = 0; n < N; ++n)
        acc += orc_bf16_to_f64(r[n]) * act[n];
    return acc;
}

/* e4m3 weights, token codes xq with scale sx: per-tensor scales (R7,
 * rs = 0: every row reads w1s[0] / w2s[0]) or per-channel scales (R8,
 * rs = 1: row r reads w1s[r] / w2s[r]). */
static double act_fp8(const uint8_t *xq, float sx, const uint8_t *w1, const float *w1s,
                      int64_t rs, int64_t K, int64_t N, int64_t n)
{
    const uint8_t *g = w1 + n * K;
    const uint8_t *u = w1 + (N + n) * K;
    double hg = 0.0, hu = 0.0;
    int64_t kk;
    for (kk = 0; kk < K; ++kk) {
        double xv = e4m3_table[xq[kk]];
        hg += e4m3_table[g[kk]] * xv;
        hu += e4m3_table[u[kk]] * xv;
    }
    hg *= (double)sx * (double)w1s[n * rs];
    hu *= (double)sx * (double)w1s[(N + n) * rs];
    return silu(hg) * hu;
}

/* e4m3 weights: y[c] = sa * w2s . (W2[c] . act codes aq). */
static double out_fp8(const uint8_t *aq, float sa, const uint8_t *w2, const float *w2s,
                      int64_t rs, int64_t N, int64_t c)
{
    const uint8_t *r = w2 + c * N;
    double acc = 0.0;
    int64_t n;
    for (n = 0; n < N; ++n)
        acc += e4m3_table[r[n]] * e4m3_table[aq[n]];
    return acc * (double)sa * (double)w2s[c * rs];
}

/* e2m1 code (low 4 bits) -> value, from the format's definition (R9). */
double orc_e2m1_to_f64(uint8_t c)
{
    int sgn = (c >> 3) & 1, ex = (c >> 1) & 3, man = c & 1;
    double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return sgn ? -v : v;
}

/* E8M0 scale byte -> 2^(e-127); 255 is NaN (R9). */
double orc_e8m0_to_f64(uint8_t e)
{
    return e == 255 ? NAN : ldexp(1.0, (int)e - 127);
}

/* Weight r,k of an MXFP4 matrix with `cols` elements per row (R9). */
static double mx_weight(const uint8_t *w, const uint8_t *sc, int64_t cols, int64_t r, int64_t k)
{
    uint8_t byte = w[r * (cols / 2) + k / 2];
    uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    return orc_e2m1_to_f64(code) * orc_e8m0_to_f64(sc[r * (cols / 32) + k / 32]);
}

/* MXFP4 weights (R9): w1 [2N, K/2] packed with scales s1 [2N, K/32];
 * act[n] from the token codes xq with scale sx. */
static double act_mxfp4(const uint8_t *xq, float sx, const uint8_t *w1, const uint8_t *s1,
                        int64_t K, int64_t N, int64_t n)
{
    double hg = 0.0, hu = 0.0;
    int64_t kk;
    for (kk = 0; kk < K; ++kk) {
        double xv = e4m3_table[xq[kk]];
        hg += mx_weight(w1, s1, K, n, kk) * xv;
        hu += mx_weight(w1, s1, K, N + n, kk) * xv;
    }
    hg *= (double)sx;
    hu *= (double)sx;
    return silu(hg) * hu;
}

/* MXFP4 weights: w2 [K, N/2] with scales s2 [K, N/32]; y[c] from the
 * activation codes aq with scale sa. */
static double out_mxfp4(const uint8_t *aq, float sa, const uint8_t *w2, const uint8_t *s2,
                        int64_t N, int64_t c)
{
    double acc = 0.0;
    int64_t n;
    for (n = 0; n < N; ++n)
        acc += mx_weight(w2, s2, N, c, n) * e4m3_table[aq[n]];
    return acc * (double)sa;
}

/* Per-token dynamic quantisation of bf16 rows (R7): xq [M,K], sx [M]. */
int orc_quant_rows_bf16(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq, float *sx)
{
    int64_t t;
    float *row;
    if (M < 0 || K <= 0)
        return ORC_ERR_ARG;
    row = (float *)malloc((size_t)K * sizeof *row);
    if (!row)
        return ORC_ERR_NOMEM;
    for (t = 0; t < M; ++t) {
        int64_t k;
        for (k = 0; k < K; ++k)
            row[k] = bf16_to_f32(x[t * K + k]);
        quant_row_f32(row, K, xq + t * K, sx + t);
    }
    free(row);
    return ORC_OK;
}

/* Per-row dynamic quantisation of fp32 rows (R7), exported for the pins. */
int orc_quant_rows_f32(const float *v, int64_t M, int64_t K, uint8_t *q, float *s)
{
    int64_t t;
    if (M < 0 || K <= 0)
        return ORC_ERR_ARG;
    for (t = 0; t < M; ++t)
        quant_row_f32(v + t * K, K, q + t * K, s + t);
    return ORC_OK;
}

/*
 * The whole layer for a list of tokens.
 *
 *   dtype     0 = bf16 weights, 1 = e4m3 weights with fp32 w1s/w2s [E] (one
 *             scale per expert tensor), 2 = e4m3 weights with fp32
 *             per-channel scales w1s [E,2N], w2s [E,K] (R8), 3 = MXFP4
 *             weights (w1[e] [2N,K/2], w2[e] [K,N/2] packed) with E8M0 byte
 *             scales w1s [E,2N,K/32], w2s [E,K,N/32] (R9)
 *   x         bf16 [M,K] (all tokens: routing of token t reads row t only)
 *   wr        bf16 [E,K]; bias fp32 [E] or NULL
 *   w1[e]     expert e's W1 [2N,K] (bf16 or e4m3), NULL if not provided
 *   w2[e]     expert e's W2 [K,N]
 *   tokens    the n_tok token indices to evaluate (each in [0,M))
 *   out       fp64 [n_tok, K]
 *   ids_out   int32 [n_tok, k] or NULL; wts_out fp64 [n_tok, k] or NULL
 *
 * Returns ORC_ERR_MISSING_EXPERT if a selected expert's weights are NULL.
 * The threads share the (slot, element) pairs of each step; every element
 * is one fixed-order sum written by one thread, and the combine then sums
 * the k slots of a token in ascending j, so results do not depend on the
 * thread count.
 */
int orc_moe_forward(int dtype, const uint16_t *x, const uint16_t *wr, const float *bias,
                    const void *const *w1, const void *const *w2,
                    const void *w1s, const void *w2s,
                    int64_t M, int64_t K, int64_t N, int64_t E, int64_t k,
                    const int64_t *tokens, int64_t n_tok,
                    double *out, int32_t *ids_out, double *wts_out)
{
    int64_t i, nslot = n_tok * k;
    int32_t *ids = NULL;
    double *wts = NULL, *y = NULL, *act = NULL;
    float *lg = NULL, *sx = NULL, *sa = NULL;
    uint8_t *xq = NULL, *aq = NULL;
    int rc = ORC_OK;
    const int quant = dtype != 0;
    if (dtype < 0 || dtype > 3 || M < 0 || K <= 0 || N <= 0 || E <= 0 ||
        k < 1 || k > E || n_tok < 0 || !x || !wr || !w1 || !w2 || !out ||
        (n_tok > 0 && !tokens) || (dtype != 0 && (!w1s || !w2s)) ||
        (dtype == 3 && (K % 32 || N % 32)))
        return ORC_ERR_ARG;
    for (i = 0; i < n_tok; ++i)
        if (tokens[i] < 0 || tokens[i] >= M)
            return ORC_ERR_ARG;
    init_e4m3_table();
    {
        const size_t ns = (size_t)(nslot > 0 ? nslot : 1), nt = (size_t)(n_tok > 0 ? n_tok : 1);
        ids = (int32_t *)malloc(ns * sizeof *ids);
        wts = (double *)malloc(ns * sizeof *wts);
        lg = (float *)malloc(nt * (size_t)E * sizeof *lg);
        y = (double *)malloc(ns * (size_t)K * sizeof *y);
        act = (double *)malloc(ns * (size_t)N * sizeof *act);
        if (quant) {
            xq = (uint8_t *)malloc(nt * (size_t)K);
            sx = (float *)malloc(nt * sizeof *sx);
            aq = (uint8_t *)malloc(ns * (size_t)N);
            sa = (float *)malloc(ns * sizeof *sa);
        }
    }
    if (!ids || !wts || !lg || !y || !act || (quant && (!xq || !sx || !aq || !sa))) {
        rc = ORC_ERR_NOMEM;
        goto done;
    }
    /* gating for the chosen tokens (R1-R3) */
    for (i = 0; i < n_tok; ++i) {
        rc = orc_logits(x + tokens[i] * K, wr, bias, 1, K, E, lg + i * E);
        if (rc)
            goto done;
    }
    rc = orc_topk(lg, n_tok, E, k, ids, wts);
    if (rc)
        goto done;
    for (i = 0; i < nslot; ++i)
        if (!w1[ids[i]] || !w2[ids[i]]) {
            rc = ORC_ERR_MISSING_EXPERT;
            goto done;
        }
    /* FP8 and MXFP4: the per-token e4m3 codes of the token rows (R7) */
    if (quant) {
        rc = ORC_OK;
#pragma omp parallel
        {
            float *xrow = (float *)malloc((size_t)K * sizeof *xrow);
            int64_t t, kk;
            if (!xrow) {
#pragma omp atomic write
                rc = ORC_ERR_NOMEM;
            }
#pragma omp for schedule(static)
            for (t = 0; t < n_tok; ++t) {
                if (!xrow)
                    continue;
                for (kk = 0; kk < K; ++kk)
                    xrow[kk] = bf16_to_f32(x[tokens[t] * K + kk]);
                quant_row_f32(xrow, K, xq + t * K, sx + t);
            }
            free(xrow);
        }
        if (rc)
            goto done;
    }
    /* the SiLU*up activation of every (slot, n) */
    {
        int64_t idx;
#pragma omp parallel for schedule(static)
        for (idx = 0; idx < nslot * N; ++idx) {
            const int64_t s = idx / N, n = idx % N, tt = s / k;
            const int e = ids[s];
            double v;
            if (dtype == 0)
                v = act_bf16(x + tokens[tt] * K, (const uint16_t *)w1[e], K, N, n);
            else if (dtype == 1)
                v = act_fp8(xq + tt * K, sx[tt], (const uint8_t *)w1[e], (const float *)w1s + e,
                            0, K, N, n);
            else if (dtype == 2)
                v = act_fp8(xq + tt * K, sx[tt], (const uint8_t *)w1[e],
                            (const float *)w1s + e * 2 * N, 1, K, N, n);
            else
                v = act_mxfp4(xq + tt * K, sx[tt], (const uint8_t *)w1[e],
                              (const uint8_t *)w1s + e * 2 * N * (K / 32), K, N, n);
            act[idx] = v;
        }
    }
    /* FP8 and MXFP4: per token-slot e4m3 codes of the activation, quantised
     * from its fp64 value rounded to fp32 (R7) */
    if (quant) {
        rc = ORC_OK;
#pragma omp parallel
        {
            float *row = (float *)malloc((size_t)N * sizeof *row);
            int64_t s, n;
            if (!row) {
#pragma omp atomic write
                rc = ORC_ERR_NOMEM;
            }
#pragma omp for schedule(static)
            for (s = 0; s < nslot; ++s) {
                if (!row)
                    continue;
                for (n = 0; n < N; ++n)
                    row[n] = (float)act[s * N + n];
                quant_row_f32(row, N, aq + s * N, sa + s);
            }
            free(row);
        }
        if (rc)
            goto done;
    }
    /* the expert output of every (slot, c) */
    {
        int64_t idx;
#pragma omp parallel for schedule(static)
        for (idx = 0; idx < nslot * K; ++idx) {
            const int64_t s = idx / K, c = idx % K;
            const int e = ids[s];
            double v;
            if (dtype == 0)
                v = out_bf16(act + s * N, (const uint16_t *)w2[e], N, c);
            else if (dtype == 1)
                v = out_fp8(aq + s * N, sa[s], (const uint8_t *)w2[e], (const float *)w2s + e, 0,
                            N, c);
            else if (dtype == 2)
                v = out_fp8(aq + s * N, sa[s], (const uint8_t *)w2[e],
                            (const float *)w2s + e * K, 1, N, c);
            else
                v = out_mxfp4(aq + s * N, sa[s], (const uint8_t *)w2[e],
                              (const uint8_t *)w2s + e * K * (N / 32), N, c);
            y[idx] = v;
        }
    }

    /* weighted combine, slots in ascending j */
    for (i = 0; i < n_tok; ++i) {
        int64_t c, j;
        for (c = 0; c < K; ++c) {
            double acc = 0.0;
            for (j = 0; j < k; ++j)
                acc += wts[i * k + j] * y[(i * k + j) * K + c];
            out[i * K + c] = acc;
        }
    }
    if (ids_out)
        memcpy(ids_out, ids, (size_t)nslot * sizeof *ids);
    if (wts_out)
        memcpy(wts_out, wts, (size_t)nslot * sizeof *wts);
done:
    free(ids);
    free(wts);
    free(lg);
    free(y);
    free(act);
    free(xq);
    free(sx);
    free(aq);
    free(sa);
    return rc;
}

/* Number of threads an OpenMP parallel region will use. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
