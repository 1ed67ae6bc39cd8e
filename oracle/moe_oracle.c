/*
 * moe_oracle.c -- plain CPU reference for the DeepSeekMoE layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, loads or calls it, and the two share no source, header or table.
 *
 * Sources (DeepSeek-V3 Technical Report, as rewritten on the "papers-reader"
 * page "DeepSeek-V3 Technical Report"):
 *   - §2.1.2 DeepSeekMoE: output = shared experts applied to every token plus
 *     the gate-weighted sum of the K_r selected routed experts; affinities are
 *     sigmoid(u_t . e_i) and the gating values are the selected affinities
 *     normalised among the selected experts.
 *   - §2.1.2 auxiliary-loss-free balancing: a per-expert bias b_i is added to
 *     the affinity for the top-K choice only; the gate uses the un-biased
 *     affinity; after each step b_i moves by gamma against the expert's
 *     whole-batch load; node-limited routing keeps each token on at most M
 *     groups of experts; no token is dropped.
 *   - §3.3 FP8 training: activations grouped in 1 x N_c tiles and weights in
 *     N_c x N_c blocks (N_c = 128), each group with its own scale; partial
 *     sums promoted to fp32 every N_c products.
 *   - §4.2 hyper-parameters: d = 7168, 1 shared + 256 routed experts, expert
 *     intermediate size 2048, 8 routed experts per token, at most 4 nodes,
 *     gamma = 0.001.
 *
 * The garbled pages drop the display equations, so several steps are readings
 * of the surrounding prose; each is marked "reading:" where it is used.
 *
 * Arithmetic policy: every dot product is a sequential sum in double precision
 * (fp64) over the values the inputs decode to; every stored intermediate is
 * rounded exactly once into its storage format (fp32, bf16 or e4m3+scale).
 * Loops are parallel over independent outputs only; no sum is reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2, OR_F64 = 3 };   /* F64: exact storage, for gradient checks */
enum { OR_ADD_RESIDUAL = 1u };

#define OR_NC 128          /* quantisation group size N_c (§3.3) */
#define OR_E4M3_MAX 448.0  /* largest finite OCP E4M3FN value    */

/* ------------------------------------------------------------------------ */
/* Storage formats                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Round a finite double to a binary floating-point format with p significand
 * bits (implicit bit included) and minimum normal exponent emin, to nearest,
 * ties to even.  Below 2^emin the spacing stays 2^(emin-p+1) (gradual
 * underflow).  A result whose magnitude exceeds maxfin becomes +-inf, or
 * +-maxfin when sat is set.  The division by the power-of-two spacing is exact.
 */
double oracle_round_format(double x, int p, int emin, double maxfin, int sat)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int ex;
    frexp(x, &ex);                 /* |x| in [2^(ex-1), 2^ex) */
    int e = ex - 1;
    if (e < emin) e = emin;
    double ulp = ldexp(1.0, e - (p - 1));
    double r = nearbyint(x / ulp) * ulp;   /* default mode: ties to even */
    if (fabs(r) > maxfin) r = sat ? copysign(maxfin, x) : copysign(INFINITY, x);
    return r;
}

static double bf16_max(void) { return ldexp(2.0 - ldexp(1.0, -7), 127); }

/* bf16 = the upper half of an IEEE binary32: 8 significand bits, emin -126 */
double oracle_round_bf16(double x) { return oracle_round_format(x, 8, -126, bf16_max(), 0); }

uint16_t oracle_encode_bf16(double x)
{
    float f = (float)oracle_round_bf16(x);   /* exact: a bf16 value is a binary32 value */
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}

static inline double dec_bf16(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 448, smallest subnormal 2^-9. */
double oracle_decode_e4m3(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
    double v;
    if (E == 15 && m == 7) return NAN;
    if (E == 0) v = ldexp((double)m, -9);                  /* m/8 * 2^-6 */
    else v = ldexp(1.0 + m / 8.0, E - 7);
    return s ? -v : v;
}

double oracle_round_e4m3(double x) { return oracle_round_format(x, 4, -6, OR_E4M3_MAX, 1); }

uint8_t oracle_encode_e4m3(double x)
{
    double r = oracle_round_e4m3(x);
    uint8_t s = (r < 0.0 || (r == 0.0 && signbit(r))) ? 0x80 : 0;
    double a = fabs(r);
    if (a == 0.0) return s;
    if (a < ldexp(1.0, -6)) return s | (uint8_t)(a / ldexp(1.0, -9));   /* subnormal */
    int ex;
    frexp(a, &ex);
    int e = ex - 1;                                                     /* a in [2^e, 2^(e+1)) */
    int m = (int)((a / ldexp(1.0, e) - 1.0) * 8.0);
    return s | (uint8_t)((e + 7) << 3) | (uint8_t)m;
}

static double e4m3_table[256];
static int e4m3_table_ready = 0;
static void init_tables(void)
{
    if (e4m3_table_ready) return;
    for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_decode_e4m3((uint8_t)c);
    e4m3_table_ready = 1;
}

/* Value of element i of a row stored in dtype (fp32, bf16).  */
static inline double load_plain(int dtype, const void *p, int64_t i)
{
    if (dtype == OR_F64) return ((const double *)p)[i];
    if (dtype == OR_F32) return (double)((const float *)p)[i];
    return dec_bf16(((const uint16_t *)p)[i]);
}

/* Store a double into dtype with one rounding. */
static inline void store_plain(int dtype, void *p, int64_t i, double v)
{
    if (dtype == OR_F32) ((float *)p)[i] = (float)v;          /* C cast: IEEE nearest-even */
    else ((uint16_t *)p)[i] = oracle_encode_bf16(v);
}

/*
 * Quantiser Q for one group of n fp32 values (§3.3: one scale per 1 x N_c
 * activation tile or N_c x N_c weight block).  reading: the scale is the
 * group's absolute maximum divided by the largest finite E4M3FN value, as a
 * plain fp32 quotient (1 for an all-zero group); each element is divided by
 * the scale in fp32, clamped to +-448 and rounded to nearest-even E4M3FN.
 */
static float quant_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }
static uint8_t quant_one(float x, float scale)
{
    float q = x / scale;                    /* binary32 division */
    if (q > 448.0f) q = 448.0f;
    if (q < -448.0f) q = -448.0f;
    return oracle_encode_e4m3((double)q);
}

/* 1 x N_c tiles along each row of x[rows][cols] (cols % 128 == 0).
 * in_dtype is OR_F32 or OR_BF16; q[rows][cols], s[rows][cols/128]. */
void oracle_quant_1x128(int64_t rows, int cols, int in_dtype, const void *x, uint8_t *q, float *s)
{
    init_tables();
    int nb = cols / OR_NC;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            float amax = 0.0f;
            for (int c = b * OR_NC; c < (b + 1) * OR_NC; ++c) {
                float v = fabsf((float)load_plain(in_dtype, x, r * cols + c));
                if (v > amax) amax = v;
            }
            float sc = quant_scale(amax);
            s[r * nb + b] = sc;
            for (int c = b * OR_NC; c < (b + 1) * OR_NC; ++c)
                q[r * cols + c] = quant_one((float)load_plain(in_dtype, x, r * cols + c), sc);
        }
    }
}

/* N_c x N_c blocks over each of nmat matrices w[nmat][rows][cols]
 * (rows, cols multiples of 128); s[nmat][rows/128][cols/128]. */
void oracle_quant_128x128(int64_t nmat, int rows, int cols, int in_dtype, const void *w, uint8_t *q, float *s)
{
    init_tables();
    int rb = rows / OR_NC, cb = cols / OR_NC;
#pragma omp parallel for collapse(3) schedule(static)
    for (int64_t m = 0; m < nmat; ++m)
        for (int bi = 0; bi < rb; ++bi)
            for (int bj = 0; bj < cb; ++bj) {
                int64_t base = m * (int64_t)rows * cols;
                float amax = 0.0f;
                for (int i = bi * OR_NC; i < (bi + 1) * OR_NC; ++i)
                    for (int j = bj * OR_NC; j < (bj + 1) * OR_NC; ++j) {
                        float v = fabsf((float)load_plain(in_dtype, w, base + (int64_t)i * cols + j));
                        if (v > amax) amax = v;
                    }
                float sc = quant_scale(amax);
                s[(m * rb + bi) * cb + bj] = sc;
                for (int i = bi * OR_NC; i < (bi + 1) * OR_NC; ++i)
                    for (int j = bj * OR_NC; j < (bj + 1) * OR_NC; ++j) {
                        int64_t k = base + (int64_t)i * cols + j;
                        q[k] = quant_one((float)load_plain(in_dtype, w, k), sc);
                    }
            }
}

/* ------------------------------------------------------------------------ */
/* Routing (§2.1.2)                                                         */
/* ------------------------------------------------------------------------ */

/* Selection and gating for one token from its fp32 affinities s[Nr].
 * reading: groups are contiguous index ranges of Nr/G experts (experts are
 * laid out node by node); a group's score is the sum of its two largest
 * biased affinities (its single affinity when a group holds one expert); the
 * Mg best groups are kept and the other experts masked to -inf; the K best
 * biased affinities among the kept experts are chosen; every tie goes to the
 * lower index; slots are ordered by decreasing biased affinity.  The gating
 * value of slot j is s_j divided by the fp32 sum of the selected un-biased
 * affinities, summed in slot order, times routed_scale. */
static void select_token(int Nr, int G, int Mg, int K, const float *s, const float *bias,
                         float routed_scale, int32_t *idx, float *w)
{
    float sb[1024];
    float gsc[1024];
    char gkeep[1024], taken[1024];
    int gs = Nr / G;
    for (int i = 0; i < Nr; ++i) sb[i] = s[i] + bias[i];          /* one fp32 add */

    for (int g = 0; g < G; ++g) {
        int a = -1;
        for (int i = g * gs; i < (g + 1) * gs; ++i)
            if (a < 0 || sb[i] > sb[a]) a = i;
        if (gs == 1) { gsc[g] = sb[a]; continue; }
        int b = -1;
        for (int i = g * gs; i < (g + 1) * gs; ++i)
            if (i != a && (b < 0 || sb[i] > sb[b])) b = i;
        gsc[g] = sb[a] + sb[b];                                   /* one fp32 add */
    }
    memset(gkeep, 0, (size_t)G);
    for (int r = 0; r < Mg; ++r) {
        int best = -1;
        for (int g = 0; g < G; ++g)
            if (!gkeep[g] && (best < 0 || gsc[g] > gsc[best])) best = g;
        gkeep[best] = 1;
    }
    for (int i = 0; i < Nr; ++i) {
        if (!gkeep[i / gs]) sb[i] = -INFINITY;
        taken[i] = 0;
    }
    for (int j = 0; j < K; ++j) {
        int best = -1;
        for (int i = 0; i < Nr; ++i)
            if (!taken[i] && (best < 0 || sb[i] > sb[best])) best = i;
        taken[best] = 1;
        idx[j] = best;
    }
    float den = 0.0f;
    for (int j = 0; j < K; ++j) den = den + s[idx[j]];
    for (int j = 0; j < K; ++j) w[j] = (s[idx[j]] / den) * routed_scale;
}

/* Affinity of expert i for one token: sigmoid of the fp64 dot product of the
 * token's FFN input with the expert's centroid, rounded once to fp32. */
static float affinity(int d, int u_dtype, const void *u, int64_t t, int e_dtype, const void *e, int i)
{
    double z = 0.0;
    for (int c = 0; c < d; ++c)
        z += load_plain(u_dtype, u, t * d + c) * load_plain(e_dtype, e, (int64_t)i * d + c);
    return (float)(1.0 / (1.0 + exp(-z)));
}

/*
 * Route n_tok tokens (token ids tok[0..n_tok), or 0..n_tok-1 when tok is NULL).
 * scores_in, when given, holds fp32 affinities [T_all][Nr] indexed by token id,
 * and replaces the computed affinities.  scores_out[n_tok][Nr], topk_idx and
 * topk_w[n_tok][K] are indexed by position in the token list.
 */
int oracle_route(int64_t n_tok, const int64_t *tok, int d, int Nr, int G, int Mg, int K,
                 int u_dtype, const void *u, int e_dtype, const void *gate_w,
                 const float *bias, const float *scores_in, float *scores_out,
                 int32_t *topk_idx, float *topk_w, float routed_scale)
{
    if (Nr > 1024 || G < 1 || Nr % G || Mg < 1 || Mg > G || K < 1 || K > Mg * (Nr / G)) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_tok; ++n) {
        int64_t t = tok ? tok[n] : n;
        float s[1024];
        for (int i = 0; i < Nr; ++i)
            s[i] = scores_in ? scores_in[t * Nr + i] : affinity(d, u_dtype, u, t, e_dtype, gate_w, i);
        if (scores_out) memcpy(scores_out + n * Nr, s, sizeof(float) * (size_t)Nr);
        select_token(Nr, G, Mg, K, s, bias, routed_scale, topk_idx + n * K, topk_w + n * K);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch bookkeeping                                                     */
/* ------------------------------------------------------------------------ */

/* counts[i] = number of (token, slot) pairs routed to expert i (whole-batch
 * load, §2.1.2); offsets = exclusive prefix sum; rows offsets[i]..offsets[i+1)
 * hold expert i's tokens in increasing token order; perm_token[row] = token;
 * inv_perm[t*K + j] = the row of slot j of token t. */
void oracle_permute(int64_t T, int K, int Nr, const int32_t *topk_idx,
                    int32_t *counts, int32_t *offsets, int32_t *perm_token, int32_t *inv_perm)
{
    for (int i = 0; i < Nr; ++i) counts[i] = 0;
    for (int64_t n = 0; n < T * K; ++n) counts[topk_idx[n]] += 1;
    offsets[0] = 0;
    for (int i = 0; i < Nr; ++i) offsets[i + 1] = offsets[i] + counts[i];
    for (int i = 0; i < Nr; ++i) {
        int32_t row = offsets[i];
        for (int64_t t = 0; t < T; ++t)
            for (int j = 0; j < K; ++j)
                if (topk_idx[t * K + j] == i) {
                    perm_token[row] = (int32_t)t;
                    inv_perm[t * K + j] = row;
                    ++row;
                }
    }
}

/* ------------------------------------------------------------------------ */
/* Expert FFN                                                               */
/* ------------------------------------------------------------------------ */

/* Decode row r of a [*, n] matrix into double.  For E4M3 the row's scales
 * are the 1 x 128 tile scales sc[r][n/128] when blk_rows == 1, or the
 * 128 x 128 block scales sc[r/128][n/128] when blk_rows == 128. */
static void load_row(int dtype, const void *p, const float *sc, int blk_rows, int64_t r, int n, double *out)
{
    if (dtype == OR_E4M3) {
        const uint8_t *q = (const uint8_t *)p + r * n;
        const float *srow = sc + (r / blk_rows) * (n / OR_NC);
        for (int c = 0; c < n; ++c) out[c] = e4m3_table[q[c]] * (double)srow[c / OR_NC];
    } else {
        for (int c = 0; c < n; ++c) out[c] = load_plain(dtype, p, r * n + c);
    }
}

static double dot(const double *a, const double *b, int n)
{
    double z = 0.0;
    for (int c = 0; c < n; ++c) z += a[c] * b[c];
    return z;
}

/*
 * One SwiGLU expert applied to one input row x[d] (already decoded):
 *   h = SiLU(W_gate x) * (W_up x),  SiLU(a) = a * sigmoid(a)   (reading: the
 *   expert form the pages leave implicit is SwiGLU without biases),
 *   y = W_down h.
 * w_dtype: storage of the weights [I][d] (gate, up) and [d][I] (down); for
 * E4M3 with 128 x 128 block scales.  h is stored in h_dtype before the down
 * projection: fp32, bf16, or (E4M3) quantised per 1 x 128 tile from its fp32
 * value.  The returned y[d] is the exact fp64 result; the caller rounds it.
 */
static void expert_row(int d, int I, int w_dtype, const void *wg, const void *wu, const void *wd,
                       const float *wg_s, const float *wu_s, const float *wd_s, int h_dtype,
                       const double *x, double *y, double *wrow, double *h)
{
    for (int k = 0; k < I; ++k) {
        load_row(w_dtype, wg, wg_s, OR_NC, k, d, wrow);
        double a = dot(x, wrow, d);
        load_row(w_dtype, wu, wu_s, OR_NC, k, d, wrow);
        double b = dot(x, wrow, d);
        double hv = a / (1.0 + exp(-a)) * b;
        if (h_dtype == OR_F32) hv = (double)(float)hv;
        else if (h_dtype == OR_BF16) hv = oracle_round_bf16(hv);
        h[k] = hv;
    }
    if (h_dtype == OR_E4M3) {
        for (int b = 0; b < I / OR_NC; ++b) {
            float amax = 0.0f;
            for (int k = b * OR_NC; k < (b + 1) * OR_NC; ++k) {
                float v = fabsf((float)h[k]);
                if (v > amax) amax = v;
            }
            float sc = quant_scale(amax);
            for (int k = b * OR_NC; k < (b + 1) * OR_NC; ++k)
                h[k] = e4m3_table[quant_one((float)h[k], sc)] * (double)sc;
        }
    }
    for (int i = 0; i < d; ++i) {
        load_row(w_dtype, wd, wd_s, OR_NC, i, I, wrow);
        y[i] = dot(h, wrow, I);
    }
}

static double round_to(int dtype, double v)
{
    return dtype == OR_F32 ? (double)(float)v : oracle_round_bf16(v);
}

/*
 * Grouped FFN on selected rows: expert e owns rows offsets[e]..offsets[e+1)
 * of x.  x is stored in x_dtype ([rows][d]; for E4M3 with 1 x 128 scales
 * x_s[rows][d/128]); weights for all experts are concatenated
 * ([n_exp][I][d] etc., E4M3 scales [n_exp][I/128][d/128] etc.).
 * For each listed row r, y[n][d] = expert(r) applied to x[r], rounded once to
 * y_dtype.
 */
int oracle_grouped_ffn(int n_exp, const int32_t *offsets, int64_t n_rows, const int64_t *rows,
                       int d, int I, int x_dtype, const void *x, const float *x_s,
                       int w_dtype, const void *wg, const void *wu, const void *wd,
                       const float *wg_s, const float *wu_s, const float *wd_s,
                       int h_dtype, int y_dtype, void *y)
{
    init_tables();
    int esz = w_dtype == OR_F32 ? 4 : w_dtype == OR_BF16 ? 2 : 1;
    int xsz = x_dtype == OR_F32 ? 4 : x_dtype == OR_BF16 ? 2 : 1;
    int err = 0;
#pragma omp parallel
    {
        double *xr = malloc(sizeof(double) * (size_t)d);
        double *yr = malloc(sizeof(double) * (size_t)d);
        double *wrow = malloc(sizeof(double) * (size_t)(d > I ? d : I));
        double *h = malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t r = rows[n];
            int e = -1;
            for (int k = 0; k < n_exp; ++k)
                if (r >= offsets[k] && r < offsets[k + 1]) e = k;
            if (e < 0) { err = -1; continue; }
            size_t wo = (size_t)e * I * d * esz;
            size_t so = (size_t)e * (I / OR_NC) * (d / OR_NC);
            load_row(x_dtype, (const char *)x, x_s, 1, r, d, xr);
            (void)xsz;
            expert_row(d, I, w_dtype, (const char *)wg + wo, (const char *)wu + wo, (const char *)wd + wo,
                       w_dtype == OR_E4M3 ? wg_s + so : NULL, w_dtype == OR_E4M3 ? wu_s + so : NULL,
                       w_dtype == OR_E4M3 ? wd_s + so : NULL, h_dtype, xr, yr, wrow, h);
            for (int i = 0; i < d; ++i) store_plain(y_dtype, y, n * d + i, yr[i]);
        }
        free(xr); free(yr); free(wrow); free(h);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Combine (§2.1.2 output equation, stripped on the page; reading: the sum  */
/* of the shared experts' outputs and the gate-weighted routed outputs,     */
/* with the residual u_t added only when asked for)                         */
/* ------------------------------------------------------------------------ */

/* For listed tokens: out[n] = sum_j topk_w[t][j] * y_perm[inv_perm[t*K+j]]
 *   + sum_s y_shared[s][t] (+ u[t]), in fp64, rounded once to y_dtype.
 * y_perm, y_shared and out are stored in y_dtype; u in u_dtype. */
void oracle_combine(int64_t n_tok, const int64_t *tok, int64_t T, int d, int K, int Ns, int y_dtype,
                    const void *y_perm, const int32_t *inv_perm, const float *topk_w,
                    const void *y_shared, int u_dtype, const void *u, void *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_tok; ++n) {
        int64_t t = tok ? tok[n] : n;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j)
                acc += (double)topk_w[t * K + j] * load_plain(y_dtype, y_perm, (int64_t)inv_perm[t * K + j] * d + i);
            for (int s = 0; s < Ns; ++s) acc += load_plain(y_dtype, y_shared, ((int64_t)s * T + t) * d + i);
            if (u) acc += load_plain(u_dtype, u, t * d + i);
            store_plain(y_dtype, out, n * d + i, acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Whole layer for a list of tokens                                         */
/* ------------------------------------------------------------------------ */

/*
 * out[n][d] for token tok[n]: route the token (own affinities, or scores_in),
 * prepare its FFN input row (u itself, or for E4M3 weights its 1 x 128
 * quantisation), apply its K experts and the Ns shared experts with the
 * storage roundings of expert_row, round each expert output to out_dtype,
 * then combine in fp64 and round once.
 * Routed weights: [Nr][I][d], [Nr][I][d], [Nr][d][I]; shared: [Ns][...].
 */
int oracle_moe_forward(int64_t n_tok, const int64_t *tok, int d, int Nr, int Ns, int G, int Mg, int K, int I,
                       int act_dtype, int w_dtype, int out_dtype, float routed_scale, unsigned flags,
                       const void *u, const void *gate_w, const float *bias, const float *scores_in,
                       const void *rwg, const void *rwu, const void *rwd,
                       const float *rwg_s, const float *rwu_s, const float *rwd_s,
                       const void *swg, const void *swu, const void *swd,
                       const float *swg_s, const float *swu_s, const float *swd_s,
                       void *out, int32_t *topk_idx, float *topk_w, float *scores_out)
{
    init_tables();
    int rc = oracle_route(n_tok, tok, d, Nr, G, Mg, K, act_dtype, u, act_dtype, gate_w, bias, scores_in,
                          scores_out, topk_idx, topk_w, routed_scale);
    if (rc) return rc;
    int h_dtype = w_dtype == OR_E4M3 ? OR_E4M3 : act_dtype;
    int esz = w_dtype == OR_F32 ? 4 : w_dtype == OR_BF16 ? 2 : 1;
    size_t wmat = (size_t)I * d;
    size_t smat = (size_t)(I / OR_NC) * (d / OR_NC);
    int nwork = K + Ns;
    double *res = malloc(sizeof(double) * (size_t)n_tok * nwork * d);
    if (!res) return -3;
#pragma omp parallel
    {
        double *xr = malloc(sizeof(double) * (size_t)d);
        double *wrow = malloc(sizeof(double) * (size_t)(d > I ? d : I));
        double *h = malloc(sizeof(double) * (size_t)I);
        uint8_t *xq = malloc((size_t)d);
        float *xs = malloc(sizeof(float) * (size_t)(d / OR_NC + 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t n = 0; n < n_tok; ++n)
            for (int j = 0; j < nwork; ++j) {
                int64_t t = tok ? tok[n] : n;
                if (w_dtype == OR_E4M3) {
                    oracle_quant_1x128(1, d, act_dtype, (const char *)u + (size_t)t * d * (act_dtype == OR_F32 ? 4 : 2), xq, xs);
                    load_row(OR_E4M3, xq, xs, 1, 0, d, xr);
                } else {
                    load_row(act_dtype, u, NULL, 1, t, d, xr);
                }
                const char *g, *up, *dn;
                const float *gs = NULL, *us = NULL, *ds = NULL;
                if (j < K) {
                    int e = topk_idx[n * K + j];
                    g = (const char *)rwg + (size_t)e * wmat * esz;
                    up = (const char *)rwu + (size_t)e * wmat * esz;
                    dn = (const char *)rwd + (size_t)e * wmat * esz;
                    if (w_dtype == OR_E4M3) { gs = rwg_s + e * smat; us = rwu_s + e * smat; ds = rwd_s + e * smat; }
                } else {
                    int s = j - K;
                    g = (const char *)swg + (size_t)s * wmat * esz;
                    up = (const char *)swu + (size_t)s * wmat * esz;
                    dn = (const char *)swd + (size_t)s * wmat * esz;
                    if (w_dtype == OR_E4M3) { gs = swg_s + s * smat; us = swu_s + s * smat; ds = swd_s + s * smat; }
                }
                double *y = res + ((size_t)n * nwork + j) * d;
                expert_row(d, I, w_dtype, g, up, dn, gs, us, ds, h_dtype, xr, y, wrow, h);
                for (int i = 0; i < d; ++i) y[i] = round_to(out_dtype, y[i]);   /* expert output storage */
            }
        free(xr); free(wrow); free(h); free(xq); free(xs);
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_tok; ++n) {
        int64_t t = tok ? tok[n] : n;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < K; ++j) acc += (double)topk_w[n * K + j] * res[((size_t)n * nwork + j) * d + i];
            for (int s = 0; s < Ns; ++s) acc += res[((size_t)n * nwork + K + s) * d + i];
            if (flags & OR_ADD_RESIDUAL) acc += load_plain(act_dtype, u, t * d + i);
            store_plain(out_dtype, out, n * d + i, acc);
        }
    }
    free(res);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Bias update (§2.1.2; rate gamma from §4.2)                               */
/* ------------------------------------------------------------------------ */

/* reading: an expert is overloaded when its load exceeds the mean load
 * T*K/Nr (as fp32), underloaded when below; b_i moves by -gamma, +gamma, or
 * not at all on an exact tie: b_i = fl32(b_i + gamma * sign(mean - load_i)). */
void oracle_bias_update(int Nr, int64_t T, int K, const int32_t *counts, float *bias, float gamma)
{
    float mean = (float)((double)(float)(T * K) / (double)(float)Nr);
    for (int i = 0; i < Nr; ++i) {
        float load = (float)counts[i];
        float sgn = load < mean ? 1.0f : (load > mean ? -1.0f : 0.0f);
        bias[i] = bias[i] + gamma * sgn;
    }
}

/*
 * Complementary sequence-wise balance statistic (§2.1.2: a tiny loss
 * alpha * sum_i f_i P_i kept next to the bias rule; §4.2: alpha = 0.0001).
 * The pages name f_i and P_i but their definitions are stripped; reading:
 * for a sequence of Ts tokens,
 *   f_i = N_r / (K * Ts) * #{(t, j) : topk_idx[t][j] == i}   (selected load, 1 when even)
 *   P_i = (1 / Ts) * sum_t s_{i,t} / sum_k s_{k,t}           (affinity share over all routed experts)
 * Sequences are consecutive runs of seq_len tokens (the last may be shorter).
 * All sums in double, each output rounded once.  counts_out [n_seq][Nr] and
 * share_out [n_seq][Nr] (P_i) may be NULL.
 */
void oracle_seq_balance(int64_t T, int Nr, int K, const float *scores, const int32_t *topk_idx, int64_t seq_len,
                        float alpha, float *loss_out, int32_t *counts_out, float *share_out)
{
    const int64_t n_seq = (T + seq_len - 1) / seq_len;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic)
#endif
    for (int64_t q = 0; q < n_seq; ++q) {
        const int64_t t0 = q * seq_len;
        const int64_t t1 = t0 + seq_len < T ? t0 + seq_len : T;
        const double Ts = (double)(t1 - t0);
        int64_t *cnt = (int64_t *)calloc((size_t)Nr, sizeof(int64_t));
        double *share = (double *)calloc((size_t)Nr, sizeof(double));
        for (int64_t t = t0; t < t1; ++t) {
            double row = 0.0;
            for (int i = 0; i < Nr; ++i) row += (double)scores[t * Nr + i];
            for (int i = 0; i < Nr; ++i) share[i] += (double)scores[t * Nr + i] / row;
            for (int j = 0; j < K; ++j) cnt[topk_idx[t * K + j]] += 1;
        }
        double loss = 0.0;
        for (int i = 0; i < Nr; ++i) {
            const double f = (double)Nr / ((double)K * Ts) * (double)cnt[i];
            const double P = share[i] / Ts;
            loss += f * P;
            if (counts_out) counts_out[q * Nr + i] = (int32_t)cnt[i];
            if (share_out) share_out[q * Nr + i] = (float)P;
        }
        loss_out[q] = (float)((double)alpha * loss);
        free(cnt);
        free(share);
    }
}

/* ------------------------------------------------------------------------ */
/* Exact layer and its gradient for a fixed selection (backward reference)   */
/* ------------------------------------------------------------------------ */

/*
 * The layer of §2.1.2 evaluated in fp64 with nothing rounded after the inputs
 * are decoded, for a given selection topk_idx [T][K] (held fixed: the
 * selection is piecewise constant, so the layer is smooth in u, the centroids
 * and the weights wherever the selection does not change):
 *   s_{t,i} = sigmoid(u_t . e_i),  g_{t,j} = rs * s_{t,e_j} / sum_k s_{t,e_k}
 *   (rs: the routed scaling factor, 1 in the pages' formula),
 *   out_t = sum_j g_{t,j} FFN_{e_j}(u_t) + sum_s FFN^shared_s(u_t),
 *   FFN(x) = W_down (SiLU(W_gate x) * (W_up x)).
 * u [T][d] and gate_w [Nr][d] are stored in a_code, the weights in w_code
 * (OR_F32, OR_BF16 or OR_F64): routed [Nr][I][d], [Nr][I][d], [Nr][d][I],
 * shared [Ns][...].  out [T][d] and topk_w [T][K] (may be NULL) are fp64.
 */
typedef struct { int code; const void *p; } omat;

static void orow(omat m, int64_t r, int n, double *out)
{
    for (int c = 0; c < n; ++c) out[c] = load_plain(m.code, m.p, r * n + c);
}

static omat osub(omat m, int64_t e, size_t elems)
{
    const size_t esz = m.code == OR_F64 ? 8 : m.code == OR_F32 ? 4 : 2;
    omat r = {m.code, (const char *)m.p + (size_t)e * elems * esz};
    return r;
}

/* a = W_gate x, b = W_up x, h = SiLU(a) b, y = W_down h (all fp64); row: d+I scratch */
static void ffn64(int d, int I, omat wg, omat wu, omat wd, const double *x, double *a, double *b, double *h,
                  double *y, double *row)
{
    for (int k = 0; k < I; ++k) {
        orow(wg, k, d, row);
        a[k] = dot(x, row, d);
        orow(wu, k, d, row);
        b[k] = dot(x, row, d);
        h[k] = a[k] / (1.0 + exp(-a[k])) * b[k];
    }
    for (int i = 0; i < d; ++i) {
        orow(wd, i, I, row);
        y[i] = dot(h, row, I);
    }
}

static void gates64(int d, int K, const double *x, omat gate_w, const int32_t *sel, double rs, double *s_sel,
                    double *g, double *row)
{
    double den = 0.0;
    for (int j = 0; j < K; ++j) {
        orow(gate_w, sel[j], d, row);
        s_sel[j] = 1.0 / (1.0 + exp(-dot(x, row, d)));
        den += s_sel[j];
    }
    for (int j = 0; j < K; ++j) g[j] = rs * s_sel[j] / den;
}

/* dh = W_down^T dy (sum over the d rows of W_down in order); row: I scratch */
static void down_t(int d, int I, omat wd, const double *dy, double *dh, double *row)
{
    for (int k = 0; k < I; ++k) dh[k] = 0.0;
    for (int c = 0; c < d; ++c) {
        orow(wd, c, I, row);
        for (int k = 0; k < I; ++k) dh[k] += row[k] * dy[c];
    }
}

int oracle_layer_f64(int64_t T, int d, int Nr, int Ns, int K, int I, int a_code, const void *u, const void *gate_w,
                     const int32_t *topk_idx, int w_code, const void *rwg, const void *rwu, const void *rwd,
                     const void *swg, const void *swu, const void *swd, double rs, double *out, double *topk_w)
{
    const size_t wm = (size_t)I * d;
    const omat U = {a_code, u}, E = {a_code, gate_w};
    const omat RG = {w_code, rwg}, RU = {w_code, rwu}, RD = {w_code, rwd};
    const omat SG = {w_code, swg}, SU = {w_code, swu}, SD = {w_code, swd};
    if (K > 32) return -2;
    (void)Nr;
#pragma omp parallel
    {
        double *a = malloc(sizeof(double) * (size_t)I), *b = malloc(sizeof(double) * (size_t)I);
        double *h = malloc(sizeof(double) * (size_t)I), *y = malloc(sizeof(double) * (size_t)d);
        double *x = malloc(sizeof(double) * (size_t)d), *row = malloc(sizeof(double) * (size_t)(d + I));
        double s_sel[32], g[32];
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            double *o = out + (size_t)t * d;
            orow(U, t, d, x);
            gates64(d, K, x, E, topk_idx + t * K, rs, s_sel, g, row);
            if (topk_w)
                for (int j = 0; j < K; ++j) topk_w[t * K + j] = g[j];
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            for (int j = 0; j < K + Ns; ++j) {
                const int routed = j < K, e = routed ? topk_idx[t * K + j] : j - K;
                ffn64(d, I, osub(routed ? RG : SG, e, wm), osub(routed ? RU : SU, e, wm), osub(routed ? RD : SD, e, wm),
                      x, a, b, h, y, row);
                const double gj = routed ? g[j] : 1.0;
                for (int i = 0; i < d; ++i) o[i] += gj * y[i];
            }
        }
        free(a); free(b); free(h); free(y); free(x); free(row);
    }
    return 0;
}

/*
 * Gradient of sum(dout * out) for the layer above (dout [T][d] fp64), by the
 * chain rule written out in fp64:
 *   dy_{t,j} = g_{t,j} dout_t,   dg_{t,j} = dout_t . y_{t,j}
 *   per expert row: dh = W_down^T dy,  dW_down += dy h^T,
 *     da = dh * b * SiLU'(a) with SiLU'(a) = sigma(a) (1 + a (1 - sigma(a))),
 *     db = dh * SiLU(a),  dx = W_gate^T da + W_up^T db,
 *     dW_gate += da x^T,  dW_up += db x^T
 *   gates g_j = rs s_j / D (D = sum of the selected s):
 *     ds_k = rs (dg_k / D - (sum_j dg_j s_j) / D^2) for selected k (no other
 *     expert receives gate gradient; the bias receives none),
 *   dz = ds * s (1 - s),  du_t += sum_j dx_{t,j} + dx_shared + sum_k dz_k e_k,
 *   de_k += dz_k u_t.
 * Subsets: du [T][d] and dtopk_w [T][K] rows are written for the listed tokens
 * only (tok = NULL: all T).  Routed weight gradients are written for the listed
 * experts (exps = NULL: all Nr), the q-th listed expert's into slot q of
 * drwg/drwu/drwd ([n][I][d], [n][I][d], [n][d][I]); each sums over every token
 * routed to it, in token order.  Shared weight gradients ([Ns][...]) and
 * dgate_w ([Nr][d], every token) only when their pointers are non-NULL.
 */
int oracle_moe_backward_f64(int64_t T, int d, int Nr, int Ns, int K, int I, int a_code, const void *u,
                            const void *gate_w, const int32_t *topk_idx, int w_code, const void *rwg, const void *rwu,
                            const void *rwd, const void *swg, const void *swu, const void *swd, double rs,
                            const double *dout, int64_t n_tok, const int64_t *tok, int n_exp, const int32_t *exps,
                            double *du, double *dtopk_w, double *dgate_w,
                            double *drwg, double *drwu, double *drwd,
                            double *dswg, double *dswu, double *dswd)
{
    const size_t wm = (size_t)I * d;
    const omat U = {a_code, u}, E = {a_code, gate_w};
    const omat RG = {w_code, rwg}, RU = {w_code, rwu}, RD = {w_code, rwd};
    const omat SG = {w_code, swg}, SU = {w_code, swu}, SD = {w_code, swd};
    if (K > 32) return -2;
    /* per-token input gradient (and gate gradient) for the listed tokens */
    if (du || dtopk_w) {
#pragma omp parallel
        {
            double *a = malloc(sizeof(double) * (size_t)I), *b = malloc(sizeof(double) * (size_t)I);
            double *h = malloc(sizeof(double) * (size_t)I), *y = malloc(sizeof(double) * (size_t)d);
            double *dh = malloc(sizeof(double) * (size_t)I), *dx = malloc(sizeof(double) * (size_t)d);
            double *x = malloc(sizeof(double) * (size_t)d), *row = malloc(sizeof(double) * (size_t)(d + I));
            double *da = malloc(sizeof(double) * (size_t)I), *db = malloc(sizeof(double) * (size_t)I);
            double *dy = malloc(sizeof(double) * (size_t)d);
            double s_sel[32], g[32], dg[32];
#pragma omp for schedule(dynamic, 1)
            for (int64_t n = 0; n < (tok ? n_tok : T); ++n) {
                const int64_t t = tok ? tok[n] : n;
                const double *dO = dout + (size_t)t * d;
                const int32_t *sel = topk_idx + t * K;
                orow(U, t, d, x);
                gates64(d, K, x, E, sel, rs, s_sel, g, row);
                for (int c = 0; c < d; ++c) dx[c] = 0.0;
                for (int j = 0; j < K + Ns; ++j) {
                    const int routed = j < K, e = routed ? sel[j] : j - K;
                    const omat wg = osub(routed ? RG : SG, e, wm), wu = osub(routed ? RU : SU, e, wm);
                    const omat wd = osub(routed ? RD : SD, e, wm);
                    ffn64(d, I, wg, wu, wd, x, a, b, h, y, row);
                    const double gj = routed ? g[j] : 1.0;
                    if (routed) dg[j] = dot(dO, y, d);
                    for (int c = 0; c < d; ++c) dy[c] = gj * dO[c];
                    down_t(d, I, wd, dy, dh, row);
                    for (int k = 0; k < I; ++k) {
                        const double sg = 1.0 / (1.0 + exp(-a[k]));
                        da[k] = dh[k] * b[k] * sg * (1.0 + a[k] * (1.0 - sg));
                        db[k] = dh[k] * a[k] * sg;
                    }
                    for (int k = 0; k < I; ++k) {
                        orow(wg, k, d, row);
                        for (int c = 0; c < d; ++c) dx[c] += row[c] * da[k];
                        orow(wu, k, d, row);
                        for (int c = 0; c < d; ++c) dx[c] += row[c] * db[k];
                    }
                }
                double den = 0.0, sdg = 0.0;
                for (int j = 0; j < K; ++j) { den += s_sel[j]; sdg += dg[j] * s_sel[j]; }
                for (int j = 0; j < K; ++j) {
                    const double dz = rs * (dg[j] / den - sdg / (den * den)) * s_sel[j] * (1.0 - s_sel[j]);
                    orow(E, sel[j], d, row);
                    for (int c = 0; c < d; ++c) dx[c] += dz * row[c];
                }
                if (du)
                    for (int c = 0; c < d; ++c) du[(size_t)t * d + c] = dx[c];
                if (dtopk_w)
                    for (int j = 0; j < K; ++j) dtopk_w[t * K + j] = dg[j];
            }
            free(a); free(b); free(h); free(y); free(dh); free(dx); free(x); free(row); free(da); free(db); free(dy);
        }
    }
    /* centroid gradient: every token contributes dz_k u_t to its selected experts */
    if (dgate_w) {
        for (size_t q = 0; q < (size_t)Nr * d; ++q) dgate_w[q] = 0.0;
        double *dzall = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * K);
#pragma omp parallel
        {
            double *a = malloc(sizeof(double) * (size_t)I), *b = malloc(sizeof(double) * (size_t)I);
            double *h = malloc(sizeof(double) * (size_t)I), *y = malloc(sizeof(double) * (size_t)d);
            double *x = malloc(sizeof(double) * (size_t)d), *row = malloc(sizeof(double) * (size_t)(d + I));
            double s_sel[32], g[32], dg[32];
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                const double *dO = dout + (size_t)t * d;
                const int32_t *sel = topk_idx + t * K;
                orow(U, t, d, x);
                gates64(d, K, x, E, sel, rs, s_sel, g, row);
                double den = 0.0, sdg = 0.0;
                for (int j = 0; j < K; ++j) {
                    ffn64(d, I, osub(RG, sel[j], wm), osub(RU, sel[j], wm), osub(RD, sel[j], wm), x, a, b, h, y, row);
                    dg[j] = dot(dO, y, d);
                    den += s_sel[j];
                    sdg += dg[j] * s_sel[j];
                }
                for (int j = 0; j < K; ++j)
                    dzall[t * K + j] = rs * (dg[j] / den - sdg / (den * den)) * s_sel[j] * (1.0 - s_sel[j]);
            }
            free(a); free(b); free(h); free(y); free(x); free(row);
        }
        for (int64_t t = 0; t < T; ++t)          /* tokens in order: fixed summation order */
            for (int j = 0; j < K; ++j) {
                double *de = dgate_w + (size_t)topk_idx[t * K + j] * d;
                for (int c = 0; c < d; ++c) de[c] += dzall[t * K + j] * load_plain(a_code, u, t * d + c);
            }
        free(dzall);
    }
    /* weight gradients: routed experts (listed) over the tokens routed to them, then shared.
     * Phase 1 (parallel over the expert's tokens): x, dy, h, da, db of each token.
     * Phase 2 (parallel over output rows): the outer products summed over the tokens in order. */
    for (int pass = 0; pass < 2; ++pass) {
        const int nE = pass == 0 ? (exps ? n_exp : (drwg ? Nr : 0)) : (dswg ? Ns : 0);
        for (int q = 0; q < nE; ++q) {
            const int e = pass == 0 ? (exps ? exps[q] : q) : q;
            const omat wg = osub(pass ? SG : RG, e, wm), wu = osub(pass ? SU : RU, e, wm);
            const omat wd = osub(pass ? SD : RD, e, wm);
            double *gwg = (pass ? dswg : drwg) + q * wm, *gwu = (pass ? dswu : drwu) + q * wm;
            double *gwd = (pass ? dswd : drwd) + q * wm;
            int64_t nt = 0;
            int64_t *tl = malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
            int *jl = malloc(sizeof(int) * (size_t)(T > 0 ? T : 1));
            for (int64_t t = 0; t < T; ++t) {
                if (pass) { tl[nt] = t; jl[nt++] = -1; continue; }
                for (int j = 0; j < K; ++j)
                    if (topk_idx[t * K + j] == e) { tl[nt] = t; jl[nt++] = j; }
            }
            const size_t per = 2 * (size_t)d + 3 * (size_t)I;   /* x[d], dy[d], h[I], da[I], db[I] */
            double *buf = malloc(sizeof(double) * per * (size_t)(nt > 0 ? nt : 1));
#pragma omp parallel
            {
                double *a = malloc(sizeof(double) * (size_t)I), *b = malloc(sizeof(double) * (size_t)I);
                double *y = malloc(sizeof(double) * (size_t)d), *row = malloc(sizeof(double) * (size_t)(d + I));
                double *dh = malloc(sizeof(double) * (size_t)I);
                double s_sel[32], g[32];
#pragma omp for schedule(dynamic, 1)
                for (int64_t n = 0; n < nt; ++n) {
                    const int64_t t = tl[n];
                    double *x = buf + per * n, *dy = x + d, *h = dy + d, *da = h + I, *db = da + I;
                    orow(U, t, d, x);
                    double gj = 1.0;
                    if (!pass) {
                        gates64(d, K, x, E, topk_idx + t * K, rs, s_sel, g, row);
                        gj = g[jl[n]];
                    }
                    ffn64(d, I, wg, wu, wd, x, a, b, h, y, row);
                    for (int c = 0; c < d; ++c) dy[c] = gj * dout[(size_t)t * d + c];
                    down_t(d, I, wd, dy, dh, row);
                    for (int k = 0; k < I; ++k) {
                        const double sg = 1.0 / (1.0 + exp(-a[k]));
                        da[k] = dh[k] * b[k] * sg * (1.0 + a[k] * (1.0 - sg));
                        db[k] = dh[k] * a[k] * sg;
                    }
                }
                free(a); free(b); free(y); free(row); free(dh);
            }
#pragma omp parallel for schedule(static)
            for (int c = 0; c < d; ++c)
                for (int k = 0; k < I; ++k) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < nt; ++n) acc += buf[per * n + d + c] * buf[per * n + 2 * d + k];
                    gwd[(size_t)c * I + k] = acc;
                }
#pragma omp parallel for schedule(static)
            for (int k = 0; k < I; ++k)
                for (int c = 0; c < d; ++c) {
                    double ag = 0.0, au = 0.0;
                    for (int64_t n = 0; n < nt; ++n) {
                        const double xc = buf[per * n + c];
                        ag += buf[per * n + 2 * d + I + k] * xc;
                        au += buf[per * n + 2 * d + 2 * I + k] * xc;
                    }
                    gwg[(size_t)k * d + c] = ag;
                    gwu[(size_t)k * d + c] = au;
                }
            free(buf); free(tl); free(jl);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FP8 backward (§3.3: Fprop, Dgrad and Wgrad GEMMs in FP8)                  */
/* ------------------------------------------------------------------------ */

/* Quantise v[n] (as fp32 values) in 1 x 128 tiles and replace it by the
 * dequantised values. */
static void q1x128_inplace(int n, double *v)
{
    for (int b = 0; b < n / OR_NC; ++b) {
        float amax = 0.0f;
        for (int k = b * OR_NC; k < (b + 1) * OR_NC; ++k) {
            float a = fabsf((float)v[k]);
            if (a > amax) amax = a;
        }
        const float sc = quant_scale(amax);
        for (int k = b * OR_NC; k < (b + 1) * OR_NC; ++k)
            v[k] = e4m3_table[quant_one((float)v[k], sc)] * (double)sc;
    }
}

/* Rows v[nr][n] (row stride n) quantised in 128 x 1 tiles: column c of the
 * rows [128 j, 128 j + 128) of the list shares one scale (the last tile may
 * be shorter); replaced by the dequantised values. */
static void q128x1_inplace(int64_t nr, int n, double *v, size_t stride)
{
    for (int64_t r0 = 0; r0 < nr; r0 += OR_NC) {
        const int64_t r1 = r0 + OR_NC < nr ? r0 + OR_NC : nr;
        for (int c = 0; c < n; ++c) {
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r) {
                float a = fabsf((float)v[r * stride + c]);
                if (a > amax) amax = a;
            }
            const float sc = quant_scale(amax);
            for (int64_t r = r0; r < r1; ++r)
                v[r * stride + c] = e4m3_table[quant_one((float)v[r * stride + c], sc)] * (double)sc;
        }
    }
}

/*
 * 128 x 1 tiles along the rows of segments (the backward's Wgrad operands):
 * segment e owns list rows off[e] .. off[e+1]; its rows are taken in runs of
 * 128 from the segment's first row (the last run may be shorter), and column
 * c of a run shares one scale.  List row r reads row (gather ? gather[r] : r)
 * of x [*][cols], stored in in_dtype: OR_F32, OR_BF16, or OR_E4M3 with 1 x 128
 * tile scales x_s[*][cols/128] (dequantised to fp32 first).  Outputs: codes
 * q[rows][cols] and scales s[nblk][cols], where run j of segment e is block
 * sum_{e' < e} ceil(len(e') / 128) + j.
 */
void oracle_quant_128x1(int n_seg, const int32_t *off, int cols, int in_dtype, const void *x, const float *x_s,
                        const int32_t *gather, uint8_t *q, float *s)
{
    init_tables();
    int64_t bbase = 0;
    for (int e = 0; e < n_seg; ++e) {
        const int64_t r0 = off[e], len = (int64_t)off[e + 1] - off[e];
        const int64_t nb = (len + OR_NC - 1) / OR_NC;
#pragma omp parallel for schedule(static)
        for (int c = 0; c < cols; ++c) {
            for (int64_t j = 0; j < nb; ++j) {
                const int64_t a = r0 + j * OR_NC, b = a + OR_NC < r0 + len ? a + OR_NC : r0 + len;
                float amax = 0.0f;
                for (int64_t r = a; r < b; ++r) {
                    const int64_t xr = gather ? gather[r] : r;
                    float v = in_dtype == OR_E4M3 ? (float)(e4m3_table[((const uint8_t *)x)[xr * cols + c]] *
                                                          (double)x_s[xr * (cols / OR_NC) + c / OR_NC])
                                                  : (float)load_plain(in_dtype, x, xr * cols + c);
                    if (fabsf(v) > amax) amax = fabsf(v);
                }
                const float sc = quant_scale(amax);
                s[(bbase + j) * cols + c] = sc;
                for (int64_t r = a; r < b; ++r) {
                    const int64_t xr = gather ? gather[r] : r;
                    float v = in_dtype == OR_E4M3 ? (float)(e4m3_table[((const uint8_t *)x)[xr * cols + c]] *
                                                          (double)x_s[xr * (cols / OR_NC) + c / OR_NC])
                                                  : (float)load_plain(in_dtype, x, xr * cols + c);
                    q[r * cols + c] = quant_one(v, sc);
                }
            }
        }
        bbase += nb;
    }
}

/*
 * One (token, expert) pair of the FP8 layer (bf16 activations, e4m3 expert
 * GEMMs) and the input-gradient chain through it, each GEMM on FP8 operands:
 *   forward (as moe_forward computes it): a, b from the token's 1 x 128 tiles x
 *     and the 128 x 128 weight blocks; h = SiLU(a) b, cached as 1 x 128 tiles
 *     (hq, dequantised); y = W_down hq, stored in bf16;
 *   dy = bf16(g dO) (the shared experts: dO);
 *   Dgrad 1: dh = bf16(W_down^T Q1x128(dy));
 *   SwiGLU gradient, elementwise in fp64 from a and b: da = bf16(dh b SiLU'(a)),
 *     db = bf16(dh SiLU(a));
 *   Dgrad 2: dx = bf16(W_gate^T da' + W_up^T db') with [da' | db'] = Q1x128([da | db]).
 * (reading: every gradient operand of a Dgrad GEMM is tiled 1 x 128 along that
 * GEMM's reduction, as the forward's activations are; the weights keep their
 * 128 x 128 blocks, which the transposed use leaves square.)
 * Outputs y, dy, hq, da, db, dx (any NULL to skip); a, b, wrow, t2 are scratch
 * of I, I, max(d, I), 2I doubles.
 */
static void fp8_pair(int d, int I, const uint8_t *wg, const uint8_t *wu, const uint8_t *wd, const float *wg_s,
                     const float *wu_s, const float *wd_s, const double *x, double gj, const double *dO, double *a,
                     double *b, double *hq, double *y, double *dy, double *da, double *db, double *dx, double *wrow,
                     double *t2)
{
    for (int k = 0; k < I; ++k) {
        load_row(OR_E4M3, wg, wg_s, OR_NC, k, d, wrow);
        a[k] = dot(x, wrow, d);
        load_row(OR_E4M3, wu, wu_s, OR_NC, k, d, wrow);
        b[k] = dot(x, wrow, d);
        hq[k] = a[k] / (1.0 + exp(-a[k])) * b[k];
    }
    q1x128_inplace(I, hq);
    for (int i = 0; i < d; ++i) {
        load_row(OR_E4M3, wd, wd_s, OR_NC, i, I, wrow);
        y[i] = oracle_round_bf16(dot(hq, wrow, I));
    }
    /* dy and its 1 x 128 tiles (t2 holds the dequantised copy, d <= 2I is not assumed) */
    double *dyq = malloc(sizeof(double) * (size_t)d);
    for (int c = 0; c < d; ++c) {
        dy[c] = gj == 1.0 ? dO[c] : oracle_round_bf16(gj * dO[c]);
        dyq[c] = dy[c];
    }
    q1x128_inplace(d, dyq);
    double *dh = t2;   /* I values */
    for (int k = 0; k < I; ++k) dh[k] = 0.0;
    for (int c = 0; c < d; ++c) {
        load_row(OR_E4M3, wd, wd_s, OR_NC, c, I, wrow);
        for (int k = 0; k < I; ++k) dh[k] += dyq[c] * wrow[k];
    }
    free(dyq);
    for (int k = 0; k < I; ++k) {
        const double hk = oracle_round_bf16(dh[k]);
        const double sg = 1.0 / (1.0 + exp(-a[k]));
        da[k] = oracle_round_bf16(hk * b[k] * sg * (1.0 + a[k] * (1.0 - sg)));
        db[k] = oracle_round_bf16(hk * a[k] * sg);
    }
    /* [da | db] in 1 x 128 tiles (I is a multiple of 128, so no tile straddles the halves) */
    double *abq = t2;
    for (int k = 0; k < I; ++k) { abq[k] = da[k]; abq[I + k] = db[k]; }
    q1x128_inplace(2 * I, abq);
    for (int c = 0; c < d; ++c) dx[c] = 0.0;
    for (int k = 0; k < I; ++k) {
        load_row(OR_E4M3, wg, wg_s, OR_NC, k, d, wrow);
        for (int c = 0; c < d; ++c) dx[c] += abq[k] * wrow[c];
    }
    for (int k = 0; k < I; ++k) {
        load_row(OR_E4M3, wu, wu_s, OR_NC, k, d, wrow);
        for (int c = 0; c < d; ++c) dx[c] += abq[I + k] * wrow[c];
    }
    for (int c = 0; c < d; ++c) dx[c] = oracle_round_bf16(dx[c]);
}

/*
 * Gradient of the FP8 layer for a fixed selection (reading R20 as for
 * oracle_moe_backward_f64, with the FP8 GEMMs of fp8_pair).  u [T][d] and
 * gate_w [Nr][d] are bf16; the expert weights are e4m3 codes with 128 x 128
 * block scales ([n][I][d] gate and up, [n][d][I] down; scales [n][I/128][d/128]
 * and [n][d/128][I/128]); dout [T][d] holds the values of the bf16 upstream
 * gradient.  The router keeps bf16 activations and fp64 gates (gating is not
 * quantised).  du and dtopk_w rows are written for the listed tokens.
 * Wgrad (reading: the activations cached in 1 x 128 tiles, u's and H's, and
 * the gradients dy, da, db are re-tiled 128 x 1 along the expert's rows, which
 * are the GEMM's reduction, in runs of 128 from the expert's first row):
 *   dW_down = sum_r Q(dy_r) Q(hq_r)^T, [dW_gate; dW_up] = sum_r Q([da_r; db_r]) Q(x_r)^T
 * summed over the expert's rows in token order (fp64).  Routed gradients for
 * the listed experts go to slot q of drwg/drwu/drwd; the shared experts' and
 * dgate_w (every token) only when their pointers are non-NULL.
 */
int oracle_moe_backward_fp8(int64_t T, int d, int Nr, int Ns, int K, int I, const uint16_t *u,
                            const uint16_t *gate_w, const int32_t *topk_idx, const uint8_t *rwg, const uint8_t *rwu,
                            const uint8_t *rwd, const float *rwg_s, const float *rwu_s, const float *rwd_s,
                            const uint8_t *swg, const uint8_t *swu, const uint8_t *swd, const float *swg_s,
                            const float *swu_s, const float *swd_s, double rs, const double *dout, int64_t n_tok,
                            const int64_t *tok, int n_exp, const int32_t *exps, double *du, double *dtopk_w,
                            double *dgate_w, double *drwg, double *drwu, double *drwd, double *dswg, double *dswu,
                            double *dswd)
{
    init_tables();
    const size_t wm = (size_t)I * d, sm = (size_t)(I / OR_NC) * (d / OR_NC);
    const omat U = {OR_BF16, u}, E = {OR_BF16, gate_w};
    if (K > 32 || d % OR_NC || I % OR_NC) return -2;
    /* the token's activations as the expert GEMMs see them: 1 x 128 tiles of u */
#define FP8_X(t, x)                                  \
    do {                                             \
        orow(U, (t), d, (x));                        \
        q1x128_inplace(d, (x));                      \
    } while (0)
    const int need_tok = du || dtopk_w, need_dz = dgate_w != NULL;
    double *dzall = need_dz ? calloc((size_t)(T > 0 ? T : 1) * K, sizeof(double)) : NULL;
    if (need_tok || need_dz) {
#pragma omp parallel
        {
            const int mx = d > I ? d : I;
            double *x = malloc(sizeof(double) * (size_t)d), *xr = malloc(sizeof(double) * (size_t)d);
            double *a = malloc(sizeof(double) * (size_t)I), *b = malloc(sizeof(double) * (size_t)I);
            double *hq = malloc(sizeof(double) * (size_t)I), *y = malloc(sizeof(double) * (size_t)d);
            double *dy = malloc(sizeof(double) * (size_t)d), *da = malloc(sizeof(double) * (size_t)I);
            double *db = malloc(sizeof(double) * (size_t)I), *dx = malloc(sizeof(double) * (size_t)d);
            double *acc = malloc(sizeof(double) * (size_t)d), *wrow = malloc(sizeof(double) * (size_t)mx);
            double *t2 = malloc(sizeof(double) * (size_t)(2 * I)), *row = malloc(sizeof(double) * (size_t)(d + I));
            double s_sel[32], g[32], dg[32];
            /* every token for the centroid gradient, else the listed ones */
            const int64_t n_all = need_dz ? T : (tok ? n_tok : T);
#pragma omp for schedule(dynamic, 1)
            for (int64_t n = 0; n < n_all; ++n) {
                const int64_t t = (need_dz || !tok) ? n : tok[n];
                int listed = 1;
                if (need_dz && tok) {
                    listed = 0;
                    for (int64_t m = 0; m < n_tok; ++m)
                        if (tok[m] == t) listed = 1;
                }
                const double *dO = dout + (size_t)t * d;
                const int32_t *sel = topk_idx + t * K;
                orow(U, t, d, xr);
                gates64(d, K, xr, E, sel, rs, s_sel, g, row);
                FP8_X(t, x);
                for (int c = 0; c < d; ++c) acc[c] = 0.0;
                for (int j = 0; j < K + Ns; ++j) {
                    const int routed = j < K, e = routed ? sel[j] : j - K;
                    if (!routed && !(listed && need_tok)) break;
                    const uint8_t *cg = (routed ? rwg : swg) + (size_t)e * wm, *cu = (routed ? rwu : swu) + (size_t)e * wm;
                    const uint8_t *cd = (routed ? rwd : swd) + (size_t)e * wm;
                    const float *sg = (routed ? rwg_s : swg_s) + (size_t)e * sm, *su = (routed ? rwu_s : swu_s) + (size_t)e * sm;
                    const float *sd = (routed ? rwd_s : swd_s) + (size_t)e * sm;
                    fp8_pair(d, I, cg, cu, cd, sg, su, sd, x, routed ? g[j] : 1.0, dO, a, b, hq, y, dy, da, db, dx,
                             wrow, t2);
                    if (routed) dg[j] = dot(dO, y, d);
                    for (int c = 0; c < d; ++c) acc[c] += dx[c];
                }
                double den = 0.0, sdg = 0.0;
                for (int j = 0; j < K; ++j) { den += s_sel[j]; sdg += dg[j] * s_sel[j]; }
                for (int j = 0; j < K; ++j) {
                    const double dz = rs * (dg[j] / den - sdg / (den * den)) * s_sel[j] * (1.0 - s_sel[j]);
                    if (need_dz) dzall[t * K + j] = dz;
                    if (listed && need_tok) {
                        orow(E, sel[j], d, row);
                        for (int c = 0; c < d; ++c) acc[c] += dz * row[c];
                    }
                }
                if (listed && du)
                    for (int c = 0; c < d; ++c) du[(size_t)t * d + c] = acc[c];
                if (listed && dtopk_w)
                    for (int j = 0; j < K; ++j) dtopk_w[t * K + j] = dg[j];
            }
            free(x); free(xr); free(a); free(b); free(hq); free(y); free(dy); free(da); free(db); free(dx);
            free(acc); free(wrow); free(t2); free(row);
        }
    }
    if (need_dz) {
        for (size_t q = 0; q < (size_t)Nr * d; ++q) dgate_w[q] = 0.0;
        for (int64_t t = 0; t < T; ++t)          /* tokens in order: fixed summation order */
            for (int j = 0; j < K; ++j) {
                double *de = dgate_w + (size_t)topk_idx[t * K + j] * d;
                for (int c = 0; c < d; ++c) de[c] += dzall[t * K + j] * load_plain(OR_BF16, u, t * d + c);
            }
        free(dzall);
    }
    /* Wgrad: per expert, the rows' dy, hq, da, db and x, re-tiled 128 x 1, then the outer products */
    for (int pass = 0; pass < 2; ++pass) {
        const int nE = pass == 0 ? (exps ? n_exp : (drwg ? Nr : 0)) : (dswg ? Ns : 0);
        for (int q = 0; q < nE; ++q) {
            const int e = pass == 0 ? (exps ? exps[q] : q) : q;
            const uint8_t *cg = (pass ? swg : rwg) + (size_t)e * wm, *cu = (pass ? swu : rwu) + (size_t)e * wm;
            const uint8_t *cd = (pass ? swd : rwd) + (size_t)e * wm;
            const float *sg = (pass ? swg_s : rwg_s) + (size_t)e * sm, *su = (pass ? swu_s : rwu_s) + (size_t)e * sm;
            const float *sd = (pass ? swd_s : rwd_s) + (size_t)e * sm;
            double *gwg = (pass ? dswg : drwg) + q * wm, *gwu = (pass ? dswu : drwu) + q * wm;
            double *gwd = (pass ? dswd : drwd) + q * wm;
            int64_t nt = 0;
            int64_t *tl = malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
            int *jl = malloc(sizeof(int) * (size_t)(T > 0 ? T : 1));
            for (int64_t t = 0; t < T; ++t) {
                if (pass) { tl[nt] = t; jl[nt++] = -1; continue; }
                for (int j = 0; j < K; ++j)
                    if (topk_idx[t * K + j] == e) { tl[nt] = t; jl[nt++] = j; }
            }
            /* per row: x[d], dy[d], hq[I], da[I], db[I] */
            const size_t per = 2 * (size_t)d + 3 * (size_t)I;
            double *buf = malloc(sizeof(double) * per * (size_t)(nt > 0 ? nt : 1));
#pragma omp parallel
            {
                const int mx = d > I ? d : I;
                double *a = malloc(sizeof(double) * (size_t)I), *b = malloc(sizeof(double) * (size_t)I);
                double *y = malloc(sizeof(double) * (size_t)d), *dx = malloc(sizeof(double) * (size_t)d);
                double *wrow = malloc(sizeof(double) * (size_t)mx), *t2 = malloc(sizeof(double) * (size_t)(2 * I));
                double *xr = malloc(sizeof(double) * (size_t)d), *row = malloc(sizeof(double) * (size_t)(d + I));
                double s_sel[32], g[32];
#pragma omp for schedule(dynamic, 1)
                for (int64_t n = 0; n < nt; ++n) {
                    const int64_t t = tl[n];
                    double *x = buf + per * n, *dy = x + d, *hq = dy + d, *da = hq + I, *db = da + I;
                    double gj = 1.0;
                    if (!pass) {
                        orow(U, t, d, xr);
                        gates64(d, K, xr, E, topk_idx + t * K, rs, s_sel, g, row);
                        gj = g[jl[n]];
                    }
                    FP8_X(t, x);
                    fp8_pair(d, I, cg, cu, cd, sg, su, sd, x, gj, dout + (size_t)t * d, a, b, hq, y, dy, da, db, dx,
                             wrow, t2);
                }
                free(a); free(b); free(y); free(dx); free(wrow); free(t2); free(xr); free(row);
            }
            /* 128 x 1 tiles along the expert's rows, column by column */
            q128x1_inplace(nt, d, buf, per);                 /* x  */
            q128x1_inplace(nt, d, buf + d, per);             /* dy */
            q128x1_inplace(nt, I, buf + 2 * d, per);         /* hq */
            q128x1_inplace(nt, I, buf + 2 * d + I, per);     /* da */
            q128x1_inplace(nt, I, buf + 2 * d + 2 * I, per); /* db */
#pragma omp parallel for schedule(static)
            for (int c = 0; c < d; ++c)
                for (int k = 0; k < I; ++k) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < nt; ++n) acc += buf[per * n + d + c] * buf[per * n + 2 * d + k];
                    gwd[(size_t)c * I + k] = acc;
                }
#pragma omp parallel for schedule(static)
            for (int k = 0; k < I; ++k)
                for (int c = 0; c < d; ++c) {
                    double ag = 0.0, au = 0.0;
                    for (int64_t n = 0; n < nt; ++n) {
                        const double xc = buf[per * n + c];
                        ag += buf[per * n + 2 * d + I + k] * xc;
                        au += buf[per * n + 2 * d + 2 * I + k] * xc;
                    }
                    gwg[(size_t)k * d + c] = ag;
                    gwu[(size_t)k * d + c] = au;
                }
            free(buf); free(tl); free(jl);
        }
    }
#undef FP8_X
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
