/*
 * oracle.c -- plain, slow CPU reference ("the oracle") for the activation-sparse
 * gated FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: it is used by the tests, by the one-shot smoke check and by the
 * CPU-baseline leg of the benchmark.  It shares no code, header, table or
 * constant generator with the HIP library.
 *
 * What it computes (each function below names the passage it follows):
 *
 *  - Decode layer.  The gated FFN y = W_down (m (.) act(W_gate x + b) (.) (W_up x))
 *    evaluated only over the intermediate neurons whose mask bit m_j is set.
 *    Neuron j owns row j of W_gate, row j of W_up and column j of W_down
 *    (denseflux, section 1 "Vi sao la FFN"); a neuron whose activation is zero
 *    contributes nothing (same section, and section 5.2).  The mask comes from
 *      ALL    every neuron (the dense FFN),
 *      EXACT  ReLU exact gating: neurons whose offset pre-activation is > 0
 *             (denseflux, sections 3 and 5.1),
 *      THRESH a threshold on |SiLU(W_gate x)| (denseflux, section 4.1; WiSparse
 *             notes, section 1.2), taken in the gate domain as g > theta,
 *      TOPK   weight-aware top-k on |a_j| * ||W_down[:, j]||_2 with
 *             k = max(1, floor(n * ratio)) and ties to the lower index
 *             (WiSparse notes, sections 2.3 and 3.2),
 *    and for a batch, optionally the union of the tokens' sets (WiSparse notes,
 *    section 5, the batch > 1 row of the troubleshooting table).
 *  - Prefill, token-selective (RedKnot article, Algorithm 1 under "why the FFN is
 *    the hidden bottleneck" and the section on token-selective sparse FFN):
 *    importance = L2 norm of each token's attention output; top-P by cumulative
 *    mass in descending order; the last recent_n tokens always kept; at least
 *    min_keep tokens; an all-zero score row or mass >= 1 means dense;
 *    X_next = Y + Z with Z = FFN(Y) on the kept rows and 0 elsewhere.
 *  - Block-granular token selection over a batch of sequences (RedKnot
 *    article, section on token-selective sparse FFN: at least min_keep tokens
 *    per sequence; and the closing paragraph of the section on adaptive expert
 *    top-K: bounds min_full_ratio / max_full_ratio on the kept fraction and a
 *    fixed-budget top-K over 128-token blocks, so the kept rows form a few
 *    contiguous runs).  The three-tier layer schedule of the same section
 *    (dense_until, deep_layer_start, mass_thresh_deep) picks each layer's mass.
 *  - Neuron order by activation frequency (WiSparse notes, section 5: count how
 *    often each neuron is active and store the neurons sorted by that count).
 *  - Adaptive expert top-K (RedKnot article, section on adaptive expert top-K):
 *    per token, rank the routed experts by routing probability and keep the
 *    smallest bucket of the top-ranked experts whose probability mass reaches
 *    the threshold (default 0.50 over buckets 3..6); the per-depth schedule
 *    caps the largest bucket.
 *
 * Precision.  Every output value is computed in fp64 from the exact fp32
 * values of the inputs (bf16 and int4*fp16 weights convert to fp32 exactly).
 * Every floating-point quantity that decides an integer (which neurons or
 * tokens are selected) is computed in the precision and the fixed summation
 * order that the GPU kernels also use, so that both sides take the same
 * decision:
 *   C1  gate / up dot products, the RMSNorm sum of squares and the token
 *       sums of squares are fp32: 64 partial accumulators, 16-byte chunk c
 *       (4 fp32, 8 bf16 or 32 int4 elements) folded into accumulator c mod 64
 *       in increasing c with fused multiply-adds, elements of a chunk in
 *       order (int4: t = sum q_e x_e from +0 by fma, then acc = fma(scale, t,
 *       acc)), then a halving tree: for off = 32, 16, ..., 1 accumulator p
 *       (p < off) adds accumulator p + off.
 *   C2  the weight-aware score is fp64: |silu(g) * u| * n_j, silu through the
 *       exp below, n_j = sqrt of the ascending fp64 sum of squares.
 *   C3  the token cumulative mass is fp64 in blocks of 256 sorted entries:
 *       sequential inside a block, block totals summed sequentially.
 *   C8  the expert cumulative mass is fp32, summed sequentially in rank order
 *       from the top-ranked expert.
 *   C9  block masses are fp64: the fp32 token scores of a block added in token
 *       order; the cumulative block mass is fp64, sequential in rank order.
 *       The block-count bounds are fp32 products: ceilf(nb * min_full_ratio),
 *       floorf(nb * max_full_ratio).
 *
 * Build: plain C99, -O2 -ffp-contract=off, no fast-math, optional OpenMP over
 * tokens / rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_I4 = 2 };
enum { ORA_RELU = 0, ORA_SILU = 1 };
enum { ORA_ALL = 0, ORA_EXACT = 1, ORA_THRESH = 2, ORA_TOPK = 3 };

#define ORA_GROUP 128

/* ------------------------------------------------------------------------ */
/* storage formats                                                           */
/* ------------------------------------------------------------------------ */

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary16 -> float, written from the format's definition. */
static float half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 31;
    int man = h & 1023;
    float v;
    if (ex == 0)
        v = ldexpf((float)man, -24); /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + man), ex - 25);
    return sign ? -v : v;
}

/* A weight matrix in its natural layout: row-major [rows][cols].
 * int4: packed [rows][cols/2], even column in the low nibble, two's
 * complement; scales [rows][cols/128] as binary16 bit patterns. */
typedef struct {
    int wt, rows, cols;
    const void *data;
    const uint16_t *scales;
} ora_mat;

static int q_at(const ora_mat *m, int r, int c)
{
    const uint8_t *b = (const uint8_t *)m->data;
    uint8_t byte = b[((size_t)r * m->cols + c) >> 1];
    int q = (c & 1) ? (byte >> 4) : (byte & 15);
    return q >= 8 ? q - 16 : q;
}

static float s_at(const ora_mat *m, int r, int c)
{
    return half_to_float(m->scales[(size_t)r * (m->cols / ORA_GROUP) + c / ORA_GROUP]);
}

/* exact fp32 value of element (r, c) */
static float w_at(const ora_mat *m, int r, int c)
{
    switch (m->wt) {
    case ORA_F32:
        return ((const float *)m->data)[(size_t)r * m->cols + c];
    case ORA_BF16:
        return bf16_to_float(((const uint16_t *)m->data)[(size_t)r * m->cols + c]);
    default:
        return (float)q_at(m, r, c) * s_at(m, r, c);
    }
}

static int chunk_elems(int wt) { return wt == ORA_F32 ? 4 : (wt == ORA_BF16 ? 8 : 32); }

/* ------------------------------------------------------------------------ */
/* C1: the fixed fp32 summation order used for every selection-deciding sum  */
/* ------------------------------------------------------------------------ */

static float halving_tree(float acc[64])
{
    for (int off = 32; off >= 1; off >>= 1)
        for (int p = 0; p < off; ++p)
            acc[p] = acc[p] + acc[p + off];
    return acc[0];
}

/* g = W[r, :] . x in the C1 order. */
float ora_dot_c1(int wt, int rows, int cols, const void *w, const uint16_t *scales,
                 int r, const float *x)
{
    ora_mat m = {wt, rows, cols, w, scales};
    float acc[64];
    for (int p = 0; p < 64; ++p) acc[p] = 0.0f;
    int E = chunk_elems(wt);
    int nch = cols / E;
    for (int c = 0; c < nch; ++c) {
        int p = c & 63;
        int c0 = c * E;
        if (wt == ORA_I4) {
            float t = 0.0f;
            for (int e = 0; e < E; ++e) t = fmaf((float)q_at(&m, r, c0 + e), x[c0 + e], t);
            acc[p] = fmaf(s_at(&m, r, c0), t, acc[p]);
        } else {
            for (int e = 0; e < E; ++e) acc[p] = fmaf(w_at(&m, r, c0 + e), x[c0 + e], acc[p]);
        }
    }
    return halving_tree(acc);
}

/* Sum of squares of an fp32 vector in the C1 order (chunks of 4). */
static float sumsq_f32_c1(const float *x, int d)
{
    float acc[64];
    for (int p = 0; p < 64; ++p) acc[p] = 0.0f;
    for (int c = 0; c < d / 4; ++c)
        for (int e = 0; e < 4; ++e) acc[c & 63] = fmaf(x[4 * c + e], x[4 * c + e], acc[c & 63]);
    return halving_tree(acc);
}

/* Sum of squares of a bf16 vector in the C1 order (chunks of 8). */
static float sumsq_bf16_c1(const uint16_t *a, int d)
{
    float acc[64];
    for (int p = 0; p < 64; ++p) acc[p] = 0.0f;
    for (int c = 0; c < d / 8; ++c)
        for (int e = 0; e < 8; ++e) {
            float v = bf16_to_float(a[8 * c + e]);
            acc[c & 63] = fmaf(v, v, acc[c & 63]);
        }
    return halving_tree(acc);
}

/* RMSNorm scale 1 / sqrt(mean(x^2) + eps), fp32, IEEE division and sqrt. */
float ora_rms_scale(const float *x, int d, float eps)
{
    float ss = sumsq_f32_c1(x, d);
    return 1.0f / sqrtf(ss / (float)d + eps);
}

/* ------------------------------------------------------------------------ */
/* C2: fp64 exp and SiLU for the weight-aware score                          */
/* ------------------------------------------------------------------------ */

/*
 * exp in fp64 by Cody-Waite argument reduction and a Taylor polynomial
 * (W. J. Cody and W. Waite, Software Manual for the Elementary Functions,
 * 1980): n = rint(z log2 e); r = z - n ln2 with ln2 split into a head with a
 * short significand and a tail, each step one fused multiply-add; then
 * e^r = sum_{k=0}^{13} r^k / k! in Horner form with fused multiply-adds
 * (|r| <= ln2/2, so the truncation error is below 2e-17 relative), scaled by
 * 2^n.  The coefficients are 1/k! rounded to the nearest double.
 */
double ora_exp64(double z)
{
    if (z > 709.0) return INFINITY;
    if (z < -745.0) return 0.0;
    const double log2e = 0x1.71547652b82fep+0;
    const double ln2_hi = 0x1.62e42feep-1;
    const double ln2_lo = 0x1.a39ef35793c76p-33;
    static const double inv_fact[14] = {
        0x1.0000000000000p+0,  0x1.0000000000000p+0,  0x1.0000000000000p-1,
        0x1.5555555555555p-3,  0x1.5555555555555p-5,  0x1.1111111111111p-7,
        0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13, 0x1.a01a01a01a01ap-16,
        0x1.71de3a556c734p-19, 0x1.27e4fb7789f5cp-22, 0x1.ae64567f544e4p-26,
        0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33};
    double n = rint(z * log2e);
    double r = fma(-n, ln2_hi, z);
    r = fma(-n, ln2_lo, r);
    double p = inv_fact[13];
    for (int k = 12; k >= 0; --k) p = fma(p, r, inv_fact[k]);
    return ldexp(p, (int)n);
}

double ora_silu64(double g) { return g / (1.0 + ora_exp64(-g)); }

/* weight-aware score |silu(g) * u| * n (WiSparse notes, section 2.3) */
double ora_score(float g, float u, double n)
{
    return fabs(ora_silu64((double)g) * (double)u) * n;
}

/* n_j = ||W_down[:, j]||_2 in fp64, ascending sum of squares, IEEE sqrt. */
void ora_down_col_norms(int wt, int d, int f, const void *wd, const uint16_t *sd, double *out)
{
    ora_mat m = {wt, d, f, wd, sd};
    for (int j = 0; j < f; ++j) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) {
            double w = (double)w_at(&m, i, j);
            s += w * w;
        }
        out[j] = sqrt(s);
    }
}

/* ------------------------------------------------------------------------ */
/* decode layer                                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    double s;
    int j;
} ranked;

/* order: score descending, index ascending */
static int cmp_ranked(const void *a, const void *b)
{
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static double act64(int act, double z)
{
    if (act == ORA_RELU) return z > 0.0 ? z : 0.0;
    return z / (1.0 + exp(-z));
}

/*
 * One gated-FFN layer for `rows` tokens.
 *
 * Inputs: weights in natural layout (W_gate, W_up [f][d], W_down [d][f]);
 * x fp32 [rows][d].  If rmsnorm, the FFN input is x_hat = x * rms_scale(x)
 * (fp32), else x itself.  The gate pre-activation is g' = fl32(g + bias),
 * with g in the C1 order.  Selection per token:
 *   ALL: every j;  EXACT: g'_j > 0;  THRESH: g'_j > theta;
 *   TOPK: the topk_k best j by (score desc, j asc), score = |silu(g') u| n_j
 *         with u in the C1 order.
 * With use_union the mask of every token is the union of the tokens' sets.
 *
 * Outputs:
 *   xhat  [rows][d]   FFN input (fp32), may be NULL
 *   g     [rows][f]   g' in the C1 order, may be NULL
 *   u     [rows][f]   u in the C1 order (TOPK only; else left untouched), may be NULL
 *   sel   [rows][f]   1 where the token's own selection holds, may be NULL
 *   used  [rows][f]   1 where the token's output sums neuron j, may be NULL
 *   y     [rows][d]   fp64: W_down (used (.) act(W_gate x_hat + b) (.) (W_up x_hat)),
 *                     plus x when residual is set.  Every dot product here is a
 *                     plain ascending fp64 sum.  NULL: the selection only (the
 *                     outputs are not computed).
 *   wdn   [f]         column norms used by TOPK, may be NULL
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int ora_decode(int wt, int d, int f, int act,
               const void *wg, const uint16_t *sg, const void *wu, const uint16_t *su,
               const void *wd, const uint16_t *sd,
               int rmsnorm, float eps, int residual,
               int mode, float bias, float theta, int topk_k, int use_union,
               int rows, const float *x,
               float *xhat_out, float *g_out, float *u_out, uint8_t *sel_out,
               uint8_t *used_out, double *y, double *wdn_out, int nthreads)
{
    if (rows < 0 || d <= 0 || f <= 0) return -1;
    if (mode == ORA_TOPK && (topk_k < 1 || topk_k > f)) return -1;
    ora_mat Mg = {wt, f, d, wg, sg}, Mu = {wt, f, d, wu, su}, Md = {wt, d, f, wd, sd};

    float *xh = (float *)malloc(sizeof(float) * (size_t)rows * d + 1);
    float *g = (float *)malloc(sizeof(float) * (size_t)rows * f + 1);
    float *u = (float *)malloc(sizeof(float) * (size_t)rows * f + 1);
    uint8_t *sel = (uint8_t *)calloc((size_t)rows * f + 1, 1);
    uint8_t *uni = (uint8_t *)calloc((size_t)f + 1, 1);
    double *wdn = (double *)malloc(sizeof(double) * (size_t)f + 1);
    if (!xh || !g || !u || !sel || !uni || !wdn) {
        free(xh); free(g); free(u); free(sel); free(uni); free(wdn);
        return -1;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    if (mode == ORA_TOPK) ora_down_col_norms(wt, d, f, wd, sd, wdn);

    /* FFN input and per-token selection */
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < rows; ++t) {
        const float *xt = x + (size_t)t * d;
        float *xht = xh + (size_t)t * d;
        if (rmsnorm) {
            float r = ora_rms_scale(xt, d, eps);
            for (int i = 0; i < d; ++i) xht[i] = xt[i] * r;
        } else {
            memcpy(xht, xt, sizeof(float) * (size_t)d);
        }
        float *gt = g + (size_t)t * f;
        float *ut = u + (size_t)t * f;
        uint8_t *st = sel + (size_t)t * f;
        for (int j = 0; j < f; ++j) gt[j] = ora_dot_c1(wt, f, d, wg, sg, j, xht) + bias;
        if (mode == ORA_TOPK) {
            ranked *rk = (ranked *)malloc(sizeof(ranked) * (size_t)f);
            for (int j = 0; j < f; ++j) {
                ut[j] = ora_dot_c1(wt, f, d, wu, su, j, xht);
                rk[j].s = ora_score(gt[j], ut[j], wdn[j]);
                rk[j].j = j;
            }
            qsort(rk, (size_t)f, sizeof(ranked), cmp_ranked);
            for (int k = 0; k < topk_k; ++k) st[rk[k].j] = 1;
            free(rk);
        } else {
            for (int j = 0; j < f; ++j) {
                int on;
                if (mode == ORA_ALL) on = 1;
                else if (mode == ORA_EXACT) on = gt[j] > 0.0f;
                else on = gt[j] > theta;
                st[j] = (uint8_t)on;
            }
        }
    }
    for (int t = 0; t < rows; ++t)
        for (int j = 0; j < f; ++j) uni[j] |= sel[(size_t)t * f + j];

    /* outputs in fp64 over the used neurons, ascending j */
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < (y ? rows : 0); ++t) {
        const float *xht = xh + (size_t)t * d;
        const uint8_t *use = use_union ? uni : sel + (size_t)t * f;
        double *yt = y + (size_t)t * d;
        double *h = (double *)calloc((size_t)f, sizeof(double));
        for (int j = 0; j < f; ++j) {
            if (!use[j]) continue;
            double g64 = 0.0, u64 = 0.0;
            for (int k = 0; k < d; ++k) {
                g64 += (double)w_at(&Mg, j, k) * (double)xht[k];
                u64 += (double)w_at(&Mu, j, k) * (double)xht[k];
            }
            h[j] = act64(act, g64 + (double)bias) * u64;
        }
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < f; ++j)
                if (use[j]) acc += h[j] * (double)w_at(&Md, i, j);
            yt[i] = residual ? acc + (double)x[(size_t)t * d + i] : acc;
        }
        free(h);
    }

    if (xhat_out) memcpy(xhat_out, xh, sizeof(float) * (size_t)rows * d);
    if (g_out) memcpy(g_out, g, sizeof(float) * (size_t)rows * f);
    if (u_out && mode == ORA_TOPK) memcpy(u_out, u, sizeof(float) * (size_t)rows * f);
    if (sel_out) memcpy(sel_out, sel, (size_t)rows * f);
    if (used_out)
        for (int t = 0; t < rows; ++t)
            memcpy(used_out + (size_t)t * f, use_union ? uni : sel + (size_t)t * f, (size_t)f);
    if (wdn_out && mode == ORA_TOPK) memcpy(wdn_out, wdn, sizeof(double) * (size_t)f);
    free(xh); free(g); free(u); free(sel); free(uni); free(wdn);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* token-selective prefill                                                   */
/* ------------------------------------------------------------------------ */

/* s_i = ||A_i||_2 with the sum of squares in the C1 order (fp32), IEEE sqrt. */
void ora_token_norms(const uint16_t *A, int L, int d, float *s, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int i = 0; i < L; ++i) s[i] = sqrtf(sumsq_bf16_c1(A + (size_t)i * d, d));
}

typedef struct {
    float s;
    int i;
} tok;

static int cmp_tok(const void *a, const void *b)
{
    const tok *x = (const tok *)a, *y = (const tok *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

#define ORA_MASS_BLOCK 256

/*
 * Token selection.  Sort tokens by (s desc, i asc); cum = the C3 blocked fp64
 * prefix of the sorted scores; total = cum[L-1]; P = the shortest prefix of the
 * sorted order with cum >= mass * total (empty when mass <= 0); S = P plus the
 * last recent_n tokens; then the highest-ranked tokens not yet in S are added
 * until |S| >= min_keep; mass >= 1 or total == 0 selects every token.  The
 * pages define the mass only for finite scores; a total that is not finite (a
 * NaN or infinite score) is read like the degenerate all-zero row: every token
 * is kept, so the FFN runs densely rather than on an arbitrary prefix.
 *
 * keep [L] receives S in ascending token order; returns |S| (or -1).
 * order [L] (optional) receives the sorted token order, cum [L] (optional) the
 * prefix.
 */
int ora_token_select(const float *s, int L, double mass, int recent_n, int min_keep,
                     int32_t *keep, int32_t *order, double *cum_out)
{
    if (L < 0 || recent_n < 0 || min_keep < 0) return -1;
    if (L == 0) return 0;
    tok *t = (tok *)malloc(sizeof(tok) * (size_t)L);
    double *cum = (double *)malloc(sizeof(double) * (size_t)L);
    uint8_t *in = (uint8_t *)calloc((size_t)L, 1);
    if (!t || !cum || !in) { free(t); free(cum); free(in); return -1; }
    for (int i = 0; i < L; ++i) { t[i].s = s[i]; t[i].i = i; }
    qsort(t, (size_t)L, sizeof(tok), cmp_tok);

    double block_base = 0.0;
    for (int b0 = 0; b0 < L; b0 += ORA_MASS_BLOCK) {
        double run = 0.0;
        int b1 = b0 + ORA_MASS_BLOCK < L ? b0 + ORA_MASS_BLOCK : L;
        for (int k = b0; k < b1; ++k) {
            run = run + (double)t[k].s;
            cum[k] = block_base + run;
        }
        block_base = block_base + run;
    }
    double total = cum[L - 1];

    if (mass >= 1.0 || total == 0.0 || !isfinite(total)) {
        for (int i = 0; i < L; ++i) in[i] = 1;
    } else {
        if (mass > 0.0) {
            double thr = mass * total;
            int m = 0;
            while (cum[m] < thr) ++m; /* cum[L-1] = total >= thr, so this stops */
            for (int k = 0; k <= m; ++k) in[t[k].i] = 1;
        }
        int r0 = L - recent_n;
        if (r0 < 0) r0 = 0;
        for (int i = r0; i < L; ++i) in[i] = 1;
        int cnt = 0;
        for (int i = 0; i < L; ++i) cnt += in[i];
        for (int k = 0; k < L && cnt < min_keep; ++k)
            if (!in[t[k].i]) { in[t[k].i] = 1; ++cnt; }
    }
    int n = 0;
    for (int i = 0; i < L; ++i)
        if (in[i]) keep[n++] = i;
    if (order)
        for (int k = 0; k < L; ++k) order[k] = t[k].i;
    if (cum_out) memcpy(cum_out, cum, sizeof(double) * (size_t)L);
    free(t); free(cum); free(in);
    return n;
}

/*
 * Block-granular token selection (RedKnot article: min_keep per sequence in
 * the section on token-selective sparse FFN; the token-level bounds and the
 * fixed-budget selection of 128-token blocks in the last paragraph of the
 * section on adaptive expert top-K).  The pages give the parts, not their
 * order; this is the plainest composition, the block analogue of
 * ora_token_select.  Sequence q holds tokens [cu[q], cu[q+1]); its nb blocks
 * of `block` consecutive tokens start at the sequence start (the last may be
 * short).  Per sequence:
 *   S_b   = sum of the block's scores (C9), blocks ranked by (S_b desc, b asc);
 *   c_k   = sum of the k top-ranked S_b (C9), total = c_nb;
 *   mass >= 1, total == 0 or a total that is not finite: every block;
 *   else K = smallest k with c_k >= mass * total (0 if mass <= 0), then
 *        K = max(min(K, floorf(nb * max_full)), ceilf(nb * min_full))
 *        (the lower bound wins when rounding crosses them), the top K blocks,
 *        plus every block holding one of the last recent_n tokens, plus
 *        further blocks in rank order while fewer than min(min_keep, Lq)
 *        tokens are kept.
 * keep receives the kept token indices of all sequences in ascending order;
 * returns their number, or -1 on bad arguments.
 */
typedef struct { double m; int b; } block_rank;

static int cmp_block(const void *a, const void *b)
{
    const block_rank *x = (const block_rank *)a, *y = (const block_rank *)b;
    if (x->m != y->m) return x->m > y->m ? -1 : 1;
    return x->b < y->b ? -1 : (x->b > y->b ? 1 : 0);
}

int ora_block_select(const float *s, int rows, const int32_t *cu, int nseq, int block, double mass,
                     float min_full, float max_full, int recent_n, int min_keep, int32_t *keep)
{
    if (rows < 0 || nseq < 1 || block < 1 || recent_n < 0 || min_keep < 0) return -1;
    if (!(min_full >= 0.0f && max_full <= 1.0f && min_full <= max_full)) return -1;
    if (cu[0] != 0 || cu[nseq] != rows) return -1;
    for (int q = 0; q < nseq; ++q)
        if (cu[q + 1] < cu[q]) return -1;
    int n = 0;
    for (int q = 0; q < nseq; ++q) {
        const int o0 = cu[q], Lq = cu[q + 1] - cu[q];
        if (Lq == 0) continue;
        const int nb = (Lq + block - 1) / block;
        block_rank *r = (block_rank *)malloc(sizeof(block_rank) * (size_t)nb);
        uint8_t *in = (uint8_t *)calloc((size_t)nb, 1);
        if (!r || !in) { free(r); free(in); return -1; }
        for (int b = 0; b < nb; ++b) {
            const int t1 = (b + 1) * block < Lq ? (b + 1) * block : Lq;
            double m = 0.0;
            for (int t = b * block; t < t1; ++t) m = m + (double)s[o0 + t];
            r[b].m = m;
            r[b].b = b;
        }
        qsort(r, (size_t)nb, sizeof(block_rank), cmp_block);
        double total = 0.0;
        for (int k = 0; k < nb; ++k) total = total + r[k].m;
        if (mass >= 1.0 || total == 0.0 || !isfinite(total)) {
            for (int b = 0; b < nb; ++b) in[b] = 1;
        } else {
            int K = 0;
            if (mass > 0.0) {
                const double thr = mass * total;
                double c = 0.0;
                while (K < nb) {
                    c = c + r[K].m;
                    ++K;
                    if (c >= thr) break;
                }
            }
            const int lo = (int)ceilf((float)nb * min_full);
            const int hi = (int)floorf((float)nb * max_full);
            if (K > hi) K = hi;
            if (K < lo) K = lo;
            for (int k = 0; k < K; ++k) in[r[k].b] = 1;
            if (recent_n > 0) {
                const int first = (Lq - recent_n > 0 ? Lq - recent_n : 0) / block;
                for (int b = first; b < nb; ++b) in[b] = 1;
            }
            const int need = min_keep < Lq ? min_keep : Lq;
            int kept = 0;
            for (int b = 0; b < nb; ++b)
                if (in[b]) kept += ((b + 1) * block < Lq ? block : Lq - b * block);
            for (int k = 0; k < nb && kept < need; ++k)
                if (!in[r[k].b]) {
                    const int b = r[k].b;
                    in[b] = 1;
                    kept += ((b + 1) * block < Lq ? block : Lq - b * block);
                }
        }
        for (int t = 0; t < Lq; ++t)
            if (in[t / block]) keep[n++] = o0 + t;
        free(r);
        free(in);
    }
    return n;
}

/*
 * Three-tier layer schedule (RedKnot article, section on token-selective
 * sparse FFN, the schedule table): layers below dense_until run dense (mass
 * 1), layers from dense_until up to deep_layer_start use mass_thresh, deeper
 * layers mass_thresh_deep.
 */
double ora_schedule_mass(int layer, int dense_until, int deep_layer_start, double mass_thresh,
                         double mass_thresh_deep)
{
    if (layer < dense_until) return 1.0;
    if (layer < deep_layer_start) return mass_thresh;
    return mass_thresh_deep;
}

/*
 * Adaptive expert top-K (RedKnot article, section on adaptive expert top-K:
 * the number of experts a token activates follows its routing probability
 * mass, threshold 0.50 over the candidate buckets 3, 4, 5, 6; confident tokens
 * take few experts, diffuse ones more).  Per token t, with p = probs[t][0..E):
 *   rank the experts by (p desc, index asc);
 *   c_b = the fp32 sum of the b top-ranked probabilities, added in rank order;
 *   K = the smallest b in [kmin, kmax] with c_b >= tau, or kmax if none.
 * k_out[t] = K; idx_out[t][0..kmax) = the top K experts in rank order then -1;
 * w_out[t][0..kmax) = their probabilities then 0.  Probabilities are >= 0.
 * Returns 0, or -1 on bad arguments.
 */
typedef struct { float p; int i; } expert_rank;

static int cmp_expert(const void *a, const void *b)
{
    const expert_rank *x = (const expert_rank *)a, *y = (const expert_rank *)b;
    if (x->p != y->p) return x->p > y->p ? -1 : 1;
    return x->i < y->i ? -1 : (x->i > y->i ? 1 : 0);
}

int ora_expert_select(const float *probs, int T, int E, float tau, int kmin, int kmax,
                      int32_t *k_out, int32_t *idx_out, float *w_out)
{
    if (T < 0 || E < 1 || kmin < 1 || kmax < kmin || kmax > E) return -1;
    expert_rank *r = (expert_rank *)malloc(sizeof(expert_rank) * (size_t)E);
    if (!r) return -1;
    for (int t = 0; t < T; ++t) {
        const float *p = probs + (size_t)t * E;
        for (int j = 0; j < E; ++j) { r[j].p = p[j]; r[j].i = j; }
        qsort(r, (size_t)E, sizeof(expert_rank), cmp_expert);
        int K = kmax;
        float c = 0.0f;
        for (int b = 1; b <= kmax; ++b) {
            c = c + r[b - 1].p;
            if (b >= kmin && c >= tau) { K = b; break; }
        }
        k_out[t] = K;
        for (int b = 0; b < kmax; ++b) {
            idx_out[(size_t)t * kmax + b] = b < K ? r[b].i : -1;
            w_out[(size_t)t * kmax + b] = b < K ? r[b].p : 0.0f;
        }
    }
    free(r);
    return 0;
}

/*
 * Z for the given rows of Y (bf16 [L][d]) through the SwiGLU FFN with bf16
 * weights in natural layout (W_gate, W_up [f][d]; W_down [d][f]), all in fp64:
 * Z_r = W_down (silu(W_gate y_r) (.) (W_up y_r)).  Z is [n][d].
 */
void ora_prefill_rows(int d, int f, const uint16_t *wg, const uint16_t *wu, const uint16_t *wd,
                      const uint16_t *Y, const int32_t *rows, int n, double *Z, int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n; ++r) {
        const uint16_t *yr = Y + (size_t)rows[r] * d;
        double *yv = (double *)malloc(sizeof(double) * (size_t)d);
        double *h = (double *)malloc(sizeof(double) * (size_t)f);
        double *z = Z + (size_t)r * d;
        for (int k = 0; k < d; ++k) yv[k] = (double)bf16_to_float(yr[k]);
        for (int j = 0; j < f; ++j) {
            double gs = 0.0, us = 0.0;
            const uint16_t *gj = wg + (size_t)j * d, *uj = wu + (size_t)j * d;
            for (int k = 0; k < d; ++k) {
                gs += (double)bf16_to_float(gj[k]) * yv[k];
                us += (double)bf16_to_float(uj[k]) * yv[k];
            }
            h[j] = gs / (1.0 + exp(-gs)) * us;
        }
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            const uint16_t *di = wd + (size_t)i * f;
            for (int j = 0; j < f; ++j) acc += (double)bf16_to_float(di[j]) * h[j];
            z[i] = acc;
        }
        free(yv);
        free(h);
    }
}

/* fp64 -> bf16 bit pattern, round to nearest, ties to even (finite inputs). */
uint16_t ora_bf16_rne(double v)
{
    /* bf16 has 8 significant bits; find the two neighbours and pick one. */
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    float lo_f = (float)v; /* any float, only used to seed the search */
    uint32_t u;
    memcpy(&u, &lo_f, 4);
    uint32_t base = u & 0xFFFF0000u; /* truncation toward zero of the float */
    /* candidates: base (toward zero) and base + 1 ulp(bf16) (away from zero) */
    float a, b;
    uint32_t ua = base, ub = base + 0x10000u;
    memcpy(&a, &ua, 4);
    memcpy(&b, &ub, 4);
    /* the truncated float may already be past v when (float)v rounded up */
    double da = fabs(v - (double)a), db = fabs((double)b - v);
    if (fabs((double)a) > fabs(v)) { /* step one back toward zero */
        ub = ua; ua = base - 0x10000u;
        memcpy(&a, &ua, 4);
        memcpy(&b, &ub, 4);
        da = fabs(v - (double)a);
        db = fabs((double)b - v);
    }
    uint32_t pick;
    if (da < db) pick = ua;
    else if (db < da) pick = ub;
    else pick = ((ua >> 16) & 1) ? ub : ua;
    return (uint16_t)(pick >> 16);
}

void ora_bf16_rne_array(const double *v, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; ++i) out[i] = ora_bf16_rne(v[i]);
}

/*
 * Neuron order by activation frequency (WiSparse notes, section 5, second
 * trick: sort the neurons by how often they are active).  counts[f] >= 0.
 *   mode 0 (cluster): perm = the neurons ranked by (count desc, index asc).
 *   mode 1 (balance): the same ranking handed out one neuron at a time to
 *     G = ceil(f / block) blocks of `block` positions (the last block holds
 *     the remainder), visiting the blocks 0..G-1, then G-1..0, then 0..G-1 and
 *     so on, and skipping a block that is full; each block lists its neurons
 *     in ascending index, the blocks follow each other in order.
 * Returns 0, or -1 on bad arguments.
 */
typedef struct { int32_t c; int32_t j; } neuron_rank;

static int cmp_neuron(const void *a, const void *b)
{
    const neuron_rank *x = (const neuron_rank *)a, *y = (const neuron_rank *)b;
    if (x->c != y->c) return x->c > y->c ? -1 : 1;
    return x->j < y->j ? -1 : (x->j > y->j ? 1 : 0);
}

static int cmp_int32(const void *a, const void *b)
{
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

int ora_frequency_order(const int32_t *counts, int f, int mode, int block, int32_t *perm)
{
    if (f < 1 || (mode != 0 && mode != 1) || (mode == 1 && (block < 1 || block > f))) return -1;
    neuron_rank *r = (neuron_rank *)malloc((size_t)f * sizeof *r);
    if (!r) return -1;
    for (int j = 0; j < f; ++j) {
        if (counts[j] < 0) { free(r); return -1; }
        r[j].c = counts[j];
        r[j].j = j;
    }
    qsort(r, (size_t)f, sizeof *r, cmp_neuron);
    if (mode == 0) {
        for (int k = 0; k < f; ++k) perm[k] = r[k].j;
        free(r);
        return 0;
    }
    const int G = (f + block - 1) / block;
    int *fill = (int *)calloc((size_t)G, sizeof *fill);
    if (!fill) { free(r); return -1; }
    /* block g owns perm[g * block .. g * block + size_g) */
    int g = 0, dir = 1;
    for (int k = 0; k < f; ++k) {
        for (;;) {
            const int size = g == G - 1 ? f - (G - 1) * block : block;
            const int here = g, room = fill[g] < size;
            /* step along the snake: ... G-2, G-1, G-1, G-2 ... 1, 0, 0, 1 ... */
            if (dir > 0) { if (g == G - 1) dir = -1; else ++g; }
            else { if (g == 0) dir = 1; else --g; }
            if (room) {
                perm[here * block + fill[here]] = r[k].j;
                ++fill[here];
                break;
            }
        }
    }
    for (int b = 0; b < G; ++b) {
        const int size = b == G - 1 ? f - (G - 1) * block : block;
        qsort(perm + (size_t)b * block, (size_t)size, sizeof *perm, cmp_int32);
    }
    free(fill);
    free(r);
    return 0;
}
