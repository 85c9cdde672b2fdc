/*
 * qmoe_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, double-precision CPU oracle of the forward pass of a top-k
 * routed Mixture-of-Experts SwiGLU FFN layer whose experts hold low-bit weights.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * it. It shares no code with the HIP library: no headers, helpers, tables or
 * constant generators; it is written from the source pages and the readings
 * listed below.
 *
 * Sources (web pages; cited by title and section):
 *  - "Quantized Mixture of Experts (Q-MoE)": section 3 components table
 *    (Gating Network = top-k routing, e.g. top-2; Expert Quantizer = per-expert
 *    precision INT8 / FP8 / mixed; Sparse Execution Engine = only the activated
 *    experts run), section 4 technical table (INT4/INT8 quantization).
 *  - "FineRMoE" (aitrends): architecture paragraph -- an expert is up, gate and
 *    down projection matrices with an activation between; shared experts sit
 *    beside the sparse ones; mixing weights are the router softmax probabilities.
 *  - IT Donga article on DREAM-MoE / SRA-MoE: DREAM-MoE section -- 16-bit to
 *    4-bit (and 3-bit) MoE weight quantization; routing flips under small
 *    perturbations (expert A 2.0 vs B 1.9 becoming 1.8 vs 1.9 picks B).
 *  - "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale":
 *    technical summary 2.1 (shared dense MLP, always active) and 2.2
 *    (expert-centric scheduling: collect tasks, group by expert id, sort by
 *    token id inside each group, grouped GEMM).
 *
 * Readings where the pages are silent:
 *  - selection is on the logits, lowest expert index wins ties; slot order is
 *    descending logit; weights are the softmax over the selected k (equal to
 *    the full softmax renormalised over the selection); renorm = 0 gives the
 *    unrenormalised full-softmax probability of each selected expert;
 *  - expert = SwiGLU: h = silu(W_gate x) * (W_up x), o = W_down h, no biases;
 *  - shared experts are always on, weight 1, same weight format;
 *  - the five weight formats and their rounding rules (fp32 arithmetic, round
 *    half to even, stored scale used for the codes, degenerate groups get
 *    scale 1 and zero codes).
 *
 * Everything the layer computes is evaluated in double precision; x (bf16) and
 * the router weight (bf16 or fp32) widen exactly. Quantization decisions are
 * taken in fp32, as the format rules fix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_INT8_SYM_CH 0
#define ORC_INT4_ASYM_G 1
#define ORC_INT4_SYM_G 2
#define ORC_INT3_SYM_G 3
#define ORC_FP8E4M3_CH 4

/* ------------------------------------------------------------------ */
/* Number formats                                                       */
/* ------------------------------------------------------------------ */

/* Nearest IEEE binary16 value to x (ties to even), returned as a float;
 * +-inf when x rounds past the largest finite half (65504). binary16 has 10
 * fraction bits, exponent range 2^-14 .. 2^15, subnormal quantum 2^-24. */
float orc_fp16_round(float x)
{
    if (x == 0.0f || isnan(x) || isinf(x))
        return x;
    double a = fabs((double)x);
    int e;
    frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1)  ->  2^(e-1) <= a < 2^e */
    int unbiased = e - 1;
    if (unbiased < -14)
        unbiased = -14;         /* subnormal range shares the quantum of 2^-14 */
    double quantum = ldexp(1.0, unbiased - 10);
    double r = rint(a / quantum) * quantum;   /* a/quantum is exact; rint is ties-to-even */
    if (r > 65504.0)
        r = INFINITY;
    return (float)(x < 0 ? -r : r);
}

/* Value of an OCP FP8 E4M3 ("e4m3fn") code: 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN, max 448. */
double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* (m/8) * 2^-6 */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 code to v (ties to even), saturating at +-448; the sign bit is
 * the sign of v (so -0.0 and small negatives that round to zero give 0x80). */
uint8_t orc_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    int e;
    double r;
    if (a == 0.0)
        return sign;
    frexp(a, &e);
    int unbiased = e - 1;
    if (unbiased < -6)
        unbiased = -6;                             /* subnormal quantum 2^-9 */
    double quantum = ldexp(1.0, unbiased - 3);
    r = rint(a / quantum) * quantum;
    if (r > 448.0)
        r = 448.0;
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6))                        /* subnormal: m * 2^-9 */
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    frexp(r, &e);
    int be = e - 1 + 7;                            /* biased exponent */
    int m = (int)((r / ldexp(1.0, e - 1) - 1.0) * 8.0);
    return sign | (uint8_t)(be << 3) | (uint8_t)m;
}

/* ------------------------------------------------------------------ */
/* Quantizers (fp32 decisions, round half to even)                    */
/* ------------------------------------------------------------------ */

static int is_group_format(int fmt)
{
    return fmt == ORC_INT4_ASYM_G || fmt == ORC_INT4_SYM_G || fmt == ORC_INT3_SYM_G;
}

static float clampf_(float v, float lo, float hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

/* Stored fp16 scale: nearest half, saturated to the largest finite half. */
static float half_scale(float s32)
{
    float s = orc_fp16_round(s32);
    if (isinf(s))
        s = 65504.0f;
    return s;
}

/* Quantize one matrix w[N][K] (row n = one output feature, K = input dim).
 * Group formats use groups of `group` consecutive k inside a row; scales and
 * zeros are [N][K/group]. Per-channel formats use [N]. Codes: signed integer
 * q for the symmetric formats, unsigned 0..15 for asymmetric INT4, the raw
 * E4M3 byte for FP8. Returns 0, or -1 if K is not a multiple of the group. */
int orc_quantize(int fmt, int N, int K, int group, const float *w, int8_t *q, float *scale, float *zero)
{
    if (is_group_format(fmt)) {
        if (group <= 0 || K % group != 0)
            return -1;
        int G = K / group;
        for (int n = 0; n < N; n++) {
            for (int g = 0; g < G; g++) {
                const float *wp = w + (size_t)n * K + (size_t)g * group;
                int8_t *qp = q + (size_t)n * K + (size_t)g * group;
                float s, z = 0.0f;
                if (fmt == ORC_INT4_ASYM_G) {
                    float mn = 0.0f, mx = 0.0f;
                    for (int i = 0; i < group; i++) {
                        if (wp[i] < mn) mn = wp[i];
                        if (wp[i] > mx) mx = wp[i];
                    }
                    s = half_scale((mx - mn) / 15.0f);
                    if (s == 0.0f) {
                        s = 1.0f;
                        for (int i = 0; i < group; i++) qp[i] = 0;
                    } else {
                        z = clampf_(rintf(-mn / s), 0.0f, 15.0f) + 0.0f;   /* +0.0 when mn == 0 */
                        for (int i = 0; i < group; i++)
                            qp[i] = (int8_t)clampf_(rintf(wp[i] / s) + z, 0.0f, 15.0f);
                    }
                } else {
                    float qmax = fmt == ORC_INT4_SYM_G ? 7.0f : 3.0f;
                    float amax = 0.0f;
                    for (int i = 0; i < group; i++)
                        if (fabsf(wp[i]) > amax) amax = fabsf(wp[i]);
                    s = half_scale(amax / qmax);
                    if (s == 0.0f) {
                        s = 1.0f;
                        for (int i = 0; i < group; i++) qp[i] = 0;
                    } else {
                        for (int i = 0; i < group; i++)
                            qp[i] = (int8_t)clampf_(rintf(wp[i] / s), -qmax - 1.0f, qmax);
                    }
                }
                scale[(size_t)n * G + g] = s;
                if (zero)
                    zero[(size_t)n * G + g] = z;
            }
        }
        return 0;
    }
    if (fmt != ORC_INT8_SYM_CH && fmt != ORC_FP8E4M3_CH)
        return -2;
    for (int n = 0; n < N; n++) {
        const float *wp = w + (size_t)n * K;
        int8_t *qp = q + (size_t)n * K;
        float amax = 0.0f;
        for (int i = 0; i < K; i++)
            if (fabsf(wp[i]) > amax) amax = fabsf(wp[i]);
        float s = amax / (fmt == ORC_INT8_SYM_CH ? 127.0f : 448.0f);
        if (s == 0.0f) {
            s = 1.0f;
            for (int i = 0; i < K; i++) qp[i] = 0;
        } else if (fmt == ORC_INT8_SYM_CH) {
            for (int i = 0; i < K; i++)
                qp[i] = (int8_t)clampf_(rintf(wp[i] / s), -127.0f, 127.0f);
        } else {
            for (int i = 0; i < K; i++)
                qp[i] = (int8_t)orc_e4m3_encode(wp[i] / s);
        }
        scale[n] = s;
        if (zero)
            zero[n] = 0.0f;
    }
    return 0;
}

/* W_hat[n][k] in double: (q - z) * s (asymmetric), q * s (symmetric),
 * value(q) * s (FP8). */
int orc_dequantize(int fmt, int N, int K, int group, const int8_t *q, const float *scale, const float *zero,
                   double *out)
{
    int G = is_group_format(fmt) ? K / group : 1;
    if (is_group_format(fmt) && (group <= 0 || K % group != 0))
        return -1;
    for (int n = 0; n < N; n++) {
        for (int k = 0; k < K; k++) {
            size_t i = (size_t)n * K + k;
            int g = is_group_format(fmt) ? k / group : 0;
            double s = scale[(size_t)n * G + g];
            double v;
            if (fmt == ORC_INT4_ASYM_G)
                v = ((double)q[i] - (double)zero[(size_t)n * G + g]) * s;
            else if (fmt == ORC_FP8E4M3_CH)
                v = orc_e4m3_decode((uint8_t)q[i]) * s;
            else
                v = (double)q[i] * s;
            out[i] = v;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Gating: top-k on logits, softmax weights                            */
/* ------------------------------------------------------------------ */

/* One token: pick the k largest logits, ties to the lowest expert index,
 * slots in descending order; weights = softmax over the selection (renorm=1)
 * or the full-softmax probability of each selected expert (renorm=0);
 * margin = k-th minus (k+1)-th largest logit (+inf when k == E).
 * If `given` is non-NULL the selection is taken from it instead. */
static void route_one(int E, int k, int renorm, const double *l, const int32_t *given, int32_t *idx, double *w,
                      double *margin, unsigned char *taken)
{
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; j++) {
        int best = -1;
        if (given) {
            best = given[j];
        } else {
            for (int e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
        }
        taken[best] = 1;
        idx[j] = best;
    }
    if (margin) {
        /* k-th largest minus (k+1)-th largest, both from the ordered logits */
        double kth = INFINITY, next = -INFINITY;
        unsigned char *sel = (unsigned char *)calloc((size_t)E, 1);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!sel[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            sel[best] = 1;
            kth = l[best];
        }
        for (int e = 0; e < E; e++)
            if (!sel[e] && l[e] > next)
                next = l[e];
        *margin = k < E ? kth - next : INFINITY;
        free(sel);
    }
    double m = l[idx[0]];
    for (int j = 1; j < k; j++)
        if (l[idx[j]] > m) m = l[idx[j]];
    double denom = 0.0;
    if (renorm) {
        for (int j = 0; j < k; j++)
            denom += exp(l[idx[j]] - m);
    } else {
        for (int e = 0; e < E; e++)
            if (l[e] > m) m = l[e];
        for (int e = 0; e < E; e++)
            denom += exp(l[e] - m);
    }
    for (int j = 0; j < k; j++)
        w[j] = exp(l[idx[j]] - m) / denom;
}

/* Routing from given fp32 logits [T][E] (widened exactly to double). */
int orc_route_f32(int T, int E, int k, int renorm, const float *logits, int32_t *idx, double *w, double *margin)
{
    if (k < 1 || k > E)
        return -1;
    #pragma omp parallel
    {
        double *l = (double *)malloc(sizeof(double) * (size_t)E);
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
        #pragma omp for schedule(static)
        for (int t = 0; t < T; t++) {
            for (int e = 0; e < E; e++)
                l[e] = (double)logits[(size_t)t * E + e];
            route_one(E, k, renorm, l, NULL, idx + (size_t)t * k, w + (size_t)t * k, margin ? margin + t : NULL,
                      taken);
        }
        free(l);
        free(taken);
    }
    return 0;
}

/* Expert-centric task list: counts per expert, exclusive-scan offsets [E+1],
 * perm[row] = pair id (t*k + j) with rows grouped by expert and, inside a
 * group, ordered by token id; inv[pair] = row. */
int orc_dispatch(int T, int E, int k, const int32_t *idx, int32_t *counts, int32_t *offsets, int32_t *perm,
                 int32_t *inv)
{
    memset(counts, 0, sizeof(int32_t) * (size_t)E);
    for (long p = 0; p < (long)T * k; p++) {
        if (idx[p] < 0 || idx[p] >= E)
            return -1;
        counts[idx[p]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            long p = (long)t * k + j;
            int e = idx[p];
            int row = offsets[e] + cursor[e]++;
            perm[row] = (int32_t)p;
            if (inv)
                inv[p] = row;
        }
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------ */
/* The layer                                                            */
/* ------------------------------------------------------------------ */

typedef struct {
    int fmt, group;
    int N, K;
    int8_t *q;
    float *scale, *zero;
} orc_matrix;

typedef struct {
    int d, F, E, k, S, Fs, fmt, group, renorm, router_fp32;
    double *w_router;   /* [E][d] widened */
    double *bias;       /* [E] or NULL */
    orc_matrix *gate, *up, *down;   /* E + S each */
} orc_layer;

static int quantize_matrix(orc_matrix *m, int fmt, int group, int N, int K, const float *w)
{
    int G = is_group_format(fmt) ? K / group : 1;
    m->fmt = fmt;
    m->group = group;
    m->N = N;
    m->K = K;
    m->q = (int8_t *)malloc((size_t)N * K);
    m->scale = (float *)malloc(sizeof(float) * (size_t)N * G);
    m->zero = (float *)malloc(sizeof(float) * (size_t)N * G);
    if (!m->q || !m->scale || !m->zero)
        return -3;
    return orc_quantize(fmt, N, K, group, w, m->q, m->scale, m->zero);
}

static void free_matrix(orc_matrix *m)
{
    free(m->q);
    free(m->scale);
    free(m->zero);
}

void orc_layer_free(void *h)
{
    orc_layer *L = (orc_layer *)h;
    if (!L)
        return;
    for (int i = 0; i < L->E + L->S; i++) {
        if (L->gate) free_matrix(&L->gate[i]);
        if (L->up) free_matrix(&L->up[i]);
        if (L->down) free_matrix(&L->down[i]);
    }
    free(L->gate);
    free(L->up);
    free(L->down);
    free(L->w_router);
    free(L->bias);
    free(L);
}

/* Build the oracle's own copy of a layer: quantize every expert matrix with the
 * oracle quantizer. w_router is [E][d] fp32 (router_fp32) or bf16 bit patterns.
 * router_quant 1 / 2 quantizes the router weight's values per expert row with
 * the oracle's INT8 / FP8 per-channel quantizer and routes with the dequantized
 * weight s_e * q_e (Q-MoE page, section 4: quantized routing); 0 routes with
 * the weight as given. fmts (NULL: every expert in fmt) gives each expert its
 * own format (Q-MoE page, section 3: the expert quantizer keeps a precision
 * per expert).
 * Weight arrays are [F][d] (gate, up) and [d][F] (down), E routed then S shared. */
void *orc_layer_create(int d, int F, int E, int k, int S, int Fs, int fmt, int group, int renorm, int router_fp32,
                       int router_quant, const int *fmts, const void *w_router, const float *bias,
                       const float *const *wg, const float *const *wu, const float *const *wd, int *err)
{
    orc_layer *L = (orc_layer *)calloc(1, sizeof(orc_layer));
    int rc = 0;
    L->d = d; L->F = F; L->E = E; L->k = k; L->S = S; L->Fs = Fs;
    L->fmt = fmt; L->group = group; L->renorm = renorm; L->router_fp32 = router_fp32;
    if (k < 1 || k > E) {
        *err = -1;
        free(L);
        return NULL;
    }
    L->w_router = (double *)malloc(sizeof(double) * (size_t)E * d);
    for (size_t i = 0; i < (size_t)E * d; i++) {
        if (router_fp32) {
            L->w_router[i] = ((const float *)w_router)[i];
        } else {
            uint32_t b = (uint32_t)((const uint16_t *)w_router)[i] << 16;
            float f;
            memcpy(&f, &b, 4);
            L->w_router[i] = f;
        }
    }
    if (router_quant == 1 || router_quant == 2) {
        /* the widened values are floats exactly: quantize them as a [E][d] matrix */
        orc_matrix r;
        float *wf = (float *)malloc(sizeof(float) * (size_t)E * d);
        for (size_t i = 0; i < (size_t)E * d; i++)
            wf[i] = (float)L->w_router[i];
        const int rfmt = router_quant == 1 ? ORC_INT8_SYM_CH : ORC_FP8E4M3_CH;
        rc = quantize_matrix(&r, rfmt, group, E, d, wf);
        if (rc == 0)
            rc = orc_dequantize(rfmt, E, d, group, r.q, r.scale, r.zero, L->w_router);
        free_matrix(&r);
        free(wf);
        if (rc != 0) {
            *err = rc;
            orc_layer_free(L);
            return NULL;
        }
    } else if (router_quant != 0) {
        *err = -1;
        orc_layer_free(L);
        return NULL;
    }
    if (bias) {
        L->bias = (double *)malloc(sizeof(double) * (size_t)E);
        for (int e = 0; e < E; e++)
            L->bias[e] = bias[e];
    }
    L->gate = (orc_matrix *)calloc((size_t)(E + S), sizeof(orc_matrix));
    L->up = (orc_matrix *)calloc((size_t)(E + S), sizeof(orc_matrix));
    L->down = (orc_matrix *)calloc((size_t)(E + S), sizeof(orc_matrix));
    #pragma omp parallel for schedule(dynamic) reduction(min : rc)
    for (int i = 0; i < E + S; i++) {
        int f = i < E ? F : Fs;
        int fi = fmts ? fmts[i] : fmt;
        int r1 = quantize_matrix(&L->gate[i], fi, group, f, d, wg[i]);
        int r2 = quantize_matrix(&L->up[i], fi, group, f, d, wu[i]);
        int r3 = quantize_matrix(&L->down[i], fi, group, d, f, wd[i]);
        int r = r1 < r2 ? r1 : r2;
        r = r < r3 ? r : r3;
        if (r < rc) rc = r;
    }
    if (rc != 0) {
        *err = rc;
        orc_layer_free(L);
        return NULL;
    }
    *err = 0;
    return L;
}

/* Copy out the oracle's codes / scales / zeros of one matrix (0 gate, 1 up,
 * 2 down) of expert `i` (routed 0..E-1, shared E..E+S-1). */
int orc_layer_codes(void *h, int i, int matrix, int8_t *q, float *scale, float *zero)
{
    orc_layer *L = (orc_layer *)h;
    if (i < 0 || i >= L->E + L->S || matrix < 0 || matrix > 2)
        return -1;
    orc_matrix *m = matrix == 0 ? &L->gate[i] : matrix == 1 ? &L->up[i] : &L->down[i];
    int G = is_group_format(m->fmt) ? m->K / m->group : 1;
    memcpy(q, m->q, (size_t)m->N * m->K);
    memcpy(scale, m->scale, sizeof(float) * (size_t)m->N * G);
    if (zero)
        memcpy(zero, m->zero, sizeof(float) * (size_t)m->N * G);
    return 0;
}

static double silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* o += wt * W_down (silu(W_gate x) * (W_up x)), all dense double. */
static void swiglu_expert(int d, int f, const double *Wg, const double *Wu, const double *Wd, const double *x,
                          double wt, double *h, double *o)
{
    for (int r = 0; r < f; r++) {
        double g = 0.0, u = 0.0;
        const double *wg = Wg + (size_t)r * d, *wu = Wu + (size_t)r * d;
        for (int c = 0; c < d; c++) {
            g += wg[c] * x[c];
            u += wu[c] * x[c];
        }
        h[r] = silu(g) * u;
    }
    for (int c = 0; c < d; c++) {
        double acc = 0.0;
        const double *wd = Wd + (size_t)c * f;
        for (int r = 0; r < f; r++)
            acc += wd[r] * h[r];
        o[c] += wt * acc;
    }
}

static double *dequant_alloc(const orc_matrix *m)
{
    double *w = (double *)malloc(sizeof(double) * (size_t)m->N * m->K);
    if (w)
        orc_dequantize(m->fmt, m->N, m->K, m->group, m->q, m->scale, m->zero, w);
    return w;
}

/* Forward for `ntok` tokens of x ([T][d] bf16 patterns; token list `tok`, or
 * tokens 0..ntok-1 when NULL).
 *   y[ntok][d]         double output
 *   logits[ntok][E]    optional: x.W_r^T + bias in double
 *   idx/w[ntok][k]     optional: the selection and its weights
 *   margin[ntok]       optional: k-th minus (k+1)-th logit
 *   given[ntok][k]     optional: use this selection instead of the oracle's own
 *                      (weights still from the oracle logits)
 * Experts run expert-major: each selected expert is dequantized once and then
 * applied to all of its tokens, in token order. */
int orc_forward(void *h, const uint16_t *x, int ntok, const int32_t *tok, const int32_t *given, double *y,
                double *logits_out, int32_t *idx_out, double *w_out, double *margin_out)
{
    orc_layer *L = (orc_layer *)h;
    int d = L->d, E = L->E, k = L->k;
    double *X = (double *)malloc(sizeof(double) * (size_t)ntok * d);
    double *lg = (double *)malloc(sizeof(double) * (size_t)ntok * E);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)ntok * k);
    double *w = (double *)malloc(sizeof(double) * (size_t)ntok * k);
    if (!X || !lg || !idx || !w)
        return -3;

    #pragma omp parallel
    {
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
        #pragma omp for schedule(static)
        for (int i = 0; i < ntok; i++) {
            int t = tok ? tok[i] : i;
            double *xi = X + (size_t)i * d;
            for (int c = 0; c < d; c++) {
                uint32_t b = (uint32_t)x[(size_t)t * d + c] << 16;
                float f;
                memcpy(&f, &b, 4);
                xi[c] = f;
            }
            /* Gating network: one logit per expert */
            for (int e = 0; e < E; e++) {
                double acc = 0.0;
                const double *wr = L->w_router + (size_t)e * d;
                for (int c = 0; c < d; c++)
                    acc += xi[c] * wr[c];
                lg[(size_t)i * E + e] = acc + (L->bias ? L->bias[e] : 0.0);
            }
            route_one(E, k, L->renorm, lg + (size_t)i * E, given ? given + (size_t)i * k : NULL,
                      idx + (size_t)i * k, w + (size_t)i * k, margin_out ? margin_out + i : NULL, taken);
        }
        free(taken);
    }
    memset(y, 0, sizeof(double) * (size_t)ntok * d);

    size_t cap = (size_t)(ntok > 0 ? ntok : 1) * (size_t)k;
    int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * cap);
    int maxf = L->F > L->Fs ? L->F : L->Fs;
    for (int e = 0; e < E + L->S; e++) {
        int n = 0;
        if (e < E) {
            /* the task list of expert e, in token order */
            for (int i = 0; i < ntok; i++)
                for (int j = 0; j < k; j++)
                    if (idx[(size_t)i * k + j] == e) {
                        rows[n] = i;
                        slot[n] = j;
                        n++;
                    }
        } else {
            for (int i = 0; i < ntok; i++) {
                rows[n] = i;
                slot[n] = -1;
                n++;
            }
        }
        if (n == 0)
            continue;
        int f = e < E ? L->F : L->Fs;
        double *Wg = dequant_alloc(&L->gate[e]);
        double *Wu = dequant_alloc(&L->up[e]);
        double *Wd = dequant_alloc(&L->down[e]);
        if (!Wg || !Wu || !Wd)
            return -3;
        #pragma omp parallel
        {
            double *hbuf = (double *)malloc(sizeof(double) * (size_t)maxf);
            #pragma omp for schedule(dynamic, 1)
            for (int r = 0; r < n; r++) {
                int i = rows[r];
                double wt = slot[r] >= 0 ? w[(size_t)i * k + slot[r]] : 1.0;
                swiglu_expert(d, f, Wg, Wu, Wd, X + (size_t)i * d, wt, hbuf, y + (size_t)i * d);
            }
            free(hbuf);
        }
        free(Wg);
        free(Wu);
        free(Wd);
    }
    if (logits_out)
        memcpy(logits_out, lg, sizeof(double) * (size_t)ntok * E);
    if (idx_out)
        memcpy(idx_out, idx, sizeof(int32_t) * (size_t)ntok * k);
    if (w_out)
        memcpy(w_out, w, sizeof(double) * (size_t)ntok * k);
    free(rows);
    free(slot);
    free(X);
    free(lg);
    free(idx);
    free(w);
    return 0;
}
