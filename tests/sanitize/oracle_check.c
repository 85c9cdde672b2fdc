/* The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure): every entry point on small, ragged and degenerate inputs
 * (each weight format, per-expert formats, shared experts, router bias and
 * router quantization, token subsets, given selections, tied logits, zero
 * rows). Results are checked elsewhere; this run checks memory and UB only,
 * plus the return codes. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float orc_fp16_round(float x);
double orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(float v);
int orc_quantize(int fmt, int N, int K, int group, const float *w, int8_t *q, float *scale, float *zero);
int orc_dequantize(int fmt, int N, int K, int group, const int8_t *q, const float *scale, const float *zero,
                   double *w);
int orc_route_f32(int T, int E, int k, int renorm, const float *logits, int32_t *idx, double *w, double *margin);
int orc_dispatch(int T, int E, int k, const int32_t *idx, int32_t *counts, int32_t *offsets, int32_t *perm,
                 int32_t *inv);
void *orc_layer_create(int d, int F, int E, int k, int S, int Fs, int fmt, int group, int renorm, int router_fp32,
                       int router_quant, const int *fmts, const void *w_router, const float *bias,
                       const float *const *wg, const float *const *wu, const float *const *wd, int *err);
void orc_layer_free(void *h);
int orc_layer_codes(void *h, int i, int matrix, int8_t *q, float *scale, float *zero);
int orc_forward(void *h, const uint16_t *x, int ntok, const int32_t *tok, const int32_t *given, double *y,
                double *logits_out, int32_t *idx_out, double *w_out, double *margin_out);

static uint32_t g_state = 777u;
static float draw(float scale)
{
    g_state = g_state * 1664525u + 1013904223u;
    return ((float)(g_state >> 8) * (1.0f / 8388608.0f) - 1.0f) * scale;
}
static uint16_t bf16_of(float v)   /* truncation: any bf16 pattern will do here */
{
    uint32_t u;
    memcpy(&u, &v, 4);
    return (uint16_t)(u >> 16);
}
static float *fill(size_t n, float scale)
{
    float *a = (float *)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; i++)
        a[i] = draw(scale);
    return a;
}

static int layer_case(int d, int F, int E, int k, int S, int Fs, int fmt, int renorm, int router_fp32, int rq,
                      int mixed, int with_bias, int T)
{
    const int n = E + S;
    float **wg = (float **)malloc(n * sizeof(float *)), **wu = (float **)malloc(n * sizeof(float *)),
          **wd = (float **)malloc(n * sizeof(float *));
    for (int i = 0; i < n; i++) {
        const int f = i < E ? F : Fs;
        wg[i] = fill((size_t)f * d, 0.02f);
        wu[i] = fill((size_t)f * d, 0.02f);
        wd[i] = fill((size_t)d * f, 0.02f);
    }
    float *wr32 = fill((size_t)E * d, 0.02f);
    uint16_t *wr16 = (uint16_t *)malloc((size_t)E * d * 2);
    for (size_t i = 0; i < (size_t)E * d; i++)
        wr16[i] = bf16_of(wr32[i]);
    float *bias = with_bias ? fill(E, 1.0f) : NULL;
    int *fmts = NULL;
    if (mixed) {
        fmts = (int *)malloc(n * sizeof(int));
        for (int i = 0; i < n; i++)
            fmts[i] = i % 5;
    }
    int err = 0, rc = 0;
    void *h = orc_layer_create(d, F, E, k, S, Fs, fmt, 128, renorm, router_fp32, rq, fmts,
                               router_fp32 ? (const void *)wr32 : (const void *)wr16, bias,
                               (const float *const *)wg, (const float *const *)wu, (const float *const *)wd, &err);
    if (!h)
        return 100 + err;
    uint16_t *x = (uint16_t *)malloc((size_t)T * d * 2);
    for (size_t i = 0; i < (size_t)T * d; i++)
        x[i] = bf16_of(draw(1.0f));
    memset(x, 0, (size_t)d * 2);   /* token 0: all-zero activations */
    double *y = (double *)malloc((size_t)T * d * sizeof(double)), *lg = (double *)malloc((size_t)T * E * 8),
           *w = (double *)malloc((size_t)T * k * 8), *m = (double *)malloc((size_t)T * 8);
    int32_t *idx = (int32_t *)malloc((size_t)T * k * 4);
    rc |= orc_forward(h, x, T, NULL, NULL, y, lg, idx, w, m);
    /* a token subset, in reverse order, and given selections for it */
    int32_t tok[3] = {T - 1, T / 2, 0};
    int32_t given[3 * 16];
    for (int t = 0; t < 3; t++)
        for (int j = 0; j < k; j++)
            given[t * k + j] = (t + j) % E;
    rc |= orc_forward(h, x, 3, tok, NULL, y, NULL, NULL, NULL, NULL);
    rc |= orc_forward(h, x, 3, tok, given, y, lg, idx, w, m);
    for (int i = 0; i < n; i++) {
        const int f = i < E ? F : Fs;
        for (int mat = 0; mat < 3; mat++) {
            const int N = mat < 2 ? f : d, K = mat < 2 ? d : f;
            int8_t *q = (int8_t *)malloc((size_t)N * K);
            float *s = (float *)malloc((size_t)N * K / 128 * 4 + 4 * N), *z = (float *)malloc((size_t)N * K / 128 * 4 + 4 * N);
            rc |= orc_layer_codes(h, i, mat, q, s, z);
            free(q);
            free(s);
            free(z);
        }
    }
    orc_layer_free(h);
    for (int i = 0; i < n; i++) {
        free(wg[i]);
        free(wu[i]);
        free(wd[i]);
    }
    free(wg); free(wu); free(wd); free(wr32); free(wr16); free(bias); free(fmts);
    free(x); free(y); free(lg); free(w); free(m); free(idx);
    return rc;
}

int main(void)
{
    int bad = 0;
    /* scalar format helpers over their whole domains */
    for (int c = 0; c < 256; c++)
        if (orc_e4m3_encode((float)orc_e4m3_decode((uint8_t)c)) > 255)
            bad++;
    const float specials[] = {0.0f, -0.0f, 1e-30f, 65504.0f, 70000.0f, 1e30f, -448.0f, 500.0f, 1e-9f};
    for (int i = 0; i < 9; i++) {
        (void)orc_fp16_round(specials[i]);
        (void)orc_e4m3_encode(specials[i]);
    }
    /* quantizer and dequantizer: every format, constant / zero / extreme rows */
    for (int fmt = 0; fmt < 5; fmt++) {
        const int N = 5, K = 384;
        float *wq = fill((size_t)N * K, 0.05f);
        for (int k2 = 0; k2 < K; k2++) {
            wq[k2] = 0.0f;
            wq[K + k2] = 0.25f;
            wq[2 * K + k2] = draw(1e4f);
            wq[3 * K + k2] = draw(1e-30f);
        }
        int8_t q[5 * 384];
        float s[5 * 3], z[5 * 3];
        double back[5 * 384];
        if (orc_quantize(fmt, N, K, 128, wq, q, s, z) || orc_dequantize(fmt, N, K, 128, q, s, z, back))
            bad++;
        free(wq);
    }
    /* routing: ties, k = E, k = 1, unrenormalised; dispatch of the result */
    {
        const int T = 9, E = 6;
        float lgt[9 * 6];
        for (int i = 0; i < T * E; i++)
            lgt[i] = (float)((i * 7) % 3);   /* many exact ties */
        int32_t idx[9 * 6], counts[6], offsets[7], perm[9 * 6], inv[9 * 6];
        double w[9 * 6], m[9];
        for (int k = 1; k <= E; k++)
            for (int renorm = 0; renorm < 2; renorm++) {
                bad += orc_route_f32(T, E, k, renorm, lgt, idx, w, m) != 0;
                bad += orc_dispatch(T, E, k, idx, counts, offsets, perm, inv) != 0;
            }
        bad += orc_route_f32(T, E, E + 1, 1, lgt, idx, w, m) == 0;   /* k > E is rejected */
    }
    /* layers */
    for (int fmt = 0; fmt < 5; fmt++)
        bad += layer_case(256, 384, 6, 2, 1, 256, fmt, 1, fmt == 0, 0, 0, fmt == 2, 11) != 0;
    bad += layer_case(256, 128, 5, 5, 0, 0, 2, 0, 0, 1, 0, 1, 4) != 0;   /* k = E, unrenormalised, INT8 router */
    bad += layer_case(256, 256, 10, 3, 2, 128, 2, 1, 1, 2, 1, 0, 7) != 0; /* per-expert formats, FP8 router */
    bad += layer_case(256, 128, 1, 1, 0, 0, 1, 1, 0, 0, 0, 0, 3) != 0;   /* one expert */
    printf(bad ? "FAILED %d\n" : "ok\n", bad);
    return bad ? 1 : 0;
}
