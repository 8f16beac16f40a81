/*
 * oracle_driver.c -- drives every function of the CPU oracle (oracle/nq_oracle.c) over small
 * random inputs and the edge cases of the method's parameters, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer can report any out-of-bounds access, leak,
 * overflow or other undefined behaviour in the oracle itself. Test infrastructure only.
 * Exit status 0 when the run completes (a sanitizer aborts it otherwise).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float nqo_h2f(uint16_t h);
uint16_t nqo_f2h_rne(float f);
uint16_t nqo_f2h_ceil(float v);
void nqo_rope_table(int32_t T, double base, float *C, float *S);
void nqo_layer_scores(const uint16_t *K, int32_t H, int32_t T, int32_t W, double *s);
int32_t nqo_keep_count(int32_t T, int32_t W, int32_t evict_permille);
int32_t nqo_select_layer(const double *s, int32_t T, int32_t W, int32_t evict_permille,
                         int32_t *positions, uint8_t *near, double *tau);
void nqo_rope_undo(const float *k, const float *C, const float *S, float *x);
void nqo_fwht_f32(float *x);
void nqo_fwht_f64(double *x);
double nqo_e8_margin(const float *u, const int8_t *c);
void nqo_e8_nearest(const float *u, int8_t *c);
void nqo_e8_nearest_many(const float *u, int64_t n_groups, int8_t *c, double *margin);
float nqo_group_u(const float *xg, uint16_t s16, int32_t bits, float *u);
int nqo_voronoi_near_tie(const float *u, const int8_t *c, float umax);
int nqo_scale_near_tie(float v, uint16_t h);
void nqo_quantize_row(const float *x, int32_t bits, uint16_t *s16, int8_t *c, uint8_t *flags);
void nqo_encode_layer(const uint16_t *K, const uint16_t *V, int32_t H, int32_t T,
                      const int32_t *positions, int32_t n_keep, const float *C, const float *S,
                      int32_t bits_k, int32_t bits_v, int8_t *codes_k, int8_t *codes_v,
                      uint16_t *scales_k, uint16_t *scales_v, uint8_t *flags_k, uint8_t *flags_v);
void nqo_decode_layer(const int8_t *codes_k, const int8_t *codes_v, const uint16_t *scales_k,
                      const uint16_t *scales_v, const int32_t *positions, int32_t n_keep,
                      int32_t H, const float *C, const float *S, double *K_out, double *V_out);
void nqo_attend_layer(const uint16_t *q, int32_t Hq, const double *K, const double *V,
                      int32_t H, int32_t n, double *out);
double nqo_nominal_ratio(int32_t H, int32_t T, int32_t n_keep, int32_t bits_k, int32_t bits_v);

static uint64_t st = 88172645463325252ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static double unif(void) { return (double)(rnd() >> 11) * 0x1p-53; }

/* exact-size heap buffers, so that any overrun lands in a redzone */
static void *buf(size_t n) { return malloc(n ? n : 1); }

static void layer_case(int32_t H, int32_t T, int32_t W, int32_t e, int32_t bk, int32_t bv,
                       double scale)
{
    size_t nrow = (size_t)H * T * 128;
    uint16_t *K = buf(nrow * 2), *V = buf(nrow * 2);
    for (size_t i = 0; i < nrow; i++) {
        K[i] = nqo_f2h_rne((float)((unif() - 0.5) * scale));
        V[i] = nqo_f2h_rne((float)((unif() - 0.5) * scale));
    }
    float *C = buf((size_t)T * 64 * 4), *S = buf((size_t)T * 64 * 4);
    nqo_rope_table(T, 1e4, C, S);
    double *s = buf((size_t)T * 8);
    nqo_layer_scores(K, H, T, W, s);
    int32_t n = nqo_keep_count(T, W, e);
    int32_t *pos = buf((size_t)n * 4);
    uint8_t *near = buf((size_t)T);
    double tau;
    int32_t got = nqo_select_layer(s, T, W, e, pos, near, &tau);
    if (got != n) { fprintf(stderr, "keep count %d != %d\n", got, n); exit(2); }
    size_t nc = (size_t)H * n * 128, ns = (size_t)H * n * 16;
    int8_t *ck = buf(nc), *cv = buf(nc);
    uint16_t *sk = buf(ns * 2), *sv = buf(ns * 2);
    uint8_t *fk = buf(ns), *fv = buf(ns);
    if (n > 0) {
        nqo_encode_layer(K, V, H, T, pos, n, C, S, bk, bv, ck, cv, sk, sv, fk, fv);
        double *Ko = buf(nc * 8), *Vo = buf(nc * 8);
        nqo_decode_layer(ck, cv, sk, sv, pos, n, H, C, S, Ko, Vo);
        int32_t Hq = 4 * H;
        uint16_t *q = buf((size_t)Hq * 128 * 2);
        for (int32_t i = 0; i < Hq * 128; i++) q[i] = nqo_f2h_rne((float)(unif() - 0.5));
        double *out = buf((size_t)Hq * 128 * 8);
        nqo_attend_layer(q, Hq, Ko, Vo, H, n, out);
        free(q);
        free(out);
        free(Ko);
        free(Vo);
    }
    (void)nqo_nominal_ratio(H, T, n > 0 ? n : 1, bk, bv);
    free(K); free(V); free(C); free(S); free(s); free(pos); free(near);
    free(ck); free(cv); free(sk); free(sv); free(fk); free(fv);
}

int main(void)
{
    /* binary16 conversions on every pattern and on special floats */
    volatile float sink = 0.0f;
    for (uint32_t h = 0; h < 65536; h++) sink += nqo_h2f((uint16_t)h) * 0.0f;
    const float sp[] = {0.0f, -0.0f, 1e-30f, 5.9e-8f, 6.1e-5f, 65504.0f, 65519.0f, 65520.0f,
                        1e10f, -1e10f, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof(sp) / sizeof(sp[0]); i++) {
        (void)nqo_f2h_rne(sp[i]);
        (void)nqo_f2h_ceil(sp[i]);
    }
    /* layers: edge cases of the parameters, then random shapes */
    const int32_t cases[][6] = {
        {1, 0, 0, 600, 3, 2}, {1, 1, 0, 600, 3, 2}, {2, 5, 10, 600, 3, 2}, {3, 40, 0, 600, 3, 2},
        {2, 97, 31, 777, 4, 4}, {1, 60, 16, 0, 2, 3}, {2, 60, 16, 1000, 3, 2},
        {8, 40, 3, 900, 3, 2}, {1, 300, 128, 600, 2, 2},
    };
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); i++)
        layer_case(cases[i][0], cases[i][1], cases[i][2], cases[i][3], cases[i][4], cases[i][5],
                   8.0);
    for (int k = 0; k < 20; k++)
        layer_case(1 + (int32_t)(rnd() % 4), (int32_t)(rnd() % 200), (int32_t)(rnd() % 40),
                   (int32_t)(rnd() % 1001), 2 + (int32_t)(rnd() % 3), 2 + (int32_t)(rnd() % 3),
                   k % 5 == 0 ? 1.3e5 : 4.0);
    /* rows through the quantizer: zeros, tiny, saturating, random; E8 on random points */
    float x[128], u[8];
    uint16_t s16[16];
    int8_t c[128];
    uint8_t fl[16];
    double m[16];
    for (int k = 0; k < 2000; k++) {
        double sc = k % 4 == 0 ? 0.0 : (k % 4 == 1 ? 1e-7 : (k % 4 == 2 ? 1e6 : 3.0));
        for (int i = 0; i < 128; i++) x[i] = (float)((unif() - 0.5) * sc);
        nqo_quantize_row(x, 2 + k % 3, s16, c, fl);
        (void)nqo_group_u(x, s16[0], 2 + k % 3, u);
        (void)nqo_voronoi_near_tie(u, c, 3.0f);
        (void)nqo_scale_near_tie(x[0] > 0 ? x[0] : -x[0], s16[0]);
        nqo_e8_nearest_many(x, 16, c, m);
        nqo_fwht_f32(x);
        double xd[128];
        for (int i = 0; i < 128; i++) xd[i] = x[i];
        nqo_fwht_f64(xd);
        float C[64], S[64], y[128];
        for (int i = 0; i < 64; i++) { C[i] = (float)cos(i); S[i] = (float)sin(i); }
        nqo_rope_undo(x, C, S, y);
    }
    printf("oracle driver ok %g\n", (double)sink);
    return 0;
}
