/*
 * encode_arith.c -- host emulation of the GPU encode's fp32 arithmetic, checked against the
 * CPU oracle. Test infrastructure: the GPU library never sees this file, and the oracle's
 * functions are only called (linked from liboracle.so), never copied.
 *
 * The GPU encode ("Como comprimir o KV cache do seu LLM em 33x sem treino", Como funciona,
 * step 5: each group of 8 floats scaled and mapped to the nearest E8 point) takes its
 * integer decisions in fp32 with its own operation sequence. This program shows which of
 * them are exact and bounds the rest:
 *
 *   scale     a/rho as fma(a, h, a * l) with h = RN(1/rho), l = RN(1/rho - h): equal to the
 *             correctly rounded a/rho for every positive fp32 a whose quotient is at least
 *             2^-100, and zero exactly when it is, for rho in {1, 3, 7}     (exhaustive)
 *   fp16 up   the smallest binary16 >= q by integer rounding of q's bits (and ceil(q * 2^24)
 *             below 2^-14): equal to the oracle's rounding for every positive fp32 q
 *                                                                        (exhaustive)
 *   1/s       h = any fp32 within one ulp of 1/s (what v_rcp_f32 may return) and
 *             l = fma(-s, h, 1) * h: the fma is exact and h + l is 1/s to 2^-45 relative,
 *             for every positive finite binary16 s                      (exhaustive)
 *   u         fma(xn, h, xn * l) equals the correctly rounded xn / s for every fp32
 *             significand of xn, every binary16 significand of s and both h (exhaustive),
 *             and, over random exponents, for every quotient of at least 2^-100, with at most
 *             one ulp of difference below                               (random)
 *   E8        the kernel's decision (rint by a magic add, distance differences in fp32,
 *             arg-max/min on |e| keys whose 3 low bits hold the index) against the oracle's
 *             nearest point: every disagreement must fall inside the oracle's Voronoi
 *             near-tie band, and the GPU point must be a nearest point up to the band
 *                                                                        (random + crafted)
 * Output: one "name key=value ..." line per check; exit status 0 when every check holds.
 * Usage: encode_arith [n_random] [n_crafted] [division_significand_stride]
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle (liboracle.so) */
float nqo_h2f(uint16_t h);
uint16_t nqo_f2h_ceil(float v);
void nqo_quantize_row(const float *x, int32_t bits, uint16_t *s16, int8_t *c, uint8_t *flags);
void nqo_e8_nearest(const float *u, int8_t *c);
double nqo_e8_margin(const float *u, const int8_t *c);
float nqo_group_u(const float *xg, uint16_t s16, int32_t bits, float *u);
int nqo_voronoi_near_tie(const float *u, const int8_t *c, float umax);

static uint32_t fbits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static float bitsf(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

/* ---- the kernel's sequences, restated -------------------------------------------------- */
/* rest of 1/rho as the host side computes it */
static float k_rho_inv_lo(float rho, float rinv) { return (float)(1.0 / (double)rho - (double)rinv); }

static float k_scale_quotient(float a, float rinv, float rinv_lo)
{
    return fmaf(a, rinv, a * rinv_lo);
}

/* the smallest binary16 >= q (q >= 0), saturating at 65504: fp16 bits */
static uint32_t k_f16_ceil(float q)
{
    uint32_t sb32 = (fbits(q) + 0x1fffu) & 0xffffe000u;
    if (sb32 > 0x477fe000u) sb32 = 0x477fe000u;
    uint32_t s16 = (sb32 >> 13) - 0x1c000u;
    if (q < 0x1p-14f) s16 = (uint32_t)ceilf(q * 0x1p24f);
    return s16 & 0xffffu;
}

/* rest of 1/s from h */
static float k_recip_lo(float s, float h) { return fmaf(-s, h, 1.0f) * h; }

static float k_quotient(float xn, float h, float l) { return fmaf(xn, h, xn * l); }

/* the fp32 neighbour of RN(1/s) on the other side of 1/s (above it when 1/s is exact): with
 * RN(1/s), the values a reciprocal accurate to one ulp may return */
static float other_recip(float s)
{
    float r = 1.0f / s;
    return bitsf(fbits(r) + ((double)r > 1.0 / (double)s ? (uint32_t)-1 : 1u));
}

/* e8_nearest_code: codes c = 2y */
static void k_e8(const float u[8], int8_t c[8])
{
    const float M = 12582944.0f;   /* 1.5 * 2^23 + 32 */
    float e[8], Sa = 0.0f;
    int B[8], N[8];
    uint32_t kmax = 0u, kmin = 0xffffffffu;
    for (int i = 0; i < 8; i++) {
        float t = u[i] + M;
        float g = M - t;
        e[i] = u[i] + g;
        B[i] = (int)(fbits(t) & 0xffu);              /* rint(u) + 32 */
        uint32_t key = (fbits(e[i]) & 0x7ffffff8u) | (uint32_t)i;
        if (key > kmax) kmax = key;
        if (key < kmin) kmin = key;
        Sa = Sa + fabsf(e[i]);
        N[i] = (int)(fbits(e[i]) >> 31);
    }
    int sb = 0, nn = 0;
    for (int i = 0; i < 8; i++) { sb += B[i]; nn += N[i]; }
    int P0 = sb & 1, P1 = P0 ^ (nn & 1);
    float amax = bitsf(kmax & ~7u), amin = bitsf(kmin & ~7u);
    float dd = 2.0f - Sa;
    if (P1) dd = fmaf(2.0f, amin, dd);
    if (P0) dd = fmaf(2.0f, amax, dd - 1.0f);
    int half = dd < 0.0f;
    int jf = (int)((half ? kmin : kmax) & 7u);
    int par = half ? P1 : P0;
    if (half)
        for (int i = 0; i < 8; i++) B[i] -= N[i];
    if (par) {
        int d = N[jf] ? -1 : 1;
        if (half) d = -d;
        B[jf] += d;
    }
    for (int i = 0; i < 8; i++) c[i] = (int8_t)(2 * B[i] + half - 64);
}

/* ---- exhaustive checks ------------------------------------------------------------------- */
static long check_scale_quotient(long *cases)
{
    long bad = 0, n = 0;
    const float rhos[3] = {1.0f, 3.0f, 7.0f};
    for (int k = 0; k < 3; k++) {
        float rho = rhos[k], rinv = 1.0f / rho, rlo = k_rho_inv_lo(rho, rinv);
        /* every positive finite fp32 */
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
        for (uint32_t b = 1; b < 0x7f800000u; b++) {
            float a = bitsf(b), want = a / rho, q = k_scale_quotient(a, rinv, rlo);
            n++;
            if (want >= 0x1p-100f ? q != want : (q == 0.0f) != (want == 0.0f)) bad++;
        }
    }
    *cases = n;
    return bad;
}

static long check_f16_ceil(void)
{
    long bad = 0;
    /* every positive fp32 up to the first value above 65504, then a few beyond */
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (uint32_t b = 1; b <= 0x477fe001u; b++) {
        float q = bitsf(b);
        if (k_f16_ceil(q) != nqo_f2h_ceil(q)) bad++;
    }
    const float big[4] = {65505.0f, 1e6f, 3.4e38f, 65504.5f};
    for (int i = 0; i < 4; i++)
        if (k_f16_ceil(big[i]) != nqo_f2h_ceil(big[i])) bad++;
    return bad;
}

/* every fp32 h within one ulp of 1/s, for every positive finite binary16 s: fma(-s, h, 1)
 * exact, and the largest |h + l - 1/s| * s */
static long check_recip(long *cases, double *worst)
{
    long bad = 0;
    *cases = 0;
    *worst = 0.0;
    for (uint32_t hb = 1; hb < 0x7c00u; hb++) {
        float s = nqo_h2f((uint16_t)hb);
        double want = 1.0 / (double)s;
        for (int d = -1; d <= 1; d++) {
            float h = bitsf(fbits(1.0f / s) + (uint32_t)d);
            if (fabs((double)h - want) > ldexp(1.0, ilogb(want) - 23)) continue;
            (*cases)++;
            if ((double)fmaf(-s, h, 1.0f) != 1.0 - (double)s * (double)h) bad++;
            double err = fabs(((double)h + (double)k_recip_lo(s, h)) * (double)s - 1.0);
            if (err > *worst) *worst = err;
        }
    }
    if (*worst > 0x1p-45) bad++;
    return bad;
}

/* every binary16 significand S (s in [1, 2)) and both candidate h against every fp32
 * significand of xn in [1, 2), the latter with the given stride (1 = exhaustive) */
static long check_quotient(uint32_t stride, long *cases)
{
    long bad = 0, n = 0;
#pragma omp parallel for reduction(+ : bad, n) schedule(dynamic)
    for (uint32_t S = 0; S < 1024; S++) {
        float s = 1.0f + (float)S / 1024.0f;
        const float hs[2] = {1.0f / s, other_recip(s)};
        for (int i = 0; i < 2; i++) {
            float h = hs[i], l = k_recip_lo(s, h);
            for (uint32_t m = 0; m < (1u << 23); m += stride) {
                float xn = bitsf(0x3f800000u + m);
                n++;
                if (k_quotient(xn, h, l) != xn / s) bad++;
            }
        }
    }
    *cases = n;
    return bad;
}

static uint64_t rng_state;
static uint64_t next_u64(void);

/* random xn over the whole fp32 range and random binary16 s (quotients from ~2^-165 up to a
 * few units): equal to xn / s at or above 2^-100, within one ulp below */
static long check_quotient_range(long n, long *below, long *below_differ)
{
    long bad = 0;
    *below = *below_differ = 0;
    for (long k = 0; k < n; k++) {
        uint32_t hb = 1u + (uint32_t)(next_u64() % 0x7bffu);
        float s = nqo_h2f((uint16_t)hb);
        float h = (next_u64() & 1) ? 1.0f / s : other_recip(s), l = k_recip_lo(s, h);
        /* |xn| up to 8 s, down to the smallest subnormal */
        int e = -150 + (int)(next_u64() % 154);
        float xn = (float)ldexp(1.0 + (double)(next_u64() >> 11) * 0x1p-53, e) * s;
        if (next_u64() & 1) xn = -xn;
        if (!(fabsf(xn) <= 8.0f * s)) continue;
        float want = xn / s, got = k_quotient(xn, h, l);
        if (fabsf(want) >= 0x1p-100f) {
            if (got != want) bad++;
        } else {
            (*below)++;
            if (got != want) {
                (*below_differ)++;
                int32_t d = (int32_t)fbits(got) - (int32_t)fbits(want);
                if (d > 1 || d < -1) bad++;
            }
        }
    }
    return bad;
}

/* ---- E8 decision ------------------------------------------------------------------------ */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double unif(void) { return (double)(next_u64() >> 11) * 0x1p-53; }
static double gauss(void)
{
    double a = unif(), b = unif();
    if (a < 1e-300) a = 1e-300;
    return sqrt(-2.0 * log(a)) * cos(6.283185307179586 * b);
}

typedef struct {
    long groups, differ, outside_band, gpu_not_nearest;
    long old_differ, old_outside_band;   /* the former u = raw * RN(c * rcp(s)), reported */
    double worst_margin_of_differing;   /* largest oracle facet distance / band among them */
} e8_stats;

/* one rotated group x8 through the kernel's scale, quotient and E8 step; compared with the
 * oracle's quantize_row on the same group */
static void one_group(const float x8[8], const float *raw8, int bits, e8_stats *st)
{
    float rho = (float)((1 << (bits - 1)) - 1), rinv = 1.0f / rho, rlo = k_rho_inv_lo(rho, rinv);
    float row[128];
    memset(row, 0, sizeof(row));
    memcpy(row, x8, sizeof(float) * 8);
    uint16_t s16o[16];
    int8_t co[128];
    uint8_t fl[16];
    nqo_quantize_row(row, bits, s16o, co, fl);
    float a = 0.0f;
    for (int i = 0; i < 8; i++) a = fmaxf(a, fabsf(x8[i]));
    uint32_t s16 = k_f16_ceil(k_scale_quotient(a, rinv, rlo));
    st->groups++;
    if (s16 != s16o[0]) { st->differ++; st->outside_band++; return; }   /* proven equal */
    if (s16 == 0) return;
    /* either reciprocal the kernel's v_rcp_f32 may return */
    float s = nqo_h2f((uint16_t)s16), u[8], uo[8];
    float h = (st->groups & 1) ? 1.0f / s : other_recip(s), l = k_recip_lo(s, h);
    for (int i = 0; i < 8; i++) {
        u[i] = k_quotient(x8[i], h, l);
        if (s16 == 0x7bffu) u[i] = fminf(fmaxf(u[i], -rho), rho);
    }
    float umax = nqo_group_u(x8, (uint16_t)s16, bits, uo);
    if (memcmp(u, uo, sizeof(u)) != 0) { st->differ++; st->outside_band++; return; }
    int8_t ck[8];
    if (raw8) {
        /* the former sequence, u = raw * RN(c * r) with r any fp32 within one ulp of 1/s (what
         * v_rcp_f32 returns): how often its point leaves the near-tie band */
        const float c = 0x1.6a09e6p-4f;
        for (int d = -1; d <= 1; d++) {
            float rr = bitsf(fbits(1.0f / s) + (uint32_t)d), f = c * rr, uold[8];
            for (int i = 0; i < 8; i++) {
                uold[i] = raw8[i] * f;
                if (s16 == 0x7bffu) uold[i] = fminf(fmaxf(uold[i], -rho), rho);
            }
            k_e8(uold, ck);
            if (memcmp(ck, co, 8) != 0) {
                st->old_differ++;
                if (!nqo_voronoi_near_tie(uo, co, umax)) st->old_outside_band++;
            }
        }
    }
    k_e8(u, ck);
    if (memcmp(ck, co, 8) == 0) return;
    st->differ++;
    double band = 1e-6 * (umax > 1.0f ? (double)umax : 1.0);
    double mo = nqo_e8_margin(u, co), mk = nqo_e8_margin(u, ck);
    if (!nqo_voronoi_near_tie(u, co, umax)) st->outside_band++;
    if (mk < -band) st->gpu_not_nearest++;
    if (mo / band > st->worst_margin_of_differing) st->worst_margin_of_differing = mo / band;
}

/* random rotated groups: Gaussian with occasional outlier-sized coordinates; raw = the
 * unnormalised rotated value, x = RN(raw / sqrt(128)) as the rotation leaves it */
static void run_random(long n, int bits, e8_stats *st)
{
    float x[8], raw[8];
    for (long k = 0; k < n; k++) {
        double sc = (k & 7) == 0 ? 8.0 : 1.0;
        for (int i = 0; i < 8; i++) {
            raw[i] = (float)(gauss() * sc * 11.3137);
            x[i] = raw[i] * 0x1.6a09e6p-4f;
        }
        one_group(x, raw, bits, st);
    }
}

/* the E8 step alone on a given u (the kernel's u equals the oracle's: see the quotient
 * check) */
static void one_u(const float u[8], int bits, e8_stats *st)
{
    float rho = (float)((1 << (bits - 1)) - 1), umax = 0.0f;
    for (int i = 0; i < 8; i++) umax = fmaxf(umax, fabsf(u[i]));
    if (umax > rho) return;
    int8_t ck[8], co[8];
    st->groups++;
    k_e8(u, ck);
    nqo_e8_nearest(u, co);
    if (memcmp(ck, co, 8) == 0) return;
    st->differ++;
    double band = 1e-6 * (umax > 1.0f ? (double)umax : 1.0);
    double mo = nqo_e8_margin(u, co), mk = nqo_e8_margin(u, ck);
    if (!nqo_voronoi_near_tie(u, co, umax)) st->outside_band++;
    if (mk < -band) st->gpu_not_nearest++;
    if (mo / band > st->worst_margin_of_differing) st->worst_margin_of_differing = mo / band;
}

static void random_lattice_point(int rho, double y[8])
{
    int half = (int)(next_u64() & 1), lim = half ? rho - 1 : rho, sum = 0;
    for (int i = 0; i < 8; i++) {
        int v = lim > 0 ? (int)(next_u64() % (uint64_t)(2 * lim + 1)) - lim : 0;
        y[i] = v + (half ? 0.5 : 0.0);
        sum += v;
    }
    if (sum & 1) y[0] += (y[0] > 0 ? -1.0 : 1.0);
}

static void random_root(double r[8])
{
    if (next_u64() & 1) {
        int i = (int)(next_u64() % 8), j = (int)(next_u64() % 7);
        if (j >= i) j++;
        for (int t = 0; t < 8; t++) r[t] = 0.0;
        r[i] = (next_u64() & 1) ? 1.0 : -1.0;
        r[j] = (next_u64() & 1) ? 1.0 : -1.0;
    } else {
        int neg = 0;
        for (int t = 0; t < 8; t++) {
            r[t] = (next_u64() & 1) ? 0.5 : -0.5;
            neg += r[t] < 0;
        }
        if (neg & 1) r[7] = -r[7];
    }
}

/* u near (or on) E8 Voronoi facets, near rounding boundaries of single coordinates, and with
 * near-equal rounding errors in two coordinates (the kernel's arg-max/min keys) */
static void run_crafted(long n, int bits, e8_stats *st)
{
    int rho = (1 << (bits - 1)) - 1;
    float u[8];
    double y[8], r[8];
    for (long k = 0; k < n; k++) {
        int kind = (int)(k % 3);
        if (kind == 0) {
            /* u = y + (1 - sqrt2 d) r / 2 (+ noise): facet distance ~d toward y + r; d = 0 is a
             * tie, otherwise log-uniform in [1e-10, 1e-5] */
            random_lattice_point(rho, y);
            random_root(r);
            double d = (k % 48 == 0) ? 0.0 : pow(10.0, -10.0 + 5.0 * unif());
            double lam = 1.0 - sqrt(2.0) * d;
            double noise = (k % 9 == 0) ? 0.0 : 1e-3;
            for (int t = 0; t < 8; t++)
                u[t] = (float)(y[t] + lam * r[t] / 2.0 + noise * (unif() - 0.5));
        } else if (kind == 1) {
            /* coordinates on or within a few ulps of half-integers */
            for (int t = 0; t < 8; t++) {
                double v = (double)((int)(next_u64() % (uint64_t)(2 * rho)) - rho) + 0.5;
                float f = (float)v;
                int ulps = (int)(next_u64() % 9) - 4;
                u[t] = (next_u64() % 3) ? bitsf(fbits(f) + (uint32_t)ulps) : (float)(2.0 * rho * (unif() - 0.5));
            }
        } else {
            /* two coordinates whose rounding errors differ by a few ulps */
            for (int t = 0; t < 8; t++) u[t] = (float)(2.0 * (rho - 0.5) * (unif() - 0.5));
            int a = (int)(next_u64() % 8), b = (int)(next_u64() % 7);
            if (b >= a) b++;
            float ea = (float)(0.5 * unif());
            float eb = bitsf(fbits(ea) + (uint32_t)((int)(next_u64() % 17) - 8));
            u[a] = rintf(u[a]) + ((next_u64() & 1) ? ea : -ea);
            u[b] = rintf(u[b]) + ((next_u64() & 1) ? eb : -eb);
        }
        one_u(u, bits, st);
    }
}

int main(int argc, char **argv)
{
    long n_random = argc > 1 ? atol(argv[1]) : 2000000;
    long n_crafted = argc > 2 ? atol(argv[2]) : 500000;
    uint32_t stride = argc > 3 ? (uint32_t)atol(argv[3]) : 1;
    int ok = 1;
    long bad, cases;

    bad = check_scale_quotient(&cases);
    printf("scale_quotient cases=%ld bad=%ld\n", cases, bad);
    ok &= bad == 0;
    bad = check_f16_ceil();
    printf("f16_ceil cases=%ld bad=%ld\n", (long)0x477fe001u + 4, bad);
    ok &= bad == 0;
    double worst;
    bad = check_recip(&cases, &worst);
    printf("reciprocal cases=%ld bad=%ld worst_rel_err=%.3g\n", cases, bad, worst);
    ok &= bad == 0;
    bad = check_quotient(stride, &cases);
    printf("quotient cases=%ld bad=%ld stride=%u\n", cases, bad, stride);
    ok &= bad == 0;
    long below, below_differ;
    bad = check_quotient_range(n_random * 4, &below, &below_differ);
    printf("quotient_range cases=%ld bad=%ld below_2^-100=%ld of_which_differ=%ld\n",
           n_random * 4, bad, below, below_differ);
    ok &= bad == 0;
    for (int bits = 2; bits <= 4; bits++) {
        e8_stats st;
        memset(&st, 0, sizeof(st));
        run_random(n_random, bits, &st);
        run_crafted(n_crafted, bits, &st);
        printf("e8 bits=%d groups=%ld differ=%ld outside_band=%ld gpu_not_nearest=%ld "
               "worst_margin_over_band=%.4f former_u_differ=%ld former_u_outside_band=%ld\n",
               bits, st.groups, st.differ, st.outside_band, st.gpu_not_nearest,
               st.worst_margin_of_differing, st.old_differ, st.old_outside_band);
        ok &= st.outside_band == 0 && st.gpu_not_nearest == 0;
    }
    printf("result %s\n", ok ? "ok" : "FAILED");
    return ok ? 0 : 1;
}
