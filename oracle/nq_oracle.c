/*
 * nq_oracle.c -- CPU oracle for the KV-cache compression hot path (key-key proxy scoring,
 * eviction, RoPE removal, Hadamard rotation, E8 lattice quantization, delta coding, and the
 * inverse reconstruction).
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's CPU-baseline
 * leg load this library; the GPU library never calls it, and the two share no code.
 *
 * Plain, sequential C, written from the method's description; every function names the passage
 * it follows. The pages cited are
 *   [NQ-zh] "NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破" (zingnex.cn forum thread)
 *   [NQ-pt] "Como comprimir o KV cache do seu LLM em 33x sem treino" (dev.to article)
 * and, for the nearest-point step, the textbook algorithm of Conway & Sloane, "Fast quantizing
 * and decoding algorithms for lattice quantizers and codes" (IEEE Trans. IT, 1982), D_n and
 * E_8 decoders.
 *
 * Precision:
 *   - proxy scores in fp64 (the window sum of fp16 keys is exact in fp64);
 *   - the encode front end (RoPE removal, Hadamard rotation, group scale, x/s) in fp32: it is
 *     the precision in which the GPU kernels take the same integer decisions (scales, codes);
 *   - the nearest E8 point of that fp32 vector is chosen by comparing fp64 squared distances
 *     (exact unless a coordinate is below 2^-29 in magnitude);
 *   - reconstruction and the attention check in fp64.
 * Built with -ffp-contract=off: no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HD 128          /* head_dim */
#define NG 16           /* 8-float groups per head row */
#define INV_SQRT128_F32 0x1.6a09e6p-4f /* fp32 nearest to 1/sqrt(128) */

/* ------------------------------------------------------------------------------------------
 * IEEE 754 binary16, from the format definition (1 sign, 5 exponent, 10 fraction bits).
 * ---------------------------------------------------------------------------------------- */
float nqo_h2f(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1f, man = h & 0x3ff;
    float v;
    if (ex == 0)
        v = ldexpf((float)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexpf((float)(man | 0x400), ex - 25);
    return sign ? -v : v;
}

/* nearest binary16, ties to even */
uint16_t nqo_f2h_rne(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;          /* rounds to infinity */
    if (a < ldexp(1.0, -14)) {                       /* subnormal range */
        double m = nearbyint(a * ldexp(1.0, 24));    /* 0..1024, 1024 = smallest normal */
        return sign | (uint16_t)m;
    }
    int e2;
    frexp(a, &e2);                                   /* a = fr * 2^e2, fr in [0.5, 1) */
    int E = e2 - 1;
    double m = nearbyint(ldexp(a, 10 - E));          /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    if (E + 15 >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024));
}

/* smallest binary16 >= v for finite v >= 0, saturating at the largest finite value 65504 */
uint16_t nqo_f2h_ceil(float v)
{
    if (!(v > 0.0f)) return 0;
    if (v > 65504.0f) return 0x7bff;
    uint16_t h = nqo_f2h_rne(v);
    if (nqo_h2f(h) < v) h = (uint16_t)(h + 1);       /* next binary16 up */
    return h;
}

/* ------------------------------------------------------------------------------------------
 * Rotary table. Split-half RoPE [NQ-zh "使用方法与兼容性"; NQ-pt "Modelos suportados"]: dims
 * i and i+64 form one rotation pair. Standard frequencies theta_i = base^(-2i/128); angles in
 * fp64, cos/sin rounded once to fp32. C, S: [T][64].
 * ---------------------------------------------------------------------------------------- */
void nqo_rope_table(int32_t T, double base, float *C, float *S)
{
    double theta[64];
    for (int i = 0; i < 64; i++) theta[i] = pow(base, -(double)i / 64.0);
    for (int32_t p = 0; p < T; p++)
        for (int i = 0; i < 64; i++) {
            double phi = (double)p * theta[i];
            C[(size_t)p * 64 + i] = (float)cos(phi);
            S[(size_t)p * 64 + i] = (float)sin(phi);
        }
}

/* ------------------------------------------------------------------------------------------
 * Key-key proxy score [NQ-zh "技术实现细节" (Key-Key proxy, no extra computation);
 * NQ-pt "Como funciona", step 1 (cross-head inner product)]. The recent window stands in for
 * the queries: qbar_h = sum over the last W keys of head h; a candidate's score is the sum over
 * heads of <qbar_h, k_{h,t}>, on the stored (rotated) keys, because RoPE removal comes after
 * eviction in the step order. Candidates are t in [1, T-W): BOS and the window are protected.
 * K: fp16 bits of one layer [H][T][128]; s: [T], entries outside the candidates set to NaN.
 * ---------------------------------------------------------------------------------------- */
void nqo_layer_scores(const uint16_t *K, int32_t H, int32_t T, int32_t W, double *s)
{
    double *qbar = (double *)calloc((size_t)H * HD, sizeof(double));
    int32_t w0 = T - W < 0 ? 0 : T - W;
    for (int32_t h = 0; h < H; h++)
        for (int32_t w = w0; w < T; w++)
            for (int i = 0; i < HD; i++)
                qbar[h * HD + i] += (double)nqo_h2f(K[((size_t)h * T + w) * HD + i]);
    for (int32_t t = 0; t < T; t++) s[t] = NAN;
    for (int32_t t = 1; t < T - W; t++) {
        double acc = 0.0;
        for (int32_t h = 0; h < H; h++)
            for (int i = 0; i < HD; i++)
                acc += qbar[h * HD + i] * (double)nqo_h2f(K[((size_t)h * T + t) * HD + i]);
        s[t] = acc;
    }
    free(qbar);
}

/* ------------------------------------------------------------------------------------------
 * Eviction [NQ-zh "Token淘汰机制" (drop the lowest-scoring tokens, always keep BOS and a recent
 * sliding window; 60% eviction gives 2.5x fewer tokens); NQ-pt "Como funciona", step 2].
 * n_evict = floor(evict_permille * T / 1000); n_keep = max(T - n_evict, |protected|).
 * ---------------------------------------------------------------------------------------- */
int32_t nqo_keep_count(int32_t T, int32_t W, int32_t evict_permille)
{
    if (T <= 0) return 0;
    int64_t n_evict = (int64_t)evict_permille * T / 1000;
    int64_t prot = (int64_t)W + 1 < T ? (int64_t)W + 1 : T;
    int64_t keep = T - n_evict;
    return (int32_t)(keep > prot ? keep : prot);
}

typedef struct { double s; int32_t t; } cand_t;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->s > b->s) return -1;        /* larger score first (+0 and -0 compare equal) */
    if (a->s < b->s) return 1;
    return (a->t > b->t) - (a->t < b->t);  /* equal scores: lower position first */
}

/* Keeps BOS, the window [max(1,T-W), T) and the m best candidates by (score desc, position
 * asc); writes the kept positions in ascending order and returns n_keep. If near is given,
 * near[t] = 1 marks candidates within 1e-6 relative of the m-th best score (eviction near-ties);
 * tau receives that score (NaN when no candidate is both kept and evicted). */
int32_t nqo_select_layer(const double *s, int32_t T, int32_t W, int32_t evict_permille,
                         int32_t *positions, uint8_t *near, double *tau)
{
    int32_t n_keep = nqo_keep_count(T, W, evict_permille);
    int32_t c_end = T - W;                              /* candidates: [1, c_end) */
    int32_t n_cand = c_end > 1 ? c_end - 1 : 0;
    int32_t prot = T - n_cand;
    int32_t m = n_keep - prot;
    uint8_t *keep = (uint8_t *)calloc(T > 0 ? T : 1, 1);
    for (int32_t t = 0; t < T; t++) keep[t] = (t == 0 || t >= c_end) ? 1 : 0;
    if (near) memset(near, 0, T > 0 ? T : 0);
    double th = NAN;
    if (n_cand > 0) {
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * n_cand);
        for (int32_t i = 0; i < n_cand; i++) { c[i].s = s[i + 1]; c[i].t = i + 1; }
        qsort(c, n_cand, sizeof(cand_t), cand_cmp);
        for (int32_t i = 0; i < m; i++) keep[c[i].t] = 1;
        if (m > 0 && m < n_cand) {
            th = c[m - 1].s;
            if (near)
                for (int32_t i = 0; i < n_cand; i++)
                    if (fabs(c[i].s - th) <= 1e-6 * fabs(th)) near[c[i].t] = 1;
        }
        free(c);
    }
    int32_t j = 0;
    for (int32_t t = 0; t < T; t++)
        if (keep[t]) positions[j++] = t;
    free(keep);
    if (tau) *tau = th;
    return j;
}

/* ------------------------------------------------------------------------------------------
 * RoPE removal on a kept key [NQ-zh "技术实现细节" (undo RoPE before quantization so the keys
 * share one subspace, restore afterwards); NQ-pt "Como funciona", step 3]. Rotation by -phi of
 * the split-half pairs (i, i+64): x_i = a*C + b*S, x_{i+64} = b*C - a*S, each product rounded
 * to fp32, then one add or subtract.
 * ---------------------------------------------------------------------------------------- */
void nqo_rope_undo(const float *k, const float *C, const float *S, float *x)
{
    for (int i = 0; i < 64; i++) {
        float a = k[i], b = k[i + 64];
        float ac = a * C[i], bs = b * S[i];
        float bc = b * C[i], as = a * S[i];
        x[i] = ac + bs;
        x[i + 64] = bc - as;
    }
}

/* ------------------------------------------------------------------------------------------
 * Normalised Hadamard rotation over head_dim = 128 [NQ-zh "E8格点量化" (Hadamard rotation
 * spreads energy evenly before the lattice step); NQ-pt "Como funciona", step 4]. Sylvester
 * order, no random signs: butterflies with half-width h = 1, 2, 4, ..., 64 in that order,
 * (a, b) -> (a + b, a - b) on pairs (j, j + h) inside blocks of 2h, then every element times
 * fp32(1/sqrt(128)).
 * ---------------------------------------------------------------------------------------- */
void nqo_fwht_f32(float *x)
{
    for (int h = 1; h < HD; h <<= 1)
        for (int j0 = 0; j0 < HD; j0 += 2 * h)
            for (int j = j0; j < j0 + h; j++) {
                float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
    for (int i = 0; i < HD; i++) x[i] = x[i] * INV_SQRT128_F32;
}

/* same butterflies in fp64; the normalised transform is its own inverse */
void nqo_fwht_f64(double *x)
{
    for (int h = 1; h < HD; h <<= 1)
        for (int j0 = 0; j0 < HD; j0 += 2 * h)
            for (int j = j0; j < j0 + h; j++) {
                double a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
    double c = 1.0 / sqrt(128.0);
    for (int i = 0; i < HD; i++) x[i] = x[i] * c;
}

/* ------------------------------------------------------------------------------------------
 * E8 nearest point [NQ-zh "E8格点量化" (groups of 8 floats mapped onto the E8 lattice);
 * NQ-pt "Como funciona", step 5 (E8 root lattice, densest 8-D packing)]. E8 = D8 u (D8 + 1/2),
 * D8 = integer vectors with even coordinate sum. Conway & Sloane: the nearest D8 point rounds
 * every coordinate and, if the sum is odd, re-rounds the coordinate with the largest rounding
 * error the other way; E8's nearest point is the nearer of D8(u) and D8(u - 1/2) + 1/2.
 * Exact-tie rules (measure zero): rint ties to even; lowest index among equal errors; a
 * coordinate with zero error moves toward zero (up from 0); D8(u) wins an exact distance tie.
 * ---------------------------------------------------------------------------------------- */
static void d8_nearest(const double *v, double *f)
{
    double sum = 0.0;
    for (int i = 0; i < 8; i++) { f[i] = nearbyint(v[i]); sum += f[i]; }
    if (fmod(sum, 2.0) != 0.0) {
        int j = 0;
        double best = -1.0;
        for (int i = 0; i < 8; i++) {
            double e = fabs(v[i] - f[i]);
            if (e > best) { best = e; j = i; }
        }
        if (v[j] > f[j]) f[j] += 1.0;
        else if (v[j] < f[j]) f[j] -= 1.0;
        else f[j] += (f[j] > 0.0) ? -1.0 : 1.0;
    }
}

/* Voronoi certificate: y is a nearest E8 point of u iff e.r <= |r|^2/2 = 1 for the 240 roots r
 * (E8's Voronoi-relevant vectors: permutations of (+-1,+-1,0^6) and (+-1/2)^8 with an even
 * number of minus signs). Returns the distance of e = u - y to the nearest Voronoi facet,
 * (1 - max_r e.r) / sqrt(2); negative means y is not a nearest point. */
double nqo_e8_margin(const float *u, const int8_t *c)
{
    double e[8], ae[8], sum_abs = 0.0, mn = INFINITY, m1 = 0.0, m2 = 0.0;
    int neg = 0;
    for (int i = 0; i < 8; i++) {
        e[i] = (double)u[i] - 0.5 * (double)c[i];
        ae[i] = fabs(e[i]);
        sum_abs += ae[i];
        if (ae[i] < mn) mn = ae[i];
        if (e[i] < 0.0) neg++;
        if (ae[i] > m1) { m2 = m1; m1 = ae[i]; }
        else if (ae[i] > m2) m2 = ae[i];
    }
    double t1 = m1 + m2;                                          /* (+-1,+-1,0^6) roots */
    double t2 = 0.5 * (sum_abs - ((neg & 1) ? 2.0 * mn : 0.0));   /* (+-1/2)^8 roots */
    double M = t1 > t2 ? t1 : t2;
    return (1.0 - M) / sqrt(2.0);
}

/* nearest E8 point of the fp32 vector u; writes c = 2y (int8) */
void nqo_e8_nearest(const float *u, int8_t *c)
{
    double v0[8], v1[8], y0[8], y1[8], d0 = 0.0, d1 = 0.0;
    for (int i = 0; i < 8; i++) { v0[i] = (double)u[i]; v1[i] = (double)u[i] - 0.5; }
    d8_nearest(v0, y0);
    d8_nearest(v1, y1);
    for (int i = 0; i < 8; i++) {
        y1[i] += 0.5;
        d0 += (v0[i] - y0[i]) * (v0[i] - y0[i]);
        d1 += (v0[i] - y1[i]) * (v0[i] - y1[i]);
    }
    const double *y = (d0 <= d1) ? y0 : y1;
    for (int i = 0; i < 8; i++) c[i] = (int8_t)(2.0 * y[i]);
}

void nqo_e8_nearest_many(const float *u, int64_t n_groups, int8_t *c, double *margin)
{
    for (int64_t g = 0; g < n_groups; g++) {
        nqo_e8_nearest(u + 8 * g, c + 8 * g);
        if (margin) margin[g] = nqo_e8_margin(u + 8 * g, c + 8 * g);
    }
}

/* ------------------------------------------------------------------------------------------
 * Group scale and lattice step for one Hadamard-rotated row, bit budget b [NQ-zh "E8格点量化"
 * (keys 3-bit, values 2-bit); NQ-pt "Os números" (ratios include the scales)]. Reading: per
 * 8-float group, absmax scaling to the radius rho_b = 2^(b-1) - 1, scale s = smallest fp16 >=
 * fp32(a / rho_b); u = clamp(x / s, -rho_b, rho_b) in fp32; a = 0 gives s = 0 and zero codes.
 * flags (optional, per group): bit 0 = Voronoi near-tie (facet distance below
 * 1e-6*max(1,|u|_inf)), bit 1 = scale near-tie (a/rho within 1e-6 relative of a binary16 step).
 * ---------------------------------------------------------------------------------------- */
static float h2f_next_down(uint16_t h) { return h == 0 ? 0.0f : nqo_h2f((uint16_t)(h - 1)); }

/* the radius rho_b = 2^(b-1) - 1 of a b-bit budget */
static float radius(int32_t bits) { return (float)((1 << (bits - 1)) - 1); }

/* the lattice-step input of one group at the fp16 scale s16: u_i = x_i / s (fp32, correctly
 * rounded), clamped to [-rho, rho] (the clamp only acts when the scale saturated); returns
 * max |u_i| */
float nqo_group_u(const float *xg, uint16_t s16, int32_t bits, float *u)
{
    float rho = radius(bits);
    float s = nqo_h2f(s16), umax = 0.0f;
    for (int i = 0; i < 8; i++) {
        float q = s16 ? xg[i] / s : 0.0f;
        if (q > rho) q = rho;
        if (q < -rho) q = -rho;
        u[i] = q;
        if (fabsf(q) > umax) umax = fabsf(q);
    }
    return umax;
}

/* Voronoi near-tie: the facet distance of u - c/2 below 1e-6 * max(1, |u|_inf) */
int nqo_voronoi_near_tie(const float *u, const int8_t *c, float umax)
{
    double lim = 1e-6 * (umax > 1.0f ? (double)umax : 1.0);
    return nqo_e8_margin(u, c) < lim;
}

/* Scale near-tie: v = fp32(a / rho) within 1e-6 relative of a binary16 value at which the
 * rounded-up scale changes: the scale h itself (v a little larger would give the next fp16)
 * or the fp16 value below it (v a little smaller would give that one). A saturated scale has
 * no upper step: every larger v keeps 65504. */
int nqo_scale_near_tie(float v, uint16_t h)
{
    double dv = (double)v, lo = (double)h2f_next_down(h), hi = (double)nqo_h2f(h);
    int near_lo = dv - lo <= 1e-6 * dv;
    int near_hi = h != 0x7bff && hi - dv <= 1e-6 * dv;
    return near_lo || near_hi;
}

void nqo_quantize_row(const float *x, int32_t bits, uint16_t *s16, int8_t *c, uint8_t *flags)
{
    float rho = radius(bits);
    for (int g = 0; g < NG; g++) {
        const float *xg = x + 8 * g;
        float a = 0.0f;
        for (int i = 0; i < 8; i++) a = fabsf(xg[i]) > a ? fabsf(xg[i]) : a;
        uint8_t fl = 0;
        if (a == 0.0f) {
            s16[g] = 0;
            for (int i = 0; i < 8; i++) c[8 * g + i] = 0;
        } else {
            float v = a / rho;
            uint16_t h = nqo_f2h_ceil(v);
            float u[8];
            float umax = nqo_group_u(xg, h, bits, u);
            s16[g] = h;
            nqo_e8_nearest(u, c + 8 * g);
            if (nqo_voronoi_near_tie(u, c + 8 * g, umax)) fl |= 1;
            if (nqo_scale_near_tie(v, h)) fl |= 2;
        }
        if (flags) flags[g] = fl;
    }
}

/* ------------------------------------------------------------------------------------------
 * Encode one compressed layer [NQ-pt "Como funciona", steps 3-6 in order; NQ-zh "E8格点量化"
 * (delta coding of consecutive tokens' lattice indices)]. For each kv head and each kept
 * position p (ascending): keys get RoPE removal at p, then keys and values get the Hadamard
 * rotation, group scales and E8 codes; codes are then delta-coded along the kept tokens per
 * (head, dim): d_0 = c_0, d_j = (c_j - c_{j-1}) mod 256 as int8.
 * K, V: fp16 bits [H][T][128]; positions [n_keep]; C, S: [T][64];
 * codes_*: int8 [H][n_keep][128]; scales_*: fp16 bits [H][n_keep][16]; flags_*: [H][n_keep][16].
 * ---------------------------------------------------------------------------------------- */
static void encode_tensor(const uint16_t *X, int is_key, int32_t H, int32_t T,
                          const int32_t *pos, int32_t n_keep, const float *C, const float *S,
                          int32_t bits, int8_t *codes, uint16_t *scales, uint8_t *flags)
{
    float k[HD], x[HD];
    for (int32_t h = 0; h < H; h++) {
        for (int32_t j = 0; j < n_keep; j++) {
            int32_t p = pos[j];
            const uint16_t *row = X + ((size_t)h * T + p) * HD;
            for (int i = 0; i < HD; i++) k[i] = nqo_h2f(row[i]);
            if (is_key)
                nqo_rope_undo(k, C + (size_t)p * 64, S + (size_t)p * 64, x);
            else
                memcpy(x, k, sizeof(x));
            nqo_fwht_f32(x);
            size_t o = (size_t)h * n_keep + j;
            nqo_quantize_row(x, bits, scales + o * NG, codes + o * HD, flags ? flags + o * NG : 0);
        }
        /* delta along the kept tokens, last to first so each step reads the absolute code */
        for (int32_t j = n_keep - 1; j >= 1; j--) {
            int8_t *cur = codes + ((size_t)h * n_keep + j) * HD;
            const int8_t *prev = cur - HD;
            for (int i = 0; i < HD; i++)
                cur[i] = (int8_t)(uint8_t)(((int)cur[i] - (int)prev[i]) & 0xff);
        }
    }
}

void nqo_encode_layer(const uint16_t *K, const uint16_t *V, int32_t H, int32_t T,
                      const int32_t *positions, int32_t n_keep, const float *C, const float *S,
                      int32_t bits_k, int32_t bits_v, int8_t *codes_k, int8_t *codes_v,
                      uint16_t *scales_k, uint16_t *scales_v, uint8_t *flags_k, uint8_t *flags_v)
{
    encode_tensor(K, 1, H, T, positions, n_keep, C, S, bits_k, codes_k, scales_k, flags_k);
    encode_tensor(V, 0, H, T, positions, n_keep, C, S, bits_v, codes_v, scales_v, flags_v);
}

/* ------------------------------------------------------------------------------------------
 * Decode one compressed layer (the inverse chain; [NQ-zh "技术实现细节": RoPE is restored after
 * quantization]). Per (head, dim) a running sum mod 256 of the deltas gives c; y = c/2;
 * x = s*y; inverse normalised Hadamard; keys get RoPE re-applied at their stored position:
 * k_i = x_i*C - x_{i+64}*S, k_{i+64} = x_{i+64}*C + x_i*S. All in fp64, cos/sin being the
 * fp32 table values. Outputs fp64 [H][n_keep][128].
 * ---------------------------------------------------------------------------------------- */
static void decode_tensor(const int8_t *d, const uint16_t *scales, int is_key, int32_t H,
                          const int32_t *pos, int32_t n_keep, const float *C, const float *S,
                          double *out)
{
    int c[HD];
    double x[HD];
    for (int32_t h = 0; h < H; h++) {
        for (int i = 0; i < HD; i++) c[i] = 0;
        for (int32_t j = 0; j < n_keep; j++) {
            size_t o = (size_t)h * n_keep + j;
            for (int i = 0; i < HD; i++) {
                c[i] = (int)(int8_t)(uint8_t)((c[i] + d[o * HD + i]) & 0xff);
                double s = (double)nqo_h2f(scales[o * NG + i / 8]);
                x[i] = s * (0.5 * (double)c[i]);
            }
            nqo_fwht_f64(x);
            double *dst = out + o * HD;
            if (is_key) {
                const float *Cp = C + (size_t)pos[j] * 64, *Sp = S + (size_t)pos[j] * 64;
                for (int i = 0; i < 64; i++) {
                    double cc = (double)Cp[i], ss = (double)Sp[i];
                    dst[i] = x[i] * cc - x[i + 64] * ss;
                    dst[i + 64] = x[i + 64] * cc + x[i] * ss;
                }
            } else {
                memcpy(dst, x, sizeof(x));
            }
        }
    }
}

void nqo_decode_layer(const int8_t *codes_k, const int8_t *codes_v, const uint16_t *scales_k,
                      const uint16_t *scales_v, const int32_t *positions, int32_t n_keep,
                      int32_t H, const float *C, const float *S, double *K_out, double *V_out)
{
    decode_tensor(codes_k, scales_k, 1, H, positions, n_keep, C, S, K_out);
    decode_tensor(codes_v, scales_v, 0, H, positions, n_keep, C, S, V_out);
}

/* ------------------------------------------------------------------------------------------
 * One-token grouped-query attention over the reconstructed cache of one layer (a consumer
 * check; the pages describe attention over reconstructed KV on the VQKV page, "推理流程集成").
 * Query head j reads kv head j / (Hq/H); z_t = <q_j, k_t> / sqrt(128); softmax over the kept
 * tokens with the maximum subtracted; o_j = sum_t p_t v_t. The query is used as given. fp64.
 * q: fp16 bits [Hq][128]; K, V: fp64 [H][n][128]; out: fp64 [Hq][128].
 * ---------------------------------------------------------------------------------------- */
void nqo_attend_layer(const uint16_t *q, int32_t Hq, const double *K, const double *V,
                      int32_t H, int32_t n, double *out)
{
    int32_t grp = Hq / H;
    double *z = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
    double scale = 1.0 / sqrt(128.0);
    for (int32_t j = 0; j < Hq; j++) {
        int32_t h = j / grp;
        double qv[HD];
        for (int i = 0; i < HD; i++) qv[i] = (double)nqo_h2f(q[(size_t)j * HD + i]);
        double mx = -INFINITY;
        for (int32_t t = 0; t < n; t++) {
            const double *k = K + ((size_t)h * n + t) * HD;
            double acc = 0.0;
            for (int i = 0; i < HD; i++) acc += qv[i] * k[i];
            z[t] = acc * scale;
            if (z[t] > mx) mx = z[t];
        }
        double den = 0.0;
        for (int32_t t = 0; t < n; t++) { z[t] = exp(z[t] - mx); den += z[t]; }
        for (int i = 0; i < HD; i++) {
            double acc = 0.0;
            for (int32_t t = 0; t < n; t++) acc += z[t] * V[((size_t)h * n + t) * HD + i];
            out[(size_t)j * HD + i] = n > 0 ? acc / den : 0.0;
        }
    }
    free(z);
}

/* ------------------------------------------------------------------------------------------
 * Nominal compressed size [NQ-pt "Os números": ratios include the overhead of scales, indices
 * and metadata]. Bits per kept token per compressed layer: per kv head 128*(b_K + b_V) lattice
 * bits plus two fp16 scales for each of the 16 groups, plus a 32-bit position. The ratio
 * compares with 2 * H * 128 * 16 bits per token of the fp16 cache.
 * ---------------------------------------------------------------------------------------- */
double nqo_nominal_ratio(int32_t H, int32_t T, int32_t n_keep, int32_t bits_k, int32_t bits_v)
{
    double per_tok = (double)H * (128.0 * (bits_k + bits_v) + 2.0 * 16.0 * 16.0) + 32.0;
    return (4096.0 * H * (double)T) / ((double)n_keep * per_tok);
}
