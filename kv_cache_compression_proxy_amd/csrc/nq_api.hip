// libnq host side: the C ABI declared in include/nq.h -- argument validation, workspace
// layout and kernel launches on the caller's stream. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nq.h"
#include "nq_attend.hpp"
#include "nq_attn_score.hpp"
#include "nq_codec.hpp"
#include "nq_fused.hpp"
#include "nq_scalar.hpp"
#include "nq_score.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int32_t compressed_layers(const nq_params *p) { return p->layer_end - p->layer_begin; }

nq_status check(const nq_params *p)
{
    if (!p) return NQ_ERR_INVALID_ARG;
    if (p->layers < 1 || p->kv_heads < 1 || p->tokens < 0 || p->head_dim < 1)
        return NQ_ERR_INVALID_ARG;
    if (p->layer_begin < 0 || p->layer_end < p->layer_begin || p->layer_end > p->layers)
        return NQ_ERR_INVALID_ARG;
    if (p->window < 0 || p->evict_permille < 0 || p->evict_permille > 1000)
        return NQ_ERR_INVALID_ARG;
    if (p->bits_k < 2 || p->bits_v < 2 || !(p->rope_base > 1.0) || !isfinite(p->rope_base))
        return NQ_ERR_INVALID_ARG;
    if (p->head_dim != 128) return NQ_ERR_UNSUPPORTED;
    if (p->bits_k > 4 || p->bits_v > 4) return NQ_ERR_UNSUPPORTED;
    // 32-bit token and tile indices inside the kernels, and 32-bit byte offsets of a token's
    // row within one head of one layer (256 bytes per fp16 row or fp32 rotary row)
    if ((int64_t)p->tokens * 256 > INT32_MAX) return NQ_ERR_UNSUPPORTED;
    if ((int64_t)p->kv_heads * 2 * compressed_layers(p) * ((int64_t)p->tokens / nq::kDecTile + 1) >
        INT32_MAX)
        return NQ_ERR_UNSUPPORTED;
    return NQ_OK;
}

int32_t keep_count(const nq_params *p)
{
    const int64_t T = p->tokens;
    if (T <= 0) return 0;
    const int64_t n_evict = (int64_t)p->evict_permille * T / 1000;
    const int64_t prot = (int64_t)p->window + 1 < T ? (int64_t)p->window + 1 : T;
    const int64_t keep = T - n_evict;
    return (int32_t)(keep > prot ? keep : prot);
}

float rho_of(int bits) { return (float)((1 << (bits - 1)) - 1); }

// An error left by an earlier, unrelated runtime call must not be reported as ours: entry
// points clear the thread's last error before they launch, then read it after.
void clear_error() { (void)hipGetLastError(); }

nq_status launched(const char *fn)
{
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return NQ_OK;
    if (getenv("NQ_VERBOSE")) fprintf(stderr, "libnq %s: %s\n", fn, hipGetErrorString(e));
    return NQ_ERR_HIP;
}

// Clears n words (16-byte aligned) and, when ticket is not null, the ticket words, with a
// kernel (no memset node in a captured graph).
void launch_reset(uint32_t *words, int64_t n, uint32_t *ticket, hipStream_t s)
{
    hipLaunchKernelGGL(nq::k_decode_reset, dim3((uint32_t)((nq::reset_threads(n) + 255) / 256)),
                       dim3(256), 0, s, words, n, ticket);
}

struct ScoreWs {
    double *qbar, *scores;
    size_t bytes;
};

ScoreWs score_ws(const nq_params *p, void *base)
{
    const size_t Lc = (size_t)compressed_layers(p);
    const size_t qb = align_up(Lc * p->kv_heads * 128 * sizeof(double));
    const size_t sc = align_up(Lc * (size_t)p->tokens * sizeof(double));
    ScoreWs w;
    w.qbar = (double *)base;
    w.scores = (double *)((char *)base + qb);
    w.bytes = qb + sc;
    return w;
}

int32_t codec_tiles(const nq_params *p) { return (keep_count(p) + nq::kCodecTile - 1) / nq::kCodecTile; }
int32_t decode_tiles(const nq_params *p) { return (keep_count(p) + nq::kDecTile - 1) / nq::kDecTile; }

// Per-layer selection: the register-resident kernel when a layer's candidates fit it (up to
// 32 keys per thread), the one with per-chunk flags in LDS up to 64 or 128 chunks per thread,
// else the one that re-reads the scores on every pass and for the emission.
constexpr int kSelRegKeys = 32;
constexpr int kSelMemChunks = 128;
void launch_select(const double *scores, int32_t T, int32_t W, int32_t n_keep, int32_t Lc,
                   int32_t *positions, hipStream_t s)
{
    const int32_t n_cand = T - W > 1 ? T - W - 1 : 0;
    if (n_cand <= kSelRegKeys * nq::kSelThreads)
        hipLaunchKernelGGL(nq::k_select_reg<kSelRegKeys>, dim3(Lc), dim3(nq::kSelThreads), 0, s,
                           scores, T, W, n_keep, positions);
    else if (n_cand <= kSelMemChunks / 2 * nq::kSelThreads)
        hipLaunchKernelGGL(nq::k_select_mem<kSelMemChunks / 2>, dim3(Lc), dim3(nq::kSelThreads),
                           0, s, scores, T, W, n_keep, positions);
    else if (n_cand <= kSelMemChunks * nq::kSelThreads)
        hipLaunchKernelGGL(nq::k_select_mem<kSelMemChunks>, dim3(Lc), dim3(nq::kSelThreads), 0,
                           s, scores, T, W, n_keep, positions);
    else
        hipLaunchKernelGGL(nq::k_select, dim3(Lc), dim3(nq::kSelThreads), 0, s, scores, T, W,
                           n_keep, positions);
}

struct DecodeWs {
    uint32_t *ticket, *agg, *incl;
    size_t bytes;
    int32_t tiles;
};

DecodeWs decode_ws(const nq_params *p, void *base)
{
    DecodeWs w;
    w.tiles = compressed_layers(p) * 2 * p->kv_heads * decode_tiles(p);
    const size_t words = (size_t)w.tiles * 16 * 4;
    const size_t t = align_up(nq::kTicketWords * sizeof(uint32_t));
    const size_t v = align_up(words * sizeof(uint32_t));
    char *b = (char *)base;
    w.ticket = (uint32_t *)b;
    w.agg = (uint32_t *)(b + t);
    w.incl = (uint32_t *)(b + t + v);   // directly follows agg: one reset covers both
    w.bytes = t + 2 * v;
    return w;
}

int attend_nsplit(const nq_params *p, int32_t n_tok)
{
    // aim for >= ~2048 blocks in total, chunks of >= 256 tokens
    const int64_t lh = (int64_t)compressed_layers(p) * p->kv_heads;
    int64_t ns = (2048 + lh - 1) / (lh > 0 ? lh : 1);
    const int64_t max_by_len = (n_tok + 255) / 256;
    if (ns > max_by_len) ns = max_by_len;
    if (ns < 1) ns = 1;
    return (int)ns;
}

struct AttWs {
    float *m, *l, *acc;
    size_t bytes;
    int nsplit;
};

AttWs attend_ws(const nq_params *p, int32_t q_heads, int32_t n_tok, void *base)
{
    AttWs w;
    w.nsplit = attend_nsplit(p, n_tok);
    const size_t G = (size_t)(q_heads / p->kv_heads);
    const size_t blocks = (size_t)compressed_layers(p) * p->kv_heads * w.nsplit;
    const size_t a = align_up(blocks * G * sizeof(float));
    const size_t c = align_up(blocks * G * 128 * sizeof(float));
    w.m = (float *)base;
    w.l = (float *)((char *)base + a);
    w.acc = (float *)((char *)base + 2 * a);
    w.bytes = 2 * a + c;
    return w;
}

struct FusedWs {
    uint32_t *ticket, *agg, *incl;
    float *part;
    size_t bytes;
    int32_t pairs, tiles;
};

FusedWs fused_ws(const nq_params *p, int32_t q_heads, void *base)
{
    FusedWs w;
    w.pairs = compressed_layers(p) * p->kv_heads;
    w.tiles = (keep_count(p) + nq::kFusedTile - 1) / nq::kFusedTile;
    const size_t G = (size_t)(q_heads / p->kv_heads);
    const size_t words = (size_t)w.pairs * w.tiles * 2 * 16 * 4;
    const size_t t = align_up(nq::kTicketWords * sizeof(uint32_t));
    const size_t v = align_up(words * sizeof(uint32_t));
    const size_t pb = align_up((size_t)w.pairs * w.tiles * G * nq::kPartStride * sizeof(float));
    char *b = (char *)base;
    w.ticket = (uint32_t *)b;
    w.agg = (uint32_t *)(b + t);
    w.incl = (uint32_t *)(b + t + v);   // directly follows agg: one reset covers both
    w.part = (float *)(b + t + 2 * v);
    w.bytes = t + 2 * v + pb;
    return w;
}

struct AttnScoreWs {
    float *bias, *colsum;
    double *scores;
    size_t bytes;
};

AttnScoreWs attn_score_ws(const nq_params *p, int32_t q_heads, void *base)
{
    const size_t pairs = (size_t)compressed_layers(p) * p->kv_heads;
    const size_t R = (size_t)(q_heads / p->kv_heads) * p->window;
    const size_t b = align_up(pairs * R * sizeof(float));
    const size_t c = align_up(pairs * (size_t)p->tokens * sizeof(float));
    const size_t d = align_up((size_t)compressed_layers(p) * p->tokens * sizeof(double));
    AttnScoreWs w;
    w.bias = (float *)base;
    w.colsum = (float *)((char *)base + b);
    w.scores = (double *)((char *)base + b + c);
    w.bytes = b + c + d;
    return w;
}

// Lloyd-Max quantizer of N(0, 1) with 2^bits levels: from levels evenly spaced on [-2, 2],
// alternate thresholds = midpoints of neighbouring levels and levels = the mean of N(0, 1) over
// each cell, until no level moves by 1e-15; then make the table exactly antisymmetric (N(0, 1)
// is symmetric; the middle threshold becomes exactly 0).
double gauss_pdf(double x) { return isfinite(x) ? exp(-0.5 * x * x) / sqrt(2.0 * M_PI) : 0.0; }
double gauss_cdf(double x)
{
    if (x == INFINITY) return 1.0;
    if (x == -INFINITY) return 0.0;
    return 0.5 * erfc(-x / sqrt(2.0));
}

void lloyd_max(int bits, double *y, double *t)
{
    const int n = 1 << bits;
    for (int i = 0; i < n; i++) y[i] = n > 1 ? i * (4.0 / (n - 1)) + -2.0 : 0.0;
    if (n > 1) y[n - 1] = 2.0;
    double e[17], yn[16];
    for (int it = 0; it < 200000; it++) {
        e[0] = -INFINITY;
        e[n] = INFINITY;
        for (int i = 0; i + 1 < n; i++) e[i + 1] = 0.5 * (y[i] + y[i + 1]);
        double d = 0.0;
        for (int i = 0; i < n; i++) {
            yn[i] = (gauss_pdf(e[i]) - gauss_pdf(e[i + 1])) / (gauss_cdf(e[i + 1]) - gauss_cdf(e[i]));
            d = fmax(d, fabs(yn[i] - y[i]));
        }
        for (int i = 0; i < n; i++) y[i] = yn[i];
        if (d < 1e-15) break;
    }
    double ys[16];
    for (int i = 0; i < n; i++) ys[i] = 0.5 * (y[i] - y[n - 1 - i]);
    for (int i = 0; i < n; i++) y[i] = ys[i];
    for (int i = 0; i + 1 < n; i++) t[i] = 0.5 * (y[i] + y[i + 1]);
}

struct LloydTables {
    double y[5][16], t[5][15];
    std::once_flag once;
};
LloydTables &lloyd_tables()
{
    static LloydTables tb;
    std::call_once(tb.once, [] {
        for (int b = 1; b <= 4; b++) lloyd_max(b, tb.y[b], tb.t[b]);
    });
    return tb;
}

nq::ScalarArgs scalar_args(const nq_params *p, const int32_t *positions, const float *rope_cos,
                           const float *rope_sin)
{
    nq::ScalarArgs a;
    memset(&a, 0, sizeof(a));
    a.positions = positions;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.H = p->kv_heads;
    a.T = p->tokens;
    a.layer_begin = p->layer_begin;
    a.n_keep = keep_count(p);
    a.tiles = (a.n_keep + nq::kScalarTile - 1) / nq::kScalarTile;
    LloydTables &tb = lloyd_tables();
    const int bits[2] = {p->bits_k, p->bits_v};
    for (int tn = 0; tn < 2; tn++) {
        const int b = bits[tn], n = 1 << b;
        a.bits[tn] = b;
        for (int i = 0; i < 15; i++) a.thr[tn][i] = i + 1 < n ? (float)tb.t[b][i] : INFINITY;
        for (int i = 0; i < 16; i++) a.lev[tn][i] = i < n ? (float)tb.y[b][i] : 0.0f;
    }
    return a;
}

}  // namespace

// Scratch of nq_decode_static, for callers that cannot allocate (code under HIP graph capture,
// serving loops, harnesses that forbid allocation): the decode's tile tickets and look-back
// words live in this file-scope device array instead of a caller workspace. The module holds
// it on every GPU it is loaded on until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies only ever get the address that
// hipGetSymbolAddress returns for the current device.
namespace {
constexpr size_t kScratchBytes = NQ_DECODE_STATIC_MAX_BYTES;
constexpr int kMaxDevices = 64;
}
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
nq_status scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return NQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return NQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            if (getenv("NQ_VERBOSE"))
                fprintf(stderr, "libnq: hipGetSymbolAddress(scratch) on device %d: %s\n", dev,
                        hipGetErrorString(e));
            return NQ_ERR_HIP;
        }
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return NQ_OK;
}
}  // namespace

extern "C" {

int32_t nq_keep_count(const nq_params *p)
{
    if (check(p) != NQ_OK) return -1;
    return keep_count(p);
}

nq_status nq_check_params(const nq_params *p) { return check(p); }

size_t nq_score_evict_workspace_bytes(const nq_params *p)
{
    if (check(p) != NQ_OK) return 0;
    return score_ws(p, nullptr).bytes;
}

size_t nq_decode_workspace_bytes(const nq_params *p)
{
    if (check(p) != NQ_OK) return 0;
    return decode_ws(p, nullptr).bytes;
}

size_t nq_attend_workspace_bytes(const nq_params *p, int32_t q_heads, int32_t n_tok)
{
    if (check(p) != NQ_OK || q_heads < 1 || n_tok < 0 || q_heads % p->kv_heads) return 0;
    return attend_ws(p, q_heads, n_tok, nullptr).bytes;
}

const char *nq_status_string(nq_status s)
{
    switch (s) {
    case NQ_OK: return "ok";
    case NQ_ERR_INVALID_ARG: return "invalid argument";
    case NQ_ERR_UNSUPPORTED: return "unsupported parameters";
    case NQ_ERR_WORKSPACE: return "workspace missing or too small";
    case NQ_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

nq_status nq_rope_table(const nq_params *p, float *cos_dev, float *sin_dev, void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    if (p->tokens == 0) return NQ_OK;
    if (!cos_dev || !sin_dev || !aligned(cos_dev, 16) || !aligned(sin_dev, 16))
        return NQ_ERR_INVALID_ARG;
    nq::RopeTheta th;
    for (int i = 0; i < 64; i++) th.v[i] = pow(p->rope_base, -(double)i / 64.0);
    const int64_t n = (int64_t)p->tokens * 64;
    clear_error();
    hipLaunchKernelGGL(nq::k_rope_table, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0,
                       as_stream(stream), th, p->tokens, cos_dev, sin_dev);
    return launched("nq_rope_table");
}

nq_status nq_score_evict(const nq_params *p, const void *K, int32_t *positions,
                         double *scores_opt, void *workspace, size_t ws_bytes, void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    const int32_t Lc = compressed_layers(p), T = p->tokens, H = p->kv_heads;
    const int32_t n_keep = keep_count(p);
    if (Lc == 0 || T == 0) return NQ_OK;
    if (!K || !positions || !aligned(K, 16) || !aligned(positions, 4)) return NQ_ERR_INVALID_ARG;
    if (scores_opt && !aligned(scores_opt, 8)) return NQ_ERR_INVALID_ARG;
    const size_t need = score_ws(p, nullptr).bytes;
    if (!workspace || ws_bytes < need || !aligned(workspace, kAlign)) return NQ_ERR_WORKSPACE;
    ScoreWs w = score_ws(p, workspace);
    double *scores = scores_opt ? scores_opt : w.scores;
    hipStream_t s = as_stream(stream);
    const uint16_t *K16 = (const uint16_t *)K;
    clear_error();
    hipLaunchKernelGGL(nq::k_window_sum, dim3(Lc * H), dim3(256), 0, s, K16, H, T, p->window,
                       p->layer_begin, w.qbar);
    const int tiles = (T + nq::kScoreTile - 1) / nq::kScoreTile;
    hipLaunchKernelGGL(nq::k_scores, dim3(Lc * tiles), dim3(256), 0, s, K16, w.qbar, H, T,
                       p->window, p->layer_begin, tiles, scores);
    launch_select(scores, T, p->window, n_keep, Lc, positions, s);
    return launched("nq_score_evict");
}

size_t nq_score_evict_attn_workspace_bytes(const nq_params *p, int32_t q_heads)
{
    if (check(p) != NQ_OK || q_heads < 1 || q_heads % p->kv_heads) return 0;
    return attn_score_ws(p, q_heads, nullptr).bytes;
}

nq_status nq_score_evict_attn(const nq_params *p, const void *K, const void *Q_obs,
                              int32_t q_heads, int32_t *positions, double *scores_opt,
                              void *workspace, size_t ws_bytes, void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    if (q_heads < 1 || q_heads % p->kv_heads) return NQ_ERR_INVALID_ARG;
    const int32_t Lc = compressed_layers(p), T = p->tokens, H = p->kv_heads, W = p->window;
    const int32_t G = q_heads / H, n_keep = keep_count(p);
    if ((int64_t)G * W > INT32_MAX / 2) return NQ_ERR_UNSUPPORTED;
    if (Lc == 0 || T == 0) return NQ_OK;
    if (!K || !positions || !aligned(K, 16) || !aligned(positions, 4)) return NQ_ERR_INVALID_ARG;
    if (W > 0 && (!Q_obs || !aligned(Q_obs, 16))) return NQ_ERR_INVALID_ARG;
    if (scores_opt && !aligned(scores_opt, 8)) return NQ_ERR_INVALID_ARG;
    const size_t need = attn_score_ws(p, q_heads, nullptr).bytes;
    if (!workspace || ws_bytes < need || !aligned(workspace, kAlign)) return NQ_ERR_WORKSPACE;
    AttnScoreWs w = attn_score_ws(p, q_heads, workspace);
    nq::AttnScoreArgs a;
    a.K = (const uint16_t *)K;
    a.Q = (const uint16_t *)Q_obs;
    a.bias = w.bias;
    a.colsum = w.colsum;
    a.scores = scores_opt ? scores_opt : w.scores;
    a.H = H;
    a.G = G;
    a.W = W;
    a.T = T;
    a.R = G * W;
    a.layer_begin = p->layer_begin;
    a.row_chunks = (a.R + nq::kAttnRows - 1) / nq::kAttnRows;
    const int c_end = T - W;
    a.key_chunks = c_end > 0 ? (c_end + nq::kAttnKeys - 1) / nq::kAttnKeys : 0;
    const int64_t pairs = (int64_t)Lc * H;
    hipStream_t s = as_stream(stream);
    clear_error();
    if (a.R > 0 && a.key_chunks > 0) {
        hipLaunchKernelGGL(nq::k_attn_rowbias, dim3((uint32_t)(pairs * a.row_chunks)),
                           dim3(nq::kAttnThreads), 0, s, a);
        hipLaunchKernelGGL(nq::k_attn_colsum, dim3((uint32_t)(pairs * a.key_chunks)),
                           dim3(nq::kAttnThreads), 0, s, a);
    }
    if (c_end > 0) {
        const int64_t n = (int64_t)Lc * c_end;
        hipLaunchKernelGGL(nq::k_attn_finish, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s,
                           a, Lc);
    }
    launch_select(a.scores, T, W, n_keep, Lc, positions, s);
    return launched("nq_score_evict_attn");
}

static nq::CodecArgs codec_args(const nq_params *p, const int32_t *positions,
                                const float *rope_cos, const float *rope_sin)
{
    nq::CodecArgs a;
    memset(&a, 0, sizeof(a));
    a.positions = positions;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.H = p->kv_heads;
    a.T = p->tokens;
    a.layer_begin = p->layer_begin;
    a.n_keep = keep_count(p);
    a.tiles_per_chain = codec_tiles(p);
    a.dec_tiles_per_chain = decode_tiles(p);
    a.rho_k = rho_of(p->bits_k);
    a.rho_v = rho_of(p->bits_v);
    a.rho_inv_k = 1.0f / a.rho_k;   // IEEE division on the host: the nearest fp32
    a.rho_inv_v = 1.0f / a.rho_v;
    // the rest of 1/rho, rounded to fp32 (rho_inv + rho_inv_lo is 1/rho to ~2^-49 relative)
    a.rho_inv_lo_k = (float)(1.0 / (double)a.rho_k - (double)a.rho_inv_k);
    a.rho_inv_lo_v = (float)(1.0 / (double)a.rho_v - (double)a.rho_inv_v);
    return a;
}

nq_status nq_encode(const nq_params *p, const void *K, const void *V, const int32_t *positions,
                    const float *rope_cos, const float *rope_sin, int8_t *codes_k,
                    int8_t *codes_v, void *scales_k, void *scales_v, void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    const int32_t Lc = compressed_layers(p);
    if (Lc == 0 || p->tokens == 0) return NQ_OK;
    const void *ptrs16[] = {K, V, rope_cos, rope_sin, codes_k, codes_v};
    for (const void *q : ptrs16)
        if (!q || !aligned(q, 16)) return NQ_ERR_INVALID_ARG;
    if (!positions || !aligned(positions, 4) || !scales_k || !scales_v || !aligned(scales_k, 4) ||
        !aligned(scales_v, 4))
        return NQ_ERR_INVALID_ARG;
    nq::CodecArgs a = codec_args(p, positions, rope_cos, rope_sin);
    a.K = (const uint16_t *)K;
    a.V = (const uint16_t *)V;
    a.codes_k = codes_k;
    a.codes_v = codes_v;
    a.scales_k = (uint16_t *)scales_k;
    a.scales_v = (uint16_t *)scales_v;
    const int64_t blocks = (int64_t)Lc * 2 * p->kv_heads * a.tiles_per_chain;
    clear_error();
    hipLaunchKernelGGL(nq::k_encode, dim3((uint32_t)blocks), dim3(nq::kCodecThreads), 0,
                       as_stream(stream), a);
    return launched("nq_encode");
}

// Argument checks of nq_decode and nq_decode_static (everything but the workspace). *skip is
// set when there is nothing to decode.
static nq_status decode_args_ok(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                                const void *scales_k, const void *scales_v,
                                const int32_t *positions, const float *rope_cos,
                                const float *rope_sin, void *K_out, void *V_out,
                                nq_out_dtype out_dtype, bool *skip)
{
    *skip = false;
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    if (out_dtype != NQ_OUT_F16 && out_dtype != NQ_OUT_F32) return NQ_ERR_INVALID_ARG;
    if (compressed_layers(p) == 0 || p->tokens == 0) {
        *skip = true;
        return NQ_OK;
    }
    const void *ptrs16[] = {codes_k, codes_v, rope_cos, rope_sin, K_out, V_out};
    for (const void *q : ptrs16)
        if (!q || !aligned(q, 16)) return NQ_ERR_INVALID_ARG;
    if (!positions || !aligned(positions, 4) || !scales_k || !scales_v || !aligned(scales_k, 4) ||
        !aligned(scales_v, 4))
        return NQ_ERR_INVALID_ARG;
    return NQ_OK;
}

// The decode launches (look-back word reset, then the tiles) with the workspace at `workspace`
// (validated by the caller).
static nq_status decode_launch(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                               const void *scales_k, const void *scales_v,
                               const int32_t *positions, const float *rope_cos,
                               const float *rope_sin, void *K_out, void *V_out,
                               nq_out_dtype out_dtype, void *workspace, void *stream,
                               const char *fn)
{
    DecodeWs w = decode_ws(p, workspace);
    nq::CodecArgs a = codec_args(p, positions, rope_cos, rope_sin);
    a.codes_k = (int8_t *)codes_k;
    a.codes_v = (int8_t *)codes_v;
    a.scales_k = (uint16_t *)scales_k;
    a.scales_v = (uint16_t *)scales_v;
    a.out_k = K_out;
    a.out_v = V_out;
    a.out_f32 = out_dtype == NQ_OUT_F32;
    a.lb_ticket = w.ticket;
    a.lb_agg = w.agg;
    a.lb_incl = w.incl;
    hipStream_t s = as_stream(stream);
    clear_error();
    const int64_t words = (int64_t)(w.incl - w.agg) + (int64_t)w.tiles * 64;
    launch_reset(w.agg, words, w.ticket, s);
    hipLaunchKernelGGL(nq::k_decode, dim3((uint32_t)w.tiles), dim3(nq::kCodecThreads), 0, s, a);
    return launched(fn);
}

nq_status nq_decode(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                    const void *scales_k, const void *scales_v, const int32_t *positions,
                    const float *rope_cos, const float *rope_sin, void *K_out, void *V_out,
                    nq_out_dtype out_dtype, void *workspace, size_t ws_bytes, void *stream)
{
    bool skip;
    nq_status st = decode_args_ok(p, codes_k, codes_v, scales_k, scales_v, positions, rope_cos,
                                  rope_sin, K_out, V_out, out_dtype, &skip);
    if (st != NQ_OK || skip) return st;
    const size_t need = decode_ws(p, nullptr).bytes;
    if (!workspace || ws_bytes < need || !aligned(workspace, kAlign)) return NQ_ERR_WORKSPACE;
    return decode_launch(p, codes_k, codes_v, scales_k, scales_v, positions, rope_cos, rope_sin,
                         K_out, V_out, out_dtype, workspace, stream, "nq_decode");
}

nq_status nq_decode_static(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                           const void *scales_k, const void *scales_v, const int32_t *positions,
                           const float *rope_cos, const float *rope_sin, void *K_out,
                           void *V_out, nq_out_dtype out_dtype, void *stream)
{
    bool skip;
    nq_status st = decode_args_ok(p, codes_k, codes_v, scales_k, scales_v, positions, rope_cos,
                                  rope_sin, K_out, V_out, out_dtype, &skip);
    if (st != NQ_OK || skip) return st;
    if (decode_ws(p, nullptr).bytes > kScratchBytes) {
        if (getenv("NQ_VERBOSE"))
            fprintf(stderr, "libnq nq_decode_static: needs %zu bytes of scratch, the static "
                    "array holds %zu\n", decode_ws(p, nullptr).bytes, kScratchBytes);
        return NQ_ERR_WORKSPACE;
    }
    void *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != NQ_OK) return st;
    return decode_launch(p, codes_k, codes_v, scales_k, scales_v, positions, rope_cos, rope_sin,
                         K_out, V_out, out_dtype, ws, stream, "nq_decode_static");
}

size_t nq_decode_attend_workspace_bytes(const nq_params *p, int32_t q_heads)
{
    if (check(p) != NQ_OK || q_heads < 1 || q_heads % p->kv_heads) return 0;
    return fused_ws(p, q_heads, nullptr).bytes;
}

nq_status nq_decode_attend(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                           const void *scales_k, const void *scales_v, const int32_t *positions,
                           const float *rope_cos, const float *rope_sin, const void *Q,
                           int32_t q_heads, float *out, void *workspace, size_t ws_bytes,
                           void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    if (q_heads < 1 || q_heads % p->kv_heads) return NQ_ERR_INVALID_ARG;
    const int G = q_heads / p->kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return NQ_ERR_UNSUPPORTED;
    const int32_t Lc = compressed_layers(p);
    if (Lc == 0) return NQ_OK;
    if (!Q || !out || !aligned(Q, 16) || !aligned(out, 16)) return NQ_ERR_INVALID_ARG;
    const int32_t n = keep_count(p);
    hipStream_t s = as_stream(stream);
    if (n == 0) {   // nothing to attend to: zeros, written by a kernel (no memset node)
        const int64_t words = (int64_t)Lc * q_heads * 128;
        clear_error();
        launch_reset((uint32_t *)out, words, nullptr, s);
        return launched("nq_decode_attend");
    }
    const void *ptrs16[] = {codes_k, codes_v, rope_cos, rope_sin};
    for (const void *q : ptrs16)
        if (!q || !aligned(q, 16)) return NQ_ERR_INVALID_ARG;
    if (!positions || !aligned(positions, 4) || !scales_k || !scales_v || !aligned(scales_k, 16) ||
        !aligned(scales_v, 16))
        return NQ_ERR_INVALID_ARG;
    const size_t need = fused_ws(p, q_heads, nullptr).bytes;
    if (!workspace || ws_bytes < need || !aligned(workspace, kAlign)) return NQ_ERR_WORKSPACE;
    FusedWs w = fused_ws(p, q_heads, workspace);
    nq::FusedArgs a;
    a.codes_k = codes_k;
    a.codes_v = codes_v;
    a.scales_k = (const uint16_t *)scales_k;
    a.scales_v = (const uint16_t *)scales_v;
    a.positions = positions;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.Q = (const uint16_t *)Q;
    a.out = out;
    a.part = w.part;
    a.lb_agg = w.agg;
    a.lb_incl = w.incl;
    a.lb_ticket = w.ticket;
    a.H = p->kv_heads;
    a.Hq = q_heads;
    a.T = p->tokens;
    a.n_keep = n;
    a.tiles = w.tiles;
    clear_error();
    const int64_t words = (int64_t)(w.incl - w.agg) + (int64_t)w.pairs * w.tiles * 2 * 64;
    launch_reset(w.agg, words, w.ticket, s);
    const dim3 grid((uint32_t)((int64_t)w.pairs * w.tiles)), blk(nq::kCodecThreads);
    const dim3 mgrid((uint32_t)(Lc * q_heads));
    switch (G) {
    case 1:
        hipLaunchKernelGGL(nq::k_decode_attend<1>, grid, blk, 0, s, a);
        hipLaunchKernelGGL(nq::k_decode_attend_merge<1>, mgrid, blk, 0, s, a);
        break;
    case 2:
        hipLaunchKernelGGL(nq::k_decode_attend<2>, grid, blk, 0, s, a);
        hipLaunchKernelGGL(nq::k_decode_attend_merge<2>, mgrid, blk, 0, s, a);
        break;
    case 4:
        hipLaunchKernelGGL(nq::k_decode_attend<4>, grid, blk, 0, s, a);
        hipLaunchKernelGGL(nq::k_decode_attend_merge<4>, mgrid, blk, 0, s, a);
        break;
    default:
        hipLaunchKernelGGL(nq::k_decode_attend<8>, grid, blk, 0, s, a);
        hipLaunchKernelGGL(nq::k_decode_attend_merge<8>, mgrid, blk, 0, s, a);
        break;
    }
    return launched("nq_decode_attend");
}

nq_status nq_lloyd_max_table(int32_t bits, double *levels, double *thresholds)
{
    if (bits < 1 || bits > 4 || !levels || !thresholds) return NQ_ERR_INVALID_ARG;
    LloydTables &tb = lloyd_tables();
    for (int i = 0; i < (1 << bits); i++) levels[i] = tb.y[bits][i];
    for (int i = 0; i + 1 < (1 << bits); i++) thresholds[i] = tb.t[bits][i];
    return NQ_OK;
}

nq_status nq_encode_scalar(const nq_params *p, const void *K, const void *V,
                           const int32_t *positions, const float *rope_cos, const float *rope_sin,
                           uint8_t *idx_k, uint8_t *idx_v, void *scales_k, void *scales_v,
                           void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    const int32_t Lc = compressed_layers(p);
    if (Lc == 0 || p->tokens == 0) return NQ_OK;
    const void *ptrs16[] = {K, V, rope_cos, rope_sin};
    for (const void *q : ptrs16)
        if (!q || !aligned(q, 16)) return NQ_ERR_INVALID_ARG;
    if (!idx_k || !idx_v || !aligned(idx_k, 8) || !aligned(idx_v, 8) || !positions ||
        !aligned(positions, 4) || !scales_k || !scales_v || !aligned(scales_k, 2) ||
        !aligned(scales_v, 2))
        return NQ_ERR_INVALID_ARG;
    nq::ScalarArgs a = scalar_args(p, positions, rope_cos, rope_sin);
    a.K = (const uint16_t *)K;
    a.V = (const uint16_t *)V;
    a.idx_k = idx_k;
    a.idx_v = idx_v;
    a.scales_k = (uint16_t *)scales_k;
    a.scales_v = (uint16_t *)scales_v;
    const int64_t blocks = (int64_t)Lc * 2 * p->kv_heads * a.tiles;
    clear_error();
    hipLaunchKernelGGL(nq::k_encode_scalar, dim3((uint32_t)blocks), dim3(nq::kCodecThreads), 0,
                       as_stream(stream), a);
    return launched("nq_encode_scalar");
}

nq_status nq_decode_scalar(const nq_params *p, const uint8_t *idx_k, const uint8_t *idx_v,
                           const void *scales_k, const void *scales_v, const int32_t *positions,
                           const float *rope_cos, const float *rope_sin, void *K_out,
                           void *V_out, nq_out_dtype out_dtype, void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    if (out_dtype != NQ_OUT_F16 && out_dtype != NQ_OUT_F32) return NQ_ERR_INVALID_ARG;
    const int32_t Lc = compressed_layers(p);
    if (Lc == 0 || p->tokens == 0) return NQ_OK;
    const void *ptrs16[] = {rope_cos, rope_sin, K_out, V_out};
    for (const void *q : ptrs16)
        if (!q || !aligned(q, 16)) return NQ_ERR_INVALID_ARG;
    if (!idx_k || !idx_v || !aligned(idx_k, 8) || !aligned(idx_v, 8) || !positions ||
        !aligned(positions, 4) || !scales_k || !scales_v || !aligned(scales_k, 2) ||
        !aligned(scales_v, 2))
        return NQ_ERR_INVALID_ARG;
    nq::ScalarArgs a = scalar_args(p, positions, rope_cos, rope_sin);
    a.idx_k = (uint8_t *)idx_k;
    a.idx_v = (uint8_t *)idx_v;
    a.scales_k = (uint16_t *)scales_k;
    a.scales_v = (uint16_t *)scales_v;
    a.out_k = K_out;
    a.out_v = V_out;
    a.out_f32 = out_dtype == NQ_OUT_F32;
    const int64_t blocks = (int64_t)Lc * 2 * p->kv_heads * a.tiles;
    clear_error();
    hipLaunchKernelGGL(nq::k_decode_scalar, dim3((uint32_t)blocks), dim3(nq::kCodecThreads), 0,
                       as_stream(stream), a);
    return launched("nq_decode_scalar");
}

nq_status nq_attend_decode(const nq_params *p, const void *Q, int32_t q_heads, const void *K,
                           const void *V, int32_t n_tok, float *out, void *workspace,
                           size_t ws_bytes, void *stream)
{
    nq_status st = check(p);
    if (st != NQ_OK) return st;
    if (q_heads < 1 || n_tok < 0 || q_heads % p->kv_heads) return NQ_ERR_INVALID_ARG;
    const int G = q_heads / p->kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return NQ_ERR_UNSUPPORTED;
    const int32_t Lc = compressed_layers(p);
    if (Lc == 0) return NQ_OK;
    const void *ptrs16[] = {Q, K, V, out};
    for (const void *q : ptrs16)
        if (!q || !aligned(q, 16)) return NQ_ERR_INVALID_ARG;
    const size_t need = attend_ws(p, q_heads, n_tok, nullptr).bytes;
    if (!workspace || ws_bytes < need || !aligned(workspace, kAlign)) return NQ_ERR_WORKSPACE;
    AttWs w = attend_ws(p, q_heads, n_tok, workspace);
    nq::AttArgs a;
    a.Q = (const uint16_t *)Q;
    a.K = (const uint16_t *)K;
    a.V = (const uint16_t *)V;
    a.out = out;
    a.part_m = w.m;
    a.part_l = w.l;
    a.part_acc = w.acc;
    a.H = p->kv_heads;
    a.Hq = q_heads;
    a.n = n_tok;
    a.nsplit = w.nsplit;
    hipStream_t s = as_stream(stream);
    const dim3 grid((uint32_t)(Lc * p->kv_heads * w.nsplit));
    clear_error();
    switch (G) {
    case 1: hipLaunchKernelGGL(nq::k_attend<1>, grid, dim3(nq::kAttThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(nq::k_attend<2>, grid, dim3(nq::kAttThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(nq::k_attend<4>, grid, dim3(nq::kAttThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(nq::k_attend<8>, grid, dim3(nq::kAttThreads), 0, s, a); break;
    }
    hipLaunchKernelGGL(nq::k_attend_merge, dim3((uint32_t)(Lc * q_heads)), dim3(128), 0, s, a, G);
    return launched("nq_attend_decode");
}

}  // extern "C"
