/*
 * nq.h -- C ABI of libnq, the MI355X (gfx950) KV-cache compression hot path.
 *
 * The method (NexusQuant as described on the pages "NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的
 * 技术突破" and "Como comprimir o KV cache do seu LLM em 33x sem treino") compresses a prefill
 * KV cache in six steps: key-key proxy scoring, eviction that always keeps BOS and a recent
 * window, RoPE removal on the kept keys, a normalised Hadamard rotation, E8 lattice
 * quantization of 8-float groups (keys 3-bit, values 2-bit), and delta coding of the lattice
 * codes along the token axis. Decoding inverts the codec steps. This header exposes those steps
 * as device-side operations over caller-owned GPU buffers.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, and live in device memory allocated by the caller (e.g.
 *    torch tensors). The library allocates no device memory and keeps no state between calls;
 *    calls on different streams with disjoint buffers may run concurrently. The one exception
 *    is nq_decode_static, whose scratch is a fixed device array of the library (see there).
 *  - K and V are fp16 [layers][kv_heads][tokens][128] (the full cache, batch 1). Outputs are
 *    indexed by compressed layer lc = l - layer_begin, 0 <= lc < layer_end - layer_begin.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call is
 *    asynchronous on that stream and never synchronises the host.
 *  - Arguments are validated on the host before anything is launched. On any error nothing is
 *    launched and output buffers are left untouched. A failed launch returns NQ_ERR_HIP.
 *  - Device pointers to fp16/fp32/fp64 data must be 16-byte aligned; int32 position arrays
 *    4-byte aligned. Inputs must be finite.
 *  - Layers outside [layer_begin, layer_end) are never read or written (the pages'
 *    protect_boundary option keeps the first/last layers in fp16: section "技术实现细节").
 */
#ifndef NQ_H
#define NQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nq_status {
    NQ_OK = 0,
    NQ_ERR_INVALID_ARG = -1,  /* a size, range, pointer or alignment is invalid */
    NQ_ERR_UNSUPPORTED = -2,  /* valid but not implemented (head_dim != 128, bits > 4, ...) */
    NQ_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the *_workspace_bytes size */
    NQ_ERR_HIP = -4           /* the HIP runtime rejected a launch */
} nq_status;

typedef enum nq_out_dtype {
    NQ_OUT_F16 = 0,           /* fp16, round to nearest even (the normal output) */
    NQ_OUT_F32 = 1            /* fp32 (for tolerance checks) */
} nq_out_dtype;

/* Shape and method parameters. Defaults of the pages' presets are set by the caller. */
typedef struct nq_params {
    int32_t layers;           /* L >= 1 */
    int32_t kv_heads;         /* H >= 1 */
    int32_t tokens;           /* T >= 0 (prefill length); above 8388607 unsupported (a layer's
                                 rows of one head are addressed with 32-bit byte offsets) */
    int32_t head_dim;         /* must be 128 */
    int32_t layer_begin;      /* compressed layer range [layer_begin, layer_end) */
    int32_t layer_end;
    int32_t window;           /* W >= 0: recent window, both protected and used as the
                                 proxy queries of the scorer */
    int32_t evict_permille;   /* eviction fraction in 1/1000 (600 = 60%), 0..1000 */
    int32_t bits_k;           /* key bit budget, 2..4 (E8 radius rho = 2^(b-1) - 1); below 2
                                 is invalid (rho = 0), above 4 unsupported */
    int32_t bits_v;           /* value bit budget, 2..4 */
    double rope_base;         /* split-half RoPE base (1e4 Llama/Mistral, 1e6 Qwen2.5), > 1 */
} nq_params;

/* Number of tokens kept per compressed layer ("Token淘汰机制": BOS and the recent window are
 * always kept; 60% eviction keeps 2.5x fewer tokens):
 *   n_evict = floor(evict_permille * T / 1000), n_keep = max(T - n_evict, min(T, 1 + W)).
 * Host-only closed form. Returns -1 if the parameters are invalid. */
int32_t nq_keep_count(const nq_params *p);

/* Returns NQ_OK if the parameters are valid and supported, else the error code. Host-only. */
nq_status nq_check_params(const nq_params *p);

/* Device workspace needed by nq_score_evict (bytes, 256-aligned). 0 if p is invalid. */
size_t nq_score_evict_workspace_bytes(const nq_params *p);

/* Device workspace needed by nq_decode (bytes). 0 if p is invalid. */
size_t nq_decode_workspace_bytes(const nq_params *p);

/* Device workspace needed by nq_attend_decode for q_heads query heads over n_tok tokens. */
size_t nq_attend_workspace_bytes(const nq_params *p, int32_t q_heads, int32_t n_tok);

/* Rotary table for split-half RoPE ("使用方法与兼容性": split-half RoPE only). Writes
 * cos_dev[p][i] = fp32(cos(p * theta_i)), sin_dev[p][i] = fp32(sin(p * theta_i)) for
 * 0 <= p < tokens, 0 <= i < 64, theta_i = rope_base^(-i/64) (fp64 angles). Both outputs are
 * fp32 [tokens][64] device buffers owned by the caller; they are inputs of nq_encode and
 * nq_decode. */
nq_status nq_rope_table(const nq_params *p, float *cos_dev, float *sin_dev, void *stream);

/* Steps 1-2: key-key proxy scoring and eviction ("技术实现细节": key-key proxy without extra
 * computation; "Como funciona" steps 1-2: cross-head inner product, evict the least important,
 * always keep BOS and a recent window). Per compressed layer, qbar_h = sum of the last W keys
 * of head h (fp64, exact), and candidate t in [1, T-W) scores s_t = sum_h <qbar_h, k_{h,t}>
 * (fp64) on the stored keys. The n_keep - |protected| best candidates by (score descending,
 * position ascending) are kept together with BOS and the window.
 *   K          fp16 [L][H][T][128]
 *   positions  int32 [layer_end-layer_begin][n_keep] out: kept positions, ascending
 *   scores_opt NULL, or fp64 [layer_end-layer_begin][T] out: s_t for candidates (other
 *              entries are not written)
 *   workspace  device scratch of nq_score_evict_workspace_bytes(p) bytes */
nq_status nq_score_evict(const nq_params *p, const void *K, int32_t *positions,
                         double *scores_opt, void *workspace, size_t ws_bytes, void *stream);

/* Device workspace needed by nq_score_evict_attn for q_heads query heads (bytes). 0 if p is
 * invalid. */
size_t nq_score_evict_attn_workspace_bytes(const nq_params *p, int32_t q_heads);

/* Steps 1-2 with the attention-weight scorer ("技术实现细节": the real attention scorer,
 * higher quality at the cost of an extra pass; "Token淘汰机制": tokens ranked by their attention
 * weights, BOS and the recent window always kept). Per compressed layer, an observation window
 * of W = window queries per query head (query w at position T - W + w; positions below 0 are
 * ignored) scores each candidate t in [1, T - W) by
 *   s_t = sum_j sum_w softmax_{t' <= T-W+w}(<q_{j,w}, k_{j/G,t'}> / sqrt(128))_t,
 * G = q_heads / H, over the stored (rotary-embedded) keys; fp16 products, fp32 sums and
 * softmax, fp64 sum over kv heads. The selection is the one of nq_score_evict.
 *   K          fp16 [L][H][T][128]
 *   Q_obs      fp16 [layer_end-layer_begin][q_heads][window][128], used as given (already
 *              rotary-embedded for their positions); q_heads a positive multiple of H
 *   positions  int32 [layer_end-layer_begin][n_keep] out: kept positions, ascending
 *   scores_opt NULL, or fp64 [layer_end-layer_begin][T] out: s_t for t in [0, T - W) (other
 *              entries are not written)
 *   workspace  device scratch of nq_score_evict_attn_workspace_bytes(p, q_heads) bytes */
nq_status nq_score_evict_attn(const nq_params *p, const void *K, const void *Q_obs,
                              int32_t q_heads, int32_t *positions, double *scores_opt,
                              void *workspace, size_t ws_bytes, void *stream);

/* Steps 3-6: RoPE removal, Hadamard rotation, E8 quantization, delta coding ("Como funciona"
 * steps 3-6; "E8格点量化"). For every compressed layer, kv head and kept position p (in the
 * order given): keys are rotated back by -p (split-half pairs (i, i+64)); keys and values get
 * the normalised 128-point Hadamard transform; each 8-float group gets the fp16 scale
 * s = smallest fp16 >= max|x| / rho_b (rho_b = 2^(b-1) - 1) and the code c = 2y of the nearest
 * E8 point y to clamp(x / s, -rho_b, rho_b); codes are delta-coded along the kept tokens per
 * (layer, head, dim): d_0 = c_0, d_j = (c_j - c_{j-1}) mod 256.
 *   K, V       fp16 [L][H][T][128]
 *   positions  int32 [L_c][n_keep], ascending, each in [0, T) (out-of-range entries are
 *              clamped into [0, T) and give meaningless codes)
 *   rope_cos, rope_sin  fp32 [T][64] from nq_rope_table
 *   codes_k, codes_v    int8 [L_c][H][n_keep][128] out (delta-coded)
 *   scales_k, scales_v  fp16 [L_c][H][n_keep][16] out */
nq_status nq_encode(const nq_params *p, const void *K, const void *V, const int32_t *positions,
                    const float *rope_cos, const float *rope_sin, int8_t *codes_k,
                    int8_t *codes_v, void *scales_k, void *scales_v, void *stream);

/* Inverse of nq_encode ("技术实现细节": RoPE is restored after quantization): running sum of the
 * deltas mod 256 -> c; x = s * c / 2; inverse normalised Hadamard transform; keys rotated
 * forward by their stored position. Inputs as produced by nq_encode: every running code must
 * stay within [-16, 16] (nq_encode's do: |c| <= 2 rho_b + 1 <= 15, 16 only on an exact
 * parity tie), so every delta lies in [-32, 32]; other byte streams decode to unspecified
 * values.
 *   K_out, V_out  [L_c][H][n_keep][128] out, fp16 or fp32 per out_dtype
 *   workspace     device scratch of nq_decode_workspace_bytes(p) bytes (tile prefixes of the
 *                 running sum; cleared by the call itself, so its contents on entry do not
 *                 matter; calls sharing one workspace must not overlap). Once the call has
 *                 completed, the uint32 at word 1 of the workspace is 0; it is nonzero only if
 *                 a tile's wait for its predecessor's prefix exceeded the kernel's spin limit
 *                 (2^26 polls, never expected), and the outputs are then invalid. */
nq_status nq_decode(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                    const void *scales_k, const void *scales_v, const int32_t *positions,
                    const float *rope_cos, const float *rope_sin, void *K_out, void *V_out,
                    nq_out_dtype out_dtype, void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory at all -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation: nq_decode with its scratch (tile tickets
 * and look-back words) in a static device array of the library instead of a caller workspace.
 * Same arguments, computation and outputs as nq_decode, minus the workspace; the call allocates
 * nothing (no hipMalloc, no library routine that allocates).
 *   - The array holds NQ_DECODE_STATIC_MAX_BYTES = 64 MiB on every GPU the library is loaded
 *     on, until the process ends. Parameters whose nq_decode_workspace_bytes(p) exceed it are
 *     rejected with NQ_ERR_WORKSPACE before any launch (64 MiB covers, e.g., 32 layers x 8 kv
 *     heads x 26215 kept tokens; set NQ_VERBOSE for the sizes).
 *   - The array is looked up once per device, on the first call with that device current;
 *     `stream` must belong to the current device.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents (the
 *     call clears what must start at zero itself). Calls that overlap on one GPU -- on two
 *     streams, or from two host threads -- race and give invalid outputs: serialise them.
 *   - The look-back spin-limit flag (word 1 of nq_decode's workspace) is not readable here. */
#define NQ_DECODE_STATIC_MAX_BYTES ((size_t)64 << 20)
nq_status nq_decode_static(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                           const void *scales_k, const void *scales_v, const int32_t *positions,
                           const float *rope_cos, const float *rope_sin, void *K_out,
                           void *V_out, nq_out_dtype out_dtype, void *stream);

/* One-token grouped-query attention over a reconstructed cache (consumer check; the VQKV page,
 * "推理流程集成", attends over reconstructed KV). Query head j reads kv head j / (q_heads / H):
 * o_j = sum_t softmax_t(<q_j, k_t> / sqrt(128)) v_t, fp32 softmax with the maximum subtracted.
 *   Q      fp16 [L_c][q_heads][128]; q_heads must be a multiple of H with q_heads/H in
 *          {1, 2, 4, 8}
 *   K, V   fp16 [L_c][H][n_tok][128] (e.g. nq_decode output)
 *   out    fp32 [L_c][q_heads][128] out
 *   workspace  nq_attend_workspace_bytes(p, q_heads, n_tok) bytes */
nq_status nq_attend_decode(const nq_params *p, const void *Q, int32_t q_heads, const void *K,
                           const void *V, int32_t n_tok, float *out, void *workspace,
                           size_t ws_bytes, void *stream);

/* Device workspace needed by nq_decode_attend for q_heads query heads (bytes). 0 if p is
 * invalid. */
size_t nq_decode_attend_workspace_bytes(const nq_params *p, int32_t q_heads);

/* One-token grouped-query attention straight from the compressed cache (the VQKV page,
 * "推理流程集成": reconstruct on demand inside attention). Computes what nq_decode followed by
 * nq_attend_decode over its fp32 output computes -- o_j = sum_t softmax_t(<q_j, k_t> /
 * sqrt(128)) v_t over the n_keep kept tokens, query head j reading kv head j / (q_heads / H),
 * k_t and v_t the reconstructions of step 7 -- without writing k_t, v_t anywhere: keys are
 * rebuilt in registers, and the value sum is accumulated on the dequantised codes with the
 * inverse Hadamard applied once per query head (it is linear). fp32 throughout; the result
 * differs from the two-call path only by rounding order.
 *   codes_k, codes_v, scales_k, scales_v, positions, rope_cos, rope_sin  as for nq_decode
 *   Q      fp16 [L_c][q_heads][128]; q_heads a multiple of H with q_heads/H in {1, 2, 4, 8}
 *   out    fp32 [L_c][q_heads][128] out (zeros when n_keep = 0)
 *   workspace  nq_decode_attend_workspace_bytes(p, q_heads) bytes (look-back words and the
 *              per-tile partials; contents on entry do not matter, calls sharing one
 *              workspace must not overlap; word 1 reports a spin-limit timeout as for
 *              nq_decode) */
nq_status nq_decode_attend(const nq_params *p, const int8_t *codes_k, const int8_t *codes_v,
                           const void *scales_k, const void *scales_v, const int32_t *positions,
                           const float *rope_cos, const float *rope_sin, const void *Q,
                           int32_t q_heads, float *out, void *workspace, size_t ws_bytes,
                           void *stream);

/* Equal-bit scalar baseline (page "Lloyd-Max量化": Lloyd-Max quantization by alternating
 * nearest-level assignment and centroid updates, then table lookup; "3-bit量化的设计选择"). The
 * Lloyd-Max table of the unit Gaussian with 2^bits levels (1 <= bits <= 4), computed on the
 * host once per bit width and made exactly antisymmetric: levels [2^bits] ascending,
 * thresholds [2^bits - 1] (midpoints). Host memory, owned by the caller. */
nq_status nq_lloyd_max_table(int32_t bits, double *levels, double *thresholds);

/* The codec's front end (keys rotated back by their position, normalised Hadamard rotation)
 * with a per-coordinate Lloyd-Max quantizer in place of the E8 step, at bits_k / bits_v bits:
 * per 8-float group the fp16 scale s = RMS of the group (fp32, squares added in dim order,
 * rounded to nearest fp16, saturating at 65504) and per coordinate the index of u = x / s in the table (number of
 * thresholds strictly below u; an all-zero group gets 2^(b-1)). No delta coding.
 *   idx_k, idx_v        uint8 [L_c][H][n_keep][128] out (8-byte aligned)
 *   scales_k, scales_v  fp16 [L_c][H][n_keep][16] out
 *   other arguments as for nq_encode */
nq_status nq_encode_scalar(const nq_params *p, const void *K, const void *V,
                           const int32_t *positions, const float *rope_cos, const float *rope_sin,
                           uint8_t *idx_k, uint8_t *idx_v, void *scales_k, void *scales_v,
                           void *stream);

/* Inverse of nq_encode_scalar: x = s * level[index], inverse normalised Hadamard transform,
 * keys rotated forward by their position; fp16 or fp32 output as for nq_decode (no workspace:
 * the indices carry no running sum). */
nq_status nq_decode_scalar(const nq_params *p, const uint8_t *idx_k, const uint8_t *idx_v,
                           const void *scales_k, const void *scales_v, const int32_t *positions,
                           const float *rope_cos, const float *rope_sin, void *K_out,
                           void *V_out, nq_out_dtype out_dtype, void *stream);

/* Static, human-readable name of a status code. */
const char *nq_status_string(nq_status s);

#ifdef __cplusplus
}
#endif

#endif /* NQ_H */
