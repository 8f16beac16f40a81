// Equal-bit scalar baseline: the lattice codec's front end (rotary embedding removed from keys,
// normalised 128-point Hadamard rotation, one fp16 scale per 8-float group) with a Lloyd-Max
// quantizer of the unit Gaussian per coordinate in place of the E8 step, at the same bits per
// coordinate (page "Lloyd-Max量化": sections "量化过程详解" -- alternate nearest-level assignment
// and centroid updates, then quantize by table lookup -- and "3-bit量化的设计选择").
//
// Group scale: the fp16 (nearest even, saturating at 65504) of the group's RMS, sqrt(sum x^2 / 8)
// in fp32 with the squares added in dim order; index = number of thresholds strictly below u = x / s (fp32
// division); an all-zero group takes index 2^(b-1). Indices are stored one per byte, with no
// delta coding. Decode: x = s * level[index], the inverse transform, RoPE at the stored
// position. Tables come from the host (computed once per bit width by the Lloyd-Max iteration).
#pragma once

#include "nq_codec.hpp"

namespace nq {

constexpr int kScalarRun = 8;                    // tokens per lane group
constexpr int kScalarTile = 16 * kScalarRun;     // tokens per block

struct ScalarArgs {
    const uint16_t *K, *V;           // fp16 [L][H][T][128]
    const int32_t *positions;        // [Lc][n_keep]
    const float *rope_cos, *rope_sin;
    uint8_t *idx_k, *idx_v;          // [Lc][H][n_keep][128]
    uint16_t *scales_k, *scales_v;   // fp16 [Lc][H][n_keep][16]
    void *out_k, *out_v;             // decode output, fp16 or fp32
    float thr[2][15];                // [K|V] thresholds, ascending
    float lev[2][16];                // [K|V] levels
    int32_t bits[2];
    int32_t H, T, layer_begin, n_keep, tiles, out_f32;
};

// indices of 8 values: NT thresholds (compile-time count)
template <int NT>
__device__ __forceinline__ uint2 scalar_indices(const float xn[8], float s, const float *thr,
                                                uint32_t half)
{
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; k++) {
        uint32_t id = half;
        if (s != 0.0f) {
            const float u = xn[k] / s;
            id = 0u;
#pragma unroll
            for (int j = 0; j < NT; j++) id += u > thr[j] ? 1u : 0u;
        }
        w[k >> 2] |= id << (8 * (k & 3));
    }
    return make_uint2(w[0], w[1]);
}

template <bool IS_KEY>
__device__ void scalar_encode_tile(const ScalarArgs &a, int lc, int h, int tile)
{
    const int tn = IS_KEY ? 0 : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane_group(lane & 15), q = wave * 4 + (lane >> 4);
    const int n_keep = a.n_keep;
    const size_t chain = (size_t)lc * a.H + h;
    const uint16_t *X = (IS_KEY ? a.K : a.V) +
                        ((size_t)(a.layer_begin + lc) * a.H + h) * (size_t)a.T * kHeadDim + 8 * g;
    const int32_t *pos = a.positions + (size_t)lc * n_keep;
    const int bits = a.bits[tn];
    const uint32_t half = 1u << (bits - 1);
    const float sg = group_sign(g);
    for (int i = 0; i < kScalarRun; i++) {
        const int j = tile * kScalarTile + q * kScalarRun + i;
        if (j >= n_keep) break;
        const int p = min(max(pos[j], 0), a.T - 1);
        TokenIn t;
        load_token<IS_KEY>(a.rope_cos, a.rope_sin, X, p, g, t);
        float x[8];
        front_end<IS_KEY>(t, g, x);
        // the normalised rotated row (x * fp32(1/sqrt(128)), lane sign restored: exact)
        float xn[8], ss = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            xn[k] = (x[k] * kInvSqrt128) * sg;
            ss = ss + xn[k] * xn[k];
        }
        const uint32_t s16 = min(f2h_bits(sqrtf(ss * 0.125f)), 0x7bffu);   // saturating
        const float s = h2f(s16);
        uint2 id;
        if (bits == 2) id = scalar_indices<3>(xn, s, a.thr[tn], half);
        else if (bits == 3) id = scalar_indices<7>(xn, s, a.thr[tn], half);
        else id = scalar_indices<15>(xn, s, a.thr[tn], half);
        const size_t row = chain * (size_t)n_keep + j;
        *reinterpret_cast<uint2 *>((IS_KEY ? a.idx_k : a.idx_v) + row * kHeadDim + 8 * g) = id;
        (IS_KEY ? a.scales_k : a.scales_v)[row * kGroups + g] = (uint16_t)s16;
    }
}

// grid: Lc * 2 * H * tiles blocks of kCodecThreads; tile = kScalarTile kept tokens of one
// (layer, K|V, head) chain
__global__ __launch_bounds__(kCodecThreads) void k_encode_scalar(ScalarArgs a)
{
    const uint32_t b = blockIdx.x;
    const int tile = b % a.tiles;
    uint32_t r = b / a.tiles;
    const int h = r % a.H;
    r /= a.H;
    if (r & 1) scalar_encode_tile<false>(a, (int)(r >> 1), h, tile);
    else scalar_encode_tile<true>(a, (int)(r >> 1), h, tile);
}

template <bool IS_KEY>
__device__ void scalar_decode_tile(const ScalarArgs &a, int lc, int h, int tile, const float *lev)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane_group(lane & 15), q = wave * 4 + (lane >> 4);
    const int n_keep = a.n_keep;
    const size_t chain = (size_t)lc * a.H + h;
    const size_t row_off = chain * (size_t)n_keep * kHeadDim;
    const int32_t *pos = a.positions + (size_t)lc * n_keep;
    for (int i = 0; i < kScalarRun; i++) {
        const int j = tile * kScalarTile + q * kScalarRun + i;
        if (j >= n_keep) break;
        const size_t row = chain * (size_t)n_keep + j;
        const uint2 id = *reinterpret_cast<const uint2 *>((IS_KEY ? a.idx_k : a.idx_v) +
                                                          row * kHeadDim + 8 * g);
        const float sc = h2f((IS_KEY ? a.scales_k : a.scales_v)[row * kGroups + g]);
        // x = s * level, with the 1/sqrt(128) of the normalised transform
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const uint32_t w = k < 4 ? id.x : id.y;
            x[k] = (sc * lev[(w >> (8 * (k & 3))) & 15u]) * kInvSqrt128;
        }
        hadamard_butterflies(x, g);   // x = group_sign(g) * (the reconstructed row)
        if (IS_KEY) {
            const int p = min(max(pos[j], 0), a.T - 1);
            float cr[8], sr[8];
            load_f32x8(a.rope_cos + (size_t)p * 64 + 8 * (g & 7), cr);
            load_f32x8(a.rope_sin + (size_t)p * 64 + 8 * (g & 7), sr);
            rope_redo(x, g, cr, sr);
        }
        store_row(IS_KEY ? a.out_k : a.out_v, a.out_f32, row_off, j, g, x);
    }
}

__global__ __launch_bounds__(kCodecThreads) void k_decode_scalar(ScalarArgs a)
{
    __shared__ float s_lev[16];
    const uint32_t b = blockIdx.x;
    const int tile = b % a.tiles;
    uint32_t r = b / a.tiles;
    const int h = r % a.H;
    r /= a.H;
    const int tn = (int)(r & 1);
    if (threadIdx.x < 16) s_lev[threadIdx.x] = a.lev[tn][threadIdx.x];
    __syncthreads();
    if (tn) scalar_decode_tile<false>(a, (int)(r >> 1), h, tile, s_lev);
    else scalar_decode_tile<true>(a, (int)(r >> 1), h, tile, s_lev);
}

}  // namespace nq
