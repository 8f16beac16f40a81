// One-token grouped-query attention over a reconstructed cache (consumer check of the decode;
// the VQKV page, "推理流程集成", attends over reconstructed KV during decoding).
//
// Split-K ("flash decoding"): a block owns a chunk of tokens of one (layer, kv head) and all G
// query heads that share that kv head, so every K/V row is read once for G queries. Each lane
// group streams rows, keeps an online softmax (running max, sum, and its 8 output dims), lane
// groups are merged in registers and LDS, and a second kernel merges the chunks. fp32.
#pragma once

#include "nq_common.hpp"

namespace nq {

constexpr int kAttThreads = 256;

struct AttArgs {
    const uint16_t *Q;      // [Lc][Hq][128]
    const uint16_t *K, *V;  // [Lc][H][n][128]
    float *out;             // [Lc][Hq][128]
    float *part_m, *part_l, *part_acc;  // [blocks][G], [blocks][G], [blocks][G][128]
    int32_t H, Hq, n, nsplit;
};

__device__ __forceinline__ void softmax_merge(float &m, float &l, float *acc, float m2, float l2,
                                              const float *acc2)
{
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float a1 = expf(m - M), a2 = expf(m2 - M);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int k = 0; k < 8; k++) acc[k] = acc[k] * a1 + acc2[k] * a2;
    m = M;
}

template <int G>
__global__ __launch_bounds__(kAttThreads) void k_attend(AttArgs a)
{
    __shared__ float s_m[4][G], s_l[4][G];
    __shared__ float s_acc[4][G][kHeadDim];
    const int blk = blockIdx.x;
    const int split = blk % a.nsplit;
    const int lh = blk / a.nsplit;
    const int lc = lh / a.H, h = lh % a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 15, q = wave * 4 + (lane >> 4);
    const int per = (a.n + a.nsplit - 1) / a.nsplit;
    const int c0 = split * per, c1 = min(a.n, c0 + per);

    float qv[G][8];
#pragma unroll
    for (int i = 0; i < G; i++)
        load_f16x8(a.Q + ((size_t)lc * a.Hq + h * G + i) * kHeadDim + 8 * g, qv[i]);
    const uint16_t *Kh = a.K + ((size_t)lc * a.H + h) * (size_t)a.n * kHeadDim + 8 * g;
    const uint16_t *Vh = a.V + ((size_t)lc * a.H + h) * (size_t)a.n * kHeadDim + 8 * g;

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int i = 0; i < G; i++) {
        m[i] = -INFINITY;
        l[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++) acc[i][k] = 0.0f;
    }
    for (int t = c0 + q; t < c1; t += 16) {
        float kx[8], vx[8];
        load_f16x8(Kh + (size_t)t * kHeadDim, kx);
        load_f16x8(Vh + (size_t)t * kHeadDim, vx);
#pragma unroll
        for (int i = 0; i < G; i++) {
            float d = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; k++) d = __builtin_fmaf(qv[i][k], kx[k], d);
#pragma unroll
            for (int msk = 1; msk < 16; msk <<= 1) d += __shfl_xor(d, msk);
            const float z = d * kInvSqrt128;
            const float M = fmaxf(m[i], z);
            const float alpha = expf(m[i] - M), p = expf(z - M);
            l[i] = l[i] * alpha + p;
#pragma unroll
            for (int k = 0; k < 8; k++) acc[i][k] = __builtin_fmaf(p, vx[k], acc[i][k] * alpha);
            m[i] = M;
        }
    }
    // merge the 4 lane groups of this wave (partner lane groups at lane distance 16, 32)
#pragma unroll
    for (int msk = 16; msk < 64; msk <<= 1) {
#pragma unroll
        for (int i = 0; i < G; i++) {
            const float m2 = __shfl_xor(m[i], msk), l2 = __shfl_xor(l[i], msk);
            float a2[8];
#pragma unroll
            for (int k = 0; k < 8; k++) a2[k] = __shfl_xor(acc[i][k], msk);
            softmax_merge(m[i], l[i], acc[i], m2, l2, a2);
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int i = 0; i < G; i++) {
            if (g == 0) { s_m[wave][i] = m[i]; s_l[wave][i] = l[i]; }
#pragma unroll
            for (int k = 0; k < 8; k++) s_acc[wave][i][8 * g + k] = acc[i][k];
        }
    }
    __syncthreads();
    // merge the 4 waves; thread (i, d) for i < G, d < 128
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kAttThreads) {
        const int i = idx / kHeadDim, d = idx % kHeadDim;
        float M = -INFINITY;
        for (int w = 0; w < 4; w++) M = fmaxf(M, s_m[w][i]);
        float L = 0.0f, A = 0.0f;
        if (M != -INFINITY) {
            for (int w = 0; w < 4; w++) {
                const float f = expf(s_m[w][i] - M);
                L += s_l[w][i] * f;
                A += s_acc[w][i][d] * f;
            }
        }
        if (d == 0) { a.part_m[(size_t)blk * G + i] = M; a.part_l[(size_t)blk * G + i] = L; }
        a.part_acc[((size_t)blk * G + i) * kHeadDim + d] = A;
    }
}

// merge the nsplit chunks: one block per (layer, query head), 128 threads
__global__ __launch_bounds__(128) void k_attend_merge(AttArgs a, int G)
{
    const int lj = blockIdx.x;
    const int lc = lj / a.Hq, j = lj % a.Hq;
    const int h = j / G, i = j % G;
    const int d = threadIdx.x;
    const size_t b0 = ((size_t)lc * a.H + h) * a.nsplit;
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; s++) M = fmaxf(M, a.part_m[(b0 + s) * G + i]);
    float L = 0.0f, A = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < a.nsplit; s++) {
            const float f = expf(a.part_m[(b0 + s) * G + i] - M);
            L += a.part_l[(b0 + s) * G + i] * f;
            A += a.part_acc[((b0 + s) * G + i) * kHeadDim + d] * f;
        }
    }
    a.out[((size_t)lc * a.Hq + j) * kHeadDim + d] = L > 0.0f ? A / L : 0.0f;
}

}  // namespace nq
