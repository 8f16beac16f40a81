// One-token grouped-query attention over a reconstructed cache (consumer check of the decode;
// the VQKV page, "推理流程集成", attends over reconstructed KV during decoding).
//
// Split-K ("flash decoding"): a block owns a chunk of tokens of one (layer, kv head) and all G
// query heads that share that kv head, so every K/V row is read once for G queries. The block
// walks its chunk in tiles with an online softmax per head (one rescale per tile), lane groups
// and waves are merged in registers and LDS, and a second kernel merges the chunks. fp32.
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

// A block walks its chunk in tiles of kAttTile tokens; lane group q takes tile rows
// q * kAttRun .. + kAttRun (consecutive rows: each lane group reads contiguous memory). Per tile:
// the scores of all rows and heads go to LDS (G dot products per lane and a transpose-reduce over
// the 16 lanes of a row, as in the fused kernel), one softmax step per head over the tile moves
// the block's running max and sum and gives every row its weight exp(z - m), and the lanes add
// weight x value into their accumulators, which are rescaled once per tile when the max grows.
// Rows past the chunk's end compute on its last row and weigh 0, so no branch sits between a
// row's load and its use; rows are requested kAttAhead rows ahead.
constexpr int kAttRun = 16;                   // rows per lane group and tile
constexpr int kAttTile = 16 * kAttRun;        // rows per tile
constexpr int kAttAhead = 2;
static_assert(kAttTile == kAttThreads, "the tile softmax gives every thread one row");

template <int G>
struct AttShared {
    float z[kAttTile][G];     // scores, then weights
    float ml[G][2];           // running max and sum per head
    float alpha[G];           // this tile's rescale of the accumulators
    float red[4][G][16][9];   // per-wave accumulators
};

template <int G>
__global__ __launch_bounds__(kAttThreads) void k_attend(AttArgs a)
{
    __shared__ AttShared<G> sh;
    const int blk = blockIdx.x;
    const int split = blk % a.nsplit;
    const int lh = blk / a.nsplit;
    const int lc = lh / a.H, h = lh % a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 15, q = wave * 4 + (lane >> 4);
    const int per = (a.n + a.nsplit - 1) / a.nsplit;
    const int c0 = split * per, c1 = min(a.n, c0 + per);

    // queries of this kv head, this lane's 8 dims, times 1/sqrt(128)
    float qv[G][8];
#pragma unroll
    for (int i = 0; i < G; i++) {
        load_f16x8(a.Q + ((size_t)lc * a.Hq + h * G + i) * kHeadDim + 8 * g, qv[i]);
#pragma unroll
        for (int k = 0; k < 8; k++) qv[i][k] *= kInvSqrt128;
    }
    const uint16_t *Kh = a.K + ((size_t)lc * a.H + h) * (size_t)a.n * kHeadDim + 8 * g;
    const uint16_t *Vh = a.V + ((size_t)lc * a.H + h) * (size_t)a.n * kHeadDim + 8 * g;
    if (threadIdx.x < G) { sh.ml[threadIdx.x][0] = -INFINITY; sh.ml[threadIdx.x][1] = 0.0f; }

    float acc[G][8];
#pragma unroll
    for (int i = 0; i < G; i++)
#pragma unroll
        for (int k = 0; k < 8; k++) acc[i][k] = 0.0f;

    for (int t0 = c0; t0 < c1; t0 += kAttTile) {
        const int nt = min(kAttTile, c1 - t0), r0 = q * kAttRun;
        // ---- scores of the tile's rows
        {
            float kx[kAttAhead + 1][8];
#pragma unroll
            for (int i = 0; i < kAttAhead; i++)
                load_f16x8_stream(Kh + (size_t)(t0 + min(r0 + i, nt - 1)) * kHeadDim, kx[i]);
#pragma unroll
            for (int i = 0; i < kAttRun; i++) {
                const int r = r0 + i, cur = i % (kAttAhead + 1);
                if (i + kAttAhead < kAttRun)
                    load_f16x8_stream(Kh + (size_t)(t0 + min(r + kAttAhead, nt - 1)) * kHeadDim,
                                      kx[(i + kAttAhead) % (kAttAhead + 1)]);
                float d[G];
#pragma unroll
                for (int hq = 0; hq < G; hq++) {
                    d[hq] = qv[hq][0] * kx[cur][0];
#pragma unroll
                    for (int k = 1; k < 8; k++) d[hq] = __builtin_fmaf(qv[hq][k], kx[cur][k], d[hq]);
                }
                const float z = row_sums<G>(d, g);
                if (r < nt && row_sum_reporter<G>(g)) sh.z[r][row_sum_index<G>(g)] = z;
            }
        }
        __syncthreads();
        // ---- one softmax step per head: wave w handles heads w, w + 4, ...
        for (int hq = wave; hq < G; hq += 4) {
            float zr[kAttTile / 64];
            float m = -INFINITY;
#pragma unroll
            for (int k = 0; k < kAttTile / 64; k++) {
                const int r = lane + 64 * k;
                zr[k] = r < nt ? sh.z[r][hq] : -INFINITY;
                m = fmaxf(m, zr[k]);
            }
#pragma unroll
            for (int msk = 1; msk < 64; msk <<= 1) m = fmaxf(m, __shfl_xor(m, msk));
            const float m_old = sh.ml[hq][0], M = fmaxf(m_old, m);   // nt >= 1: M is finite
            float l = 0.0f;
#pragma unroll
            for (int k = 0; k < kAttTile / 64; k++) {
                const int r = lane + 64 * k;
                const float pr = r < nt ? expf(zr[k] - M) : 0.0f;
                sh.z[r][hq] = pr;   // 0 past the chunk's end
                l += pr;
            }
#pragma unroll
            for (int msk = 1; msk < 64; msk <<= 1) l += __shfl_xor(l, msk);
            if (lane == 0) {
                const float al = m_old == -INFINITY ? 0.0f : expf(m_old - M);
                sh.alpha[hq] = al;
                sh.ml[hq][1] = sh.ml[hq][1] * al + l;
                sh.ml[hq][0] = M;
            }
        }
        __syncthreads();
        // ---- weighted values
        {
#pragma unroll
            for (int hq = 0; hq < G; hq++) {
                const float al = sh.alpha[hq];
#pragma unroll
                for (int k = 0; k < 8; k++) acc[hq][k] *= al;
            }
            float vx[kAttAhead + 1][8];
#pragma unroll
            for (int i = 0; i < kAttAhead; i++)
                load_f16x8_stream(Vh + (size_t)(t0 + min(r0 + i, nt - 1)) * kHeadDim, vx[i]);
#pragma unroll
            for (int i = 0; i < kAttRun; i++) {
                const int r = r0 + i, cur = i % (kAttAhead + 1);
                if (i + kAttAhead < kAttRun)
                    load_f16x8_stream(Vh + (size_t)(t0 + min(r + kAttAhead, nt - 1)) * kHeadDim,
                                      vx[(i + kAttAhead) % (kAttAhead + 1)]);
#pragma unroll
                for (int hq = 0; hq < G; hq++) {
                    const float w = sh.z[r][hq];
#pragma unroll
                    for (int k = 0; k < 8; k++) acc[hq][k] = __builtin_fmaf(w, vx[cur][k], acc[hq][k]);
                }
            }
        }
        __syncthreads();   // the weights and alpha of this tile are no longer read
    }
    // sum over the 4 rows of the wave (lane distance 16, 32), then over the 4 waves in LDS
#pragma unroll
    for (int msk = 16; msk < 64; msk <<= 1)
#pragma unroll
        for (int hq = 0; hq < G; hq++)
#pragma unroll
            for (int k = 0; k < 8; k++) acc[hq][k] += __shfl_xor(acc[hq][k], msk);
    if (lane < 16) {
#pragma unroll
        for (int hq = 0; hq < G; hq++)
#pragma unroll
            for (int k = 0; k < 8; k++) sh.red[wave][hq][lane][k] = acc[hq][k];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kAttThreads) {
        const int i = idx / kHeadDim, d = idx % kHeadDim, l16 = d >> 3, k = d & 7;
        const float A = sh.red[0][i][l16][k] + sh.red[1][i][l16][k] + sh.red[2][i][l16][k] +
                        sh.red[3][i][l16][k];
        if (d == 0) {
            a.part_m[(size_t)blk * G + i] = sh.ml[i][0];
            a.part_l[(size_t)blk * G + i] = sh.ml[i][1];
        }
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
