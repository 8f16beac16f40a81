// Attention-weight scoring (the "real attention scorer" choice of the page
// "NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破", section "技术实现细节"; tokens are
// ranked by their attention weights, section "Token淘汰机制").
//
// An observation window of W queries per query head (query w at position P_w = T - W + w)
// scores every key by the softmax weight it receives, summed over the window and over all query
// heads: s_t = sum_j sum_w [t <= P_w] softmax_{t' <= P_w}(q_{j,w} . k_{h(j),t'} / sqrt(128))_t,
// h(j) = j / G. Per (layer, kv head) pair the G * W query rows and the T keys form a matrix
// product with k = 128 -- the one dense contraction of the method, on matrix cores
// (v_mfma_f32_32x32x16_f16: fp16 products exact, fp32 sums). Two passes:
//   1. k_attn_rowbias: for every query row the log2-domain max m and sum l of its softmax
//      (online over key tiles); stored as the bias m + log2 l.
// Exponentials are the hardware's v_exp_f32 (exp2): terms below 2^-126 -- against a softmax sum
// of at least 1 -- may flush to zero.
//   2. k_attn_colsum: for every candidate key the column sum of exp2(z - bias) over the pair's
//      rows. Candidates (t < T - W) precede every query's position, so no mask is needed.
// k_attn_finish adds the kv heads in fp64; the selection is the key-key path's k_select.
//
// MFMA lane layout (32x32x16, wave64; A 32 x 16, B 16 x 32, D 32 x 32): lane l supplies row
// l % 32 of A and column l % 32 of B, 8 halves each, for contraction slots (l / 32, e); D
// element (i / 4) * 8 + (l / 32) * 4 + i % 4, l % 32 sits in accumulator i of lane l. The
// contraction's dims are assigned to slots as dim = (l / 32) * 64 + step * 8 + e, so each lane
// reads one contiguous 128-byte half of a row over the 8 steps.
#pragma once

#include <type_traits>

#include "nq_common.hpp"

namespace nq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAttnThreads = 512;                 // 8 waves
constexpr int kAttnRows = 256;                    // query rows per pass-1 block (8 x 32)
constexpr int kAttnKeys = 256;                    // keys per pass-2 block (8 x 32)
constexpr int kKTile = 64;                        // keys per LDS tile (pass 1)
constexpr int kQTile = 32;                        // query rows per LDS tile (pass 2)
constexpr int kRowPad = kHeadDim + 8;             // LDS row stride in halves: 272 B, so the
                                                  // 16-byte reads of 16 lanes hit 64 banks
constexpr float kLog2eInvSqrt128 = 0x1.0527dcp-3f;   // fp32(log2(e) / sqrt(128))

struct AttnScoreArgs {
    const uint16_t *K;     // fp16 [L][H][T][128]
    const uint16_t *Q;     // fp16 [Lc][Hq][W][128]
    float *bias;           // [pairs][R]: m + log2 l of each query row (log2 units)
    float *colsum;         // [pairs][T]: column sums (t < T - W)
    double *scores;        // [Lc][T]
    int32_t H, G, W, T, R, layer_begin, row_chunks, key_chunks;
};

// block -> (pair, chunk): the chunks of one pair get block ids of equal residue mod 8, i.e.
// land on one XCD (blocks are dealt to the 8 XCDs round-robin), and start close in time, so the
// operand they share (the pair's keys, resp. queries) is fetched once into that XCD's L2
__device__ __forceinline__ void pair_chunk(uint32_t b, int pairs, int chunks, int &pair,
                                           int &chunk)
{
    if ((pairs & 7) == 0) {
        const uint32_t rest = b >> 3;
        chunk = (int)(rest % (uint32_t)chunks);
        pair = (int)((rest / (uint32_t)chunks) * 8 + (b & 7));
    } else {
        pair = (int)(b / (uint32_t)chunks);
        chunk = (int)(b % (uint32_t)chunks);
    }
}

// wait for every outstanding vector-memory load of this wave (vmcnt 0; other counters left
// at their maxima). Issued before the tile loops, so that the operands loaded once up front
// are known to be complete inside the loop, whose only outstanding load is then the prefetch
// of the next tile -- without it the compiler waits for that prefetch before the first matrix
// instruction of every iteration.
// s_waitcnt encoding (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ f16x8 lds_f16x8(const _Float16 *p)
{
    return *reinterpret_cast<const f16x8 *>(p);
}

__device__ __forceinline__ f16x8 gl_f16x8(const uint16_t *p)
{
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    return __builtin_bit_cast(f16x8, v);
}

// sum of 16 values as a balanced tree (rounding error grows with the depth, 4, not the count)
__device__ __forceinline__ float sum16(const float (&e)[16])
{
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; i++) a[i] = e[2 * i] + e[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; i++) a[i] = a[2 * i] + a[2 * i + 1];
    return (a[0] + a[1]) + (a[2] + a[3]);
}

// ---- pass 1: per-row softmax statistics ----------------------------------------------------
// block = 256 query rows of one pair (wave w owns rows w*32 .. +32, one per lane column);
// D = K_tile (32 keys) x Q^T (32 rows): every lane ends with 16 logits of its own row.
__global__ __launch_bounds__(kAttnThreads) void k_attn_rowbias(AttnScoreArgs a)
{
    __shared__ __align__(16) _Float16 ks[2][kKTile][kRowPad];
    int pair, chunk;
    pair_chunk(blockIdx.x, (int)(gridDim.x / (uint32_t)a.row_chunks), a.row_chunks, pair, chunk);
    const int lc = pair / a.H, h = pair % a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, h2 = lane >> 5;
    const int T = a.T, W = a.W;
    const int r = chunk * kAttnRows + wave * 32 + n;
    const bool valid = r < a.R;
    const int wq = valid ? r % W : 0;
    const int j = h * a.G + (valid ? r / W : 0);
    const int P = valid ? T - W + wq : -1;          // this row's position; < 0: sees no key

    f16x8 qb[8];
    {
        const uint16_t *qp = a.Q + (((size_t)lc * (a.H * a.G) + j) * W + wq) * kHeadDim + h2 * 64;
#pragma unroll
        for (int s = 0; s < 8; s++) qb[s] = valid ? gl_f16x8(qp + s * 8) : f16x8{};
    }
    // keys 0 .. pmax are needed by some row of the block
    const int r0 = chunk * kAttnRows, r1 = min(a.R, r0 + kAttnRows) - 1;
    const int wmax = (r1 - r0 + 1 >= W || r0 % W > r1 % W) ? W - 1 : r1 % W;
    const int pmax = min(T - 1, T - W + wmax);
    const int nkt = pmax >= 0 ? pmax / kKTile + 1 : 0;
    const uint16_t *Kp = a.K + ((size_t)(a.layer_begin + lc) * a.H + h) * (size_t)T * kHeadDim;

    // staging: a tile is 64 rows x 16 chunks of 16 B; thread c moves chunks c and c + 512
    uint4 st[2];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int c = threadIdx.x + u * kAttnThreads, row = c >> 4, part = c & 15;
            const int t = kt * kKTile + row;
            st[u] = t < T ? *reinterpret_cast<const uint4 *>(Kp + (size_t)t * kHeadDim + part * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int c = threadIdx.x + u * kAttnThreads, row = c >> 4, part = c & 15;
            *reinterpret_cast<uint4 *>(&ks[buf][row][part * 8]) = st[u];
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;
    // one 64-key tile: 2 x (8 matrix steps, then the online max/sum of 16 logits per lane);
    // MASK: the tile holds keys past some row's position (only the last tiles do)
    auto tile = [&](int kt, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int buf = kt & 1;
        if (kt + 1 < nkt) load_tile(kt + 1);
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < 8; s++)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    lds_f16x8(&ks[buf][kb * 32 + n][h2 * 64 + s * 8]), qb[s], acc, 0, 0, 0);
            // raw logits (the positive scale commutes with max); masked keys -> -inf
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                if constexpr (MASK) {
                    const int t = kt * kKTile + kb * 32 + (i >> 2) * 8 + h2 * 4 + (i & 3);
                    acc[i] = t <= P ? acc[i] : -INFINITY;
                }
                mt = fmaxf(mt, acc[i]);
            }
            const float mn = fmaxf(m_run, mt * kLog2eInvSqrt128);
            const float mref = mn == -INFINITY ? 0.0f : mn;
            float e[16];
#pragma unroll
            for (int i = 0; i < 16; i++)
                e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], kLog2eInvSqrt128, -mref));
            // the block's 16 terms summed as a tree, then one step of the running sum: the
            // sequential chain over a row is T / 32 adds long instead of T / 2
            l_run = __builtin_fmaf(l_run, __builtin_amdgcn_exp2f(m_run - mref), sum16(e));
            m_run = mn;
        }
        asm volatile("" ::"v"(l_run), "v"(m_run) : "memory");   // as in k_attn_colsum
        if (kt + 1 < nkt) store_tile(buf ^ 1);
        __syncthreads();
    };
    if (nkt > 0) {
        load_tile(0);
        store_tile(0);
    }
    wait_vmem();
    __syncthreads();
    // tiles whose keys all precede the first window position need no mask
    const int nkt_plain = min(nkt, max(0, (T - W + 1) / kKTile));
    for (int kt = 0; kt < nkt_plain; kt++) tile(kt, std::false_type{});
    for (int kt = nkt_plain; kt < nkt; kt++) tile(kt, std::true_type{});
    // lanes n and n + 32 saw different keys of the same row
    const float m2 = __shfl_xor(m_run, 32), l2 = __shfl_xor(l_run, 32);
    const float M = fmaxf(m_run, m2);
    const float Mr = M == -INFINITY ? 0.0f : M;
    const float L = l_run * __builtin_amdgcn_exp2f(m_run - Mr) + l2 * __builtin_amdgcn_exp2f(m2 - Mr);
    if (valid && h2 == 0) a.bias[(size_t)pair * a.R + r] = Mr + log2f(L);
}

// ---- pass 2: column sums over the query rows ------------------------------------------------
// block = 256 candidate keys of one pair (wave w owns keys w*32 .. +32, one per lane column);
// D = Q_tile (32 rows) x K^T (32 keys): every lane accumulates 16 rows of its own key column.
__global__ __launch_bounds__(kAttnThreads) void k_attn_colsum(AttnScoreArgs a)
{
    __shared__ __align__(16) _Float16 qs[3][kQTile][kRowPad];
    __shared__ __align__(16) float bs[3][kQTile];
    int pair, chunk;
    pair_chunk(blockIdx.x, (int)(gridDim.x / (uint32_t)a.key_chunks), a.key_chunks, pair, chunk);
    const int lc = pair / a.H, h = pair % a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, h2 = lane >> 5;
    const int T = a.T, W = a.W, c_end = T - W;
    const int t = chunk * kAttnKeys + wave * 32 + n;
    const bool valid = t < c_end;

    f16x8 kb[8];
    {
        const uint16_t *kp =
            a.K + (((size_t)(a.layer_begin + lc) * a.H + h) * (size_t)T + (valid ? t : 0)) *
                      kHeadDim + h2 * 64;
#pragma unroll
        for (int s = 0; s < 8; s++) kb[s] = valid ? gl_f16x8(kp + s * 8) : f16x8{};
    }
    const int nqt = (a.R + kQTile - 1) / kQTile;
    const int Hq = a.H * a.G;
    // staging: a tile is 32 rows x 16 chunks of 16 B, one chunk per thread (row threadIdx / 16),
    // plus the 32 rows' biases (threads 0..31, row threadIdx). Row r is window query r % W of
    // query head h * G + r / W; each thread walks its row's (head, w) along with the tiles.
    uint4 st;
    float sb = INFINITY;
    const int my_row = threadIdx.x >> 4, part = threadIdx.x & 15;
    int qh = my_row / W, qw = my_row % W;                     // staged chunk's row
    int bw = threadIdx.x % W;                                 // staged bias's row (< 32)
    const uint16_t *Qpair = a.Q + ((size_t)lc * Hq + h * a.G) * W * kHeadDim + part * 8;
    auto load_tile = [&](int qt) {
        const int r = qt * kQTile + my_row;
        const bool ok = r < a.R && T - W + qw >= 0;
        st = ok ? *reinterpret_cast<const uint4 *>(Qpair + ((size_t)qh * W + qw) * kHeadDim)
                : make_uint4(0u, 0u, 0u, 0u);
        if (threadIdx.x < kQTile) {
            const int rb = qt * kQTile + threadIdx.x;
            const bool okb = rb < a.R && T - W + bw >= 0;
            sb = okb ? a.bias[(size_t)pair * a.R + rb] : INFINITY;   // invalid rows weigh 0
        }
        // advance both rows by one tile (32 rows)
        qw += kQTile;
        bw += kQTile;
        while (qw >= W) { qw -= W; qh++; }
        while (bw >= W) bw -= W;
    };
    auto store_tile = [&](int buf) {
        *reinterpret_cast<uint4 *>(&qs[buf][my_row][part * 8]) = st;
        if (threadIdx.x < kQTile) bs[buf][threadIdx.x] = sb;
    };

    // Software pipeline over the query tiles, three LDS buffers: in iteration qt the matrix
    // steps of tile qt + 1 are issued (into the second accumulator) before the exponentials of
    // tile qt, so the matrix pipe and the vector ALU work at the same time; tile qt + 2 is
    // fetched meanwhile and stored at the end of the iteration.
    auto chain = [&](int buf) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < 8; s++)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(lds_f16x8(&qs[buf][n][h2 * 64 + s * 8]),
                                                         kb[s], acc, 0, 0, 0);
        return acc;
    };
    float col = 0.0f;
    if (nqt > 0) {
        load_tile(0);
        store_tile(0);
    }
    if (nqt > 1) {
        load_tile(1);
        store_tile(1);
    }
    wait_vmem();
    __syncthreads();
    // one pipeline step: issue tile qt + 1 into `next`, exponentiate tile qt from `cur`
    // (buffer qt % 3), store tile qt + 2; two steps per loop trip with the accumulators'
    // roles swapped, so no accumulator is copied
    auto step = [&](int qt, const f32x16 &cur, f32x16 &next) {
        const int buf = qt % 3, nbuf = (qt + 1) % 3, fbuf = (qt + 2) % 3;
        if (qt + 2 < nqt) load_tile(qt + 2);
        if (qt + 1 < nqt) next = chain(nbuf);
        // row of accumulator i: (i / 4) * 8 + h2 * 4 + i % 4 -> biases in 4 runs of 4
        float e[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; i4++) {
            const float4 b = *reinterpret_cast<const float4 *>(&bs[buf][i4 * 8 + h2 * 4]);
            e[4 * i4 + 0] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[4 * i4 + 0], kLog2eInvSqrt128, -b.x));
            e[4 * i4 + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[4 * i4 + 1], kLog2eInvSqrt128, -b.y));
            e[4 * i4 + 2] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[4 * i4 + 2], kLog2eInvSqrt128, -b.z));
            e[4 * i4 + 3] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[4 * i4 + 3], kLog2eInvSqrt128, -b.w));
        }
        col += sum16(e);
        // keep the store of the prefetched tile (and its wait for the load) below the
        // exponentials: an empty asm that consumes their sum and orders memory; the compiler
        // would otherwise hoist the store, stall on the load, and sink the math past the barrier
        asm volatile("" ::"v"(col) : "memory");
        if (qt + 2 < nqt) store_tile(fbuf);
        __syncthreads();
    };
    f32x16 acc0 = nqt > 0 ? chain(0) : f32x16{}, acc1 = {};
    for (int qt = 0; qt < nqt; qt += 2) {
        step(qt, acc0, acc1);
        if (qt + 1 < nqt) step(qt + 1, acc1, acc0);
    }
    col += __shfl_xor(col, 32);   // lanes n and n + 32 summed different rows of one key
    if (valid && h2 == 0) a.colsum[(size_t)pair * T + t] = col;
}

// ---- the kv heads' column sums added in fp64: scores of t < T - W ---------------------------
__global__ __launch_bounds__(256) void k_attn_finish(AttnScoreArgs a, int Lc)
{
    const int c_end = a.T - a.W;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c_end <= 0 || i >= (int64_t)Lc * c_end) return;
    const int64_t lc = i / c_end, t = i % c_end;
    double s = 0.0;   // no query rows (W = 0): every weight is 0
    if (a.R > 0)
        for (int h = 0; h < a.H; h++) s += (double)a.colsum[((size_t)lc * a.H + h) * a.T + t];
    a.scores[(size_t)lc * a.T + t] = s;
}

}  // namespace nq
