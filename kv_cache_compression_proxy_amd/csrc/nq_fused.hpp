// One-token grouped-query attention straight from the compressed cache: the delta codes and
// scales are decoded inside the attention kernel and the reconstructed K/V never reach HBM
// (the VQKV page, "推理流程集成": reconstruct on demand while decoding, attending over the
// reconstructed cache).
//
// A block owns one tile of kFusedTile kept tokens of one (layer, kv head) pair and the G query
// heads that share that kv head. Keys: the K chain's running codes come from the same staged
// scan and decoupled look-back as nq_decode; each key row is rebuilt in registers (inverse
// Hadamard, RoPE at its position) and dotted with the G queries. Values: because
// v_t = H x_t / sqrt(128) with x_t = s_t c_t / 2 and H linear, the softmax-weighted sum of the
// values is H (sum_t p_t x_t) / sqrt(128) -- the tile accumulates sum_t p_t x_t on the codes
// directly and the inverse Hadamard runs once per query head in the merge kernel. Tiles write
// (max, sum, accumulator) partials; the merge combines them (flash-decoding style).
#pragma once

#include "nq_codec.hpp"

namespace nq {

struct FusedArgs {
    const int8_t *codes_k, *codes_v;      // [Lc][H][n][128], delta-coded
    const uint16_t *scales_k, *scales_v;  // [Lc][H][n][16] fp16
    const int32_t *positions;             // [Lc][n]
    const float *rope_cos, *rope_sin;     // [T][64]
    const uint16_t *Q;                    // [Lc][Hq][128] fp16
    float *out;                           // [Lc][Hq][128]
    float *part;                          // [pairs][tiles][G][kPartStride]
    uint32_t *lb_agg, *lb_incl, *lb_ticket;
    int32_t H, Hq, T, n_keep, tiles;      // tiles per pair
};

// a tile partial per query head: running max, sum of weights, then 128 accumulated dims
constexpr int kPartStride = 2 + kHeadDim;
constexpr int kFusedRun = 16;                  // tokens per lane group
constexpr int kFusedTile = 16 * kFusedRun;     // tokens per block

template <int G>
struct FusedShared {
    uint2 tot[4][16];
    uint2 excl[16];
    int32_t pos[kFusedTile];
    float z[kFusedTile][G];   // scores, then weights exp(z - m)
    float ml[G][2];         // the tile's max and sum per query head
    union {
        struct {
            uint4 scale[kFusedTile * kGroups * 2 / 16];
            uint4 delta[kFusedTile * kHeadDim / 16];
        } t;
        float red[4][G][16][9];   // per-wave sums of the value accumulators
    } u;
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// One transpose-reduce level across lane partners l ^ m (DPP control CTRL): lanes whose
// selecting bit is clear keep a + a(partner), the others b + b(partner).
template <int CTRL>
__device__ __forceinline__ float tr_level(float a, float b, bool hi)
{
    return (hi ? b : a) + dpp_f<CTRL>(hi ? a : b);
}

// Sums of G per-lane values d[0..G) over the 16 lanes of a row. Transpose-reduce: the levels
// run over lane partners l ^ 8, l ^ 7, l ^ 2, l ^ 1 (row_ror:8, row_half_mirror, quad_perm);
// while more than one value is live, each level halves them, keeping in every lane the half
// picked by one bit of l (bits 3, 2, 1), so all levels together cost G - 1 + log2(16 / G)
// adds instead of 4 G. Returns the sum of value row_sum_index<G>(l) for this lane l.
template <int G>
__device__ __forceinline__ float row_sums(const float (&d)[G], int l)
{
    constexpr int kRor8 = kDppRor8, kHm = 0x141, kX2 = 0x4E, kX1 = 0xB1;
    const bool b3 = l & 8, b2 = l & 4, b1 = l & 2;
    if constexpr (G == 1) {
        float v = d[0] + dpp_f<kRor8>(d[0]);
        v += dpp_f<kHm>(v);
        v += dpp_f<kX2>(v);
        return v + dpp_f<kX1>(v);
    } else if constexpr (G == 2) {
        float v = tr_level<kRor8>(d[0], d[1], b3);
        v += dpp_f<kHm>(v);
        v += dpp_f<kX2>(v);
        return v + dpp_f<kX1>(v);
    } else if constexpr (G == 4) {
        const float v01 = tr_level<kRor8>(d[0], d[1], b3);
        const float v23 = tr_level<kRor8>(d[2], d[3], b3);
        float v = tr_level<kHm>(v01, v23, b2);
        v += dpp_f<kX2>(v);
        return v + dpp_f<kX1>(v);
    } else {
        static_assert(G == 8, "G in {1, 2, 4, 8}");
        const float v01 = tr_level<kRor8>(d[0], d[1], b3);
        const float v23 = tr_level<kRor8>(d[2], d[3], b3);
        const float v45 = tr_level<kRor8>(d[4], d[5], b3);
        const float v67 = tr_level<kRor8>(d[6], d[7], b3);
        const float v03 = tr_level<kHm>(v01, v23, b2);
        const float v47 = tr_level<kHm>(v45, v67, b2);
        const float v = tr_level<kX2>(v03, v47, b1);
        return v + dpp_f<kX1>(v);
    }
}

// which value row_sums<G> leaves in lane l (0..15), and whether lane l is the one that
// reports it (one lane per value)
template <int G>
__device__ __forceinline__ int row_sum_index(int l)
{
    return (G >= 2 ? (l >> 3) & 1 : 0) | (G >= 4 ? ((l >> 2) & 1) << 1 : 0) |
           (G >= 8 ? ((l >> 1) & 1) << 2 : 0);
}

template <int G>
__device__ __forceinline__ bool row_sum_reporter(int l)
{
    return (l & (G == 1 ? 15 : G == 2 ? 7 : G == 4 ? 3 : 1)) == 0;
}

// grid: pairs * tiles blocks (pairs = Lc * H); tickets tile-major over the pairs as in
// k_decode. Look-back slots: 2 * ticket + tensor (K = 0, V = 1).
template <int G>
__global__ __launch_bounds__(kCodecThreads) void k_decode_attend(FusedArgs a)
{
    __shared__ int s_ticket;
    __shared__ FusedShared<G> sh;
    const int pairs = (int)(gridDim.x / (uint32_t)a.tiles);
    if (threadIdx.x == 0) s_ticket = take_ticket(a.lb_ticket, (uint32_t)pairs);
    __syncthreads();
    const int ticket = s_ticket;
    const int tile = ticket / pairs;
    const int pair = ticket % pairs;
    const int h = pair % a.H, lc = pair / a.H;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane_group(lane & 15), q = wave * 4 + (lane >> 4);
    const int n_keep = a.n_keep;
    const int t0 = tile * kFusedTile;
    const int nt = min(kFusedTile, n_keep - t0);
    const int jl0 = q * kFusedRun;                     // this lane group's first tile row
    const size_t row0 = (size_t)pair * n_keep + t0;    // chain row of the tile's first token

    // queries of this kv head, this lane's 8 dims, times group_sign(g) / sqrt(128): the keys
    // come out of decode_row with group_sign(g) applied, so q . x is the true score
    float qv[G][8];
    {
        const float f = group_sign(g) * kInvSqrt128;
#pragma unroll
        for (int i = 0; i < G; i++) {
            load_f16x8(a.Q + ((size_t)lc * a.Hq + h * G + i) * kHeadDim + 8 * g, qv[i]);
#pragma unroll
            for (int k = 0; k < 8; k++) qv[i][k] *= f;
        }
    }

    // ---- keys: scores z[t][i] of the tile
    stage_tile<kFusedRun>(a.codes_k, a.scales_k, row0, nt, a.positions + (size_t)lc * n_keep + t0, a.T,
               sh.u.t.delta, sh.u.t.scale, sh.pos);
    {
        uint2 run = tile_run_base<kFusedRun>(sh.u.t.delta, nt, q, g, sh.tot, sh.excl, a.lb_agg, a.lb_incl,
                                  2 * (size_t)ticket, 2 * (size_t)pairs, tile,
                                  a.lb_ticket + kTicketErr);
        const uint2 *sd = reinterpret_cast<const uint2 *>(sh.u.t.delta) + g;
        const uint16_t *sl = reinterpret_cast<const uint16_t *>(sh.u.t.scale);
        const int jend = min(nt, jl0 + kFusedRun);
        float rc[2][8], rs[2][8];   // rotary rows of the current and the next token
        if (jl0 < jend) {
            const size_t p = (size_t)sh.pos[jl0] * 64 + 8 * (g & 7);
            load_f32x8(a.rope_cos + p, rc[0]);
            load_f32x8(a.rope_sin + p, rs[0]);
        }
#pragma unroll
        for (int i = 0; i < kFusedRun; i++) {
            const int jl = jl0 + i, cur = i & 1;
            if (jl < jend) {
                if (jl + 1 < jend) {
                    const size_t p = (size_t)sh.pos[jl + 1] * 64 + 8 * (g & 7);
                    load_f32x8(a.rope_cos + p, rc[cur ^ 1]);
                    load_f32x8(a.rope_sin + p, rs[cur ^ 1]);
                }
                run = run_step(run, sd[jl * 16]);
                float x[8];
                decode_row<true>(g, run, sl[jl * kGroups + g], rc[cur], rs[cur], x);
                float d[G];
#pragma unroll
                for (int hq = 0; hq < G; hq++) {
                    d[hq] = 0.0f;
#pragma unroll
                    for (int k = 0; k < 8; k++) d[hq] = __builtin_fmaf(qv[hq][k], x[k], d[hq]);
                }
                const float z = row_sums<G>(d, lane & 15);
                if (row_sum_reporter<G>(lane & 15)) sh.z[jl][row_sum_index<G>(lane & 15)] = z;
            }
        }
    }
    __syncthreads();

    // ---- softmax within the tile: wave w handles query heads w, w + 4, ...; kFusedTile / 64
    //      rows per lane
    constexpr int kRows = kFusedTile / 64;
    for (int hq = wave; hq < G; hq += 4) {
        float zr[kRows];
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            zr[r] = lane + 64 * r < nt ? sh.z[lane + 64 * r][hq] : -INFINITY;
            m = fmaxf(m, zr[r]);
        }
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) m = fmaxf(m, __shfl_xor(m, msk));
        float l = 0.0f;
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            const float pr = lane + 64 * r < nt ? expf(zr[r] - m) : 0.0f;
            if (lane + 64 * r < nt) sh.z[lane + 64 * r][hq] = pr;
            l += pr;
        }
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) l += __shfl_xor(l, msk);
        if (lane == 0) { sh.ml[hq][0] = m; sh.ml[hq][1] = l; }
    }
    __syncthreads();   // also: every key row has been read, the staging area may be reused

    // ---- values: acc[i][k] = sum_t p_t,i * (s_t / 2) * (c_t,k + 64), W[i] = sum_t p_t,i s_t / 2
    stage_tile<kFusedRun>(a.codes_v, a.scales_v, row0, nt, nullptr, a.T, sh.u.t.delta, sh.u.t.scale,
               nullptr);
    float acc[G][8], W[G];
#pragma unroll
    for (int i = 0; i < G; i++) {
        W[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++) acc[i][k] = 0.0f;
    }
    {
        uint2 run = tile_run_base<kFusedRun>(sh.u.t.delta, nt, q, g, sh.tot, sh.excl, a.lb_agg, a.lb_incl,
                                  2 * (size_t)ticket + 1, 2 * (size_t)pairs, tile,
                                  a.lb_ticket + kTicketErr);
        const uint2 *sd = reinterpret_cast<const uint2 *>(sh.u.t.delta) + g;
        const uint16_t *sl = reinterpret_cast<const uint16_t *>(sh.u.t.scale);
        const int jend = min(nt, jl0 + kFusedRun);
#pragma unroll
        for (int i = 0; i < kFusedRun; i++) {
            const int jl = jl0 + i;
            if (jl < jend) {
                run = run_step(run, sd[jl * 16]);
                const float hs = 0.5f * h2f(sl[jl * kGroups + g]);
                float b[8];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    b[k] = (float)((run.x >> (8 * k)) & 0xffu);
                    b[k + 4] = (float)((run.y >> (8 * k)) & 0xffu);
                }
#pragma unroll
                for (int hq = 0; hq < G; hq++) {
                    const float w = sh.z[jl][hq] * hs;
                    W[hq] += w;
#pragma unroll
                    for (int k = 0; k < 8; k++) acc[hq][k] = __builtin_fmaf(w, b[k], acc[hq][k]);
                }
            }
        }
    }
    // remove the +64 offset: acc = sum w (c + 64) - 64 sum w
#pragma unroll
    for (int hq = 0; hq < G; hq++)
#pragma unroll
        for (int k = 0; k < 8; k++) acc[hq][k] = __builtin_fmaf(-64.0f, W[hq], acc[hq][k]);
    // sum over the 4 rows of the wave (lane distance 16, 32), then over the 4 waves in LDS
#pragma unroll
    for (int msk = 16; msk < 64; msk <<= 1)
#pragma unroll
        for (int hq = 0; hq < G; hq++)
#pragma unroll
            for (int k = 0; k < 8; k++) acc[hq][k] += __shfl_xor(acc[hq][k], msk);
    __syncthreads();   // the value rows are no longer read: the staging area becomes red
    if (lane < 16) {
#pragma unroll
        for (int hq = 0; hq < G; hq++)
#pragma unroll
            for (int k = 0; k < 8; k++) sh.u.red[wave][hq][lane][k] = acc[hq][k];
    }
    __syncthreads();
    // partial of query head hq: [m, l, acc in natural dim order]
    float *part = a.part + ((size_t)pair * a.tiles + tile) * G * kPartStride;
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kCodecThreads) {
        const int hq = idx / kHeadDim, r = idx % kHeadDim;   // r = lane slot * 8 + k
        const int l16 = r >> 3, k = r & 7;
        const float v = sh.u.red[0][hq][l16][k] + sh.u.red[1][hq][l16][k] +
                        sh.u.red[2][hq][l16][k] + sh.u.red[3][hq][l16][k];
        part[hq * kPartStride + 2 + 8 * lane_group(l16) + k] = v;
    }
    if (threadIdx.x < G) {
        part[threadIdx.x * kPartStride] = sh.ml[threadIdx.x][0];
        part[threadIdx.x * kPartStride + 1] = sh.ml[threadIdx.x][1];
    }
}

// One block of 256 threads per (layer, query head): the 16 lane groups combine the tiles of the
// pair (online max / sum), merge through LDS, then lane group 0 applies the inverse Hadamard to
// the weighted code sum and divides by the weight sum: o = H acc / (sqrt(128) l).
template <int G>
__global__ __launch_bounds__(kCodecThreads) void k_decode_attend_merge(FusedArgs a)
{
    __shared__ float s_m[16], s_l[16];
    __shared__ float s_acc[16][kHeadDim];
    const int lj = blockIdx.x;
    const int lc = lj / a.Hq, j = lj % a.Hq;
    const int h = j / G, hq = j % G;
    const int pair = lc * a.H + h;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane_group(lane & 15), q = wave * 4 + (lane >> 4);
    float m = -INFINITY, l = 0.0f, acc[8];
#pragma unroll
    for (int k = 0; k < 8; k++) acc[k] = 0.0f;
    for (int t = q; t < a.tiles; t += 16) {
        const float *pp = a.part + (((size_t)pair * a.tiles + t) * G + hq) * kPartStride;
        const float m2 = pp[0], l2 = pp[1];
        float a2[8];
#pragma unroll
        for (int k = 0; k < 8; k++) a2[k] = pp[2 + 8 * g + k];
        const float M = fmaxf(m, m2);
        if (M != -INFINITY) {
            const float f1 = expf(m - M), f2 = expf(m2 - M);
            l = l * f1 + l2 * f2;
#pragma unroll
            for (int k = 0; k < 8; k++) acc[k] = acc[k] * f1 + a2[k] * f2;
            m = M;
        }
    }
    if ((lane & 15) == 0) { s_m[q] = m; s_l[q] = l; }
#pragma unroll
    for (int k = 0; k < 8; k++) s_acc[q][8 * g + k] = acc[k];
    __syncthreads();
    if (q != 0) return;
    float M = -INFINITY;
    for (int r = 0; r < 16; r++) M = fmaxf(M, s_m[r]);
    float L = 0.0f, x[8];
#pragma unroll
    for (int k = 0; k < 8; k++) x[k] = 0.0f;
    if (M != -INFINITY) {
        for (int r = 0; r < 16; r++) {
            const float f = expf(s_m[r] - M);
            L += s_l[r] * f;
#pragma unroll
            for (int k = 0; k < 8; k++) x[k] = __builtin_fmaf(s_acc[r][8 * g + k], f, x[k]);
        }
    }
    hadamard_butterflies(x, g);   // x = group_sign(g) * H acc
    const float f = L > 0.0f ? group_sign(g) * kInvSqrt128 / L : 0.0f;
    float *o = a.out + ((size_t)lc * a.Hq + j) * kHeadDim + 8 * g;
#pragma unroll
    for (int k = 0; k < 8; k++) o[k] = x[k] * f;
}

}  // namespace nq
