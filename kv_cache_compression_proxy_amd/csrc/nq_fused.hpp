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
// 12 tokens per lane group: a 192-token tile's staging (about 35 KB of LDS) lets four blocks
// share a CU, as many as the kernel's 128 VGPRs allow
constexpr int kFusedRun = 12;                  // tokens per lane group
constexpr int kFusedTile = 16 * kFusedRun;     // tokens per block
static_assert(kFusedTile % 64 == 0, "the tile softmax gives every lane kFusedTile / 64 rows");
constexpr int kRotAhead = 2;                  // keys: rotary rows requested this many tokens ahead

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

// One key row in the fused kernel's key layout: lane g holds dims 4g + m (x[m]) and
// 64 + 4g + m (x[4 + m]), m = 0..3, so both members of each RoPE pair (i, i + 64) sit in one
// lane. code: the running code bytes of those dims (offset form c + 64; .x the low dims, .y the
// high ones); s_lo, s_hi: the fp16 scales of their groups g / 2 and 8 + g / 2 in the low
// halves; (cr, sr): the rotary table row of the token's position at dims 4g..4g+3. Returns
// x = group_sign(g) * 2 sqrt(128) times the reconstructed key K = RoPE(H y), H the normalised
// Hadamard transform: the constant factor is left to the caller (the queries carry it).
//
// The Hadamard stages commute, so they run in the order this layout makes cheap: h = 1, 2 on
// the integer codes in packed fp16 (exact, as in decode_row), the scale, h = 4, 8, 16, 32 across
// lanes (partners g ^ 1, g ^ 2, g ^ 4, g ^ 8, the butterflies of hadamard_cross_lane), and
// h = 64 inside the lane fused with the rotation: with (a, b) = the pair before stage 64,
//   k_i      = (a + b) C - (a - b) S = a (C - S) + b (C + S),
//   k_{i+64} = (a - b) C + (a + b) S = a (C + S) - b (C - S).
__device__ __forceinline__ void decode_key_split(int g, uint2 code, uint32_t s_lo, uint32_t s_hi,
                                                 const float cr[4], const float sr[4], float x[8])
{
    uint32_t q0 = __builtin_amdgcn_perm(0x64646464u, code.x, 0x04010400u);   // (c0, c1)
    uint32_t q1 = __builtin_amdgcn_perm(0x64646464u, code.x, 0x04030402u);   // (c2, c3)
    uint32_t q2 = __builtin_amdgcn_perm(0x64646464u, code.y, 0x04010400u);   // (c4, c5)
    uint32_t q3 = __builtin_amdgcn_perm(0x64646464u, code.y, 0x04030402u);   // (c6, c7)
    uint32_t r0, r1, r2, r3;
    asm("v_pk_add_f16 %0, %0, %4\n"
        "v_pk_add_f16 %1, %1, %4\n"
        "v_pk_add_f16 %2, %2, %4\n"
        "v_pk_add_f16 %3, %3, %4\n"
        // h = 1: (a, b) -> (a + b, a - b) inside each register
        "v_pk_add_f16 %0, %0, %0 op_sel:[0,1] op_sel_hi:[0,1] neg_hi:[0,1]\n"
        "v_pk_add_f16 %1, %1, %1 op_sel:[0,1] op_sel_hi:[0,1] neg_hi:[0,1]\n"
        "v_pk_add_f16 %2, %2, %2 op_sel:[0,1] op_sel_hi:[0,1] neg_hi:[0,1]\n"
        "v_pk_add_f16 %3, %3, %3 op_sel:[0,1] op_sel_hi:[0,1] neg_hi:[0,1]\n"
        : "+v"(q0), "+v"(q1), "+v"(q2), "+v"(q3)
        : "s"(0xE440E440u));   // (-1088, -1088)
    // h = 2 within each half: q0 = (y0, y1), q1 = (y2, y3) -> (z0, z2), (z1, z3); same above
    asm("v_pk_add_f16 %0, %4, %5 op_sel:[0,0] op_sel_hi:[0,0] neg_hi:[0,1]\n"
        "v_pk_add_f16 %1, %4, %5 op_sel:[1,1] op_sel_hi:[1,1] neg_hi:[0,1]\n"
        "v_pk_add_f16 %2, %6, %7 op_sel:[0,0] op_sel_hi:[0,0] neg_hi:[0,1]\n"
        "v_pk_add_f16 %3, %6, %7 op_sel:[1,1] op_sel_hi:[1,1] neg_hi:[0,1]\n"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(q0), "v"(q1), "v"(q2), "v"(q3));
    // fp16 sums times the fp16 scale: exact products in fp32 (at most 16 significant bits)
    asm("v_fma_mix_f32 %0, %8, %12, 0 op_sel:[0,0,0] op_sel_hi:[1,1,0]\n"
        "v_fma_mix_f32 %2, %8, %12, 0 op_sel:[1,0,0] op_sel_hi:[1,1,0]\n"
        "v_fma_mix_f32 %1, %9, %12, 0 op_sel:[0,0,0] op_sel_hi:[1,1,0]\n"
        "v_fma_mix_f32 %3, %9, %12, 0 op_sel:[1,0,0] op_sel_hi:[1,1,0]\n"
        "v_fma_mix_f32 %4, %10, %13, 0 op_sel:[0,0,0] op_sel_hi:[1,1,0]\n"
        "v_fma_mix_f32 %6, %10, %13, 0 op_sel:[1,0,0] op_sel_hi:[1,1,0]\n"
        "v_fma_mix_f32 %5, %11, %13, 0 op_sel:[0,0,0] op_sel_hi:[1,1,0]\n"
        "v_fma_mix_f32 %7, %11, %13, 0 op_sel:[1,0,0] op_sel_hi:[1,1,0]\n"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7])
        : "v"(r0), "v"(r1), "v"(r2), "v"(r3), "v"(s_lo), "v"(s_hi));
    hadamard_cross_lane(x, g);   // stages h = 4..32; x = group_sign(g) * (the row before h = 64)
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const float A = cr[m] - sr[m], B = cr[m] + sr[m];
        const float a = x[m], b = x[4 + m];
        x[m] = __builtin_fmaf(b, B, a * A);
        x[4 + m] = __builtin_fmaf(-b, A, a * B);
    }
}

// Two code bytes of a running word (offset form c + 64, picked by the v_perm selector sel) as
// exact fp16 values c: under the exponent byte 0x64 a byte b is the fp16 1024 + b, and one
// packed add of -1088 leaves c (|c| <= 16, so every step is exact).
__device__ __forceinline__ f16x2 codes_f16(uint32_t word, uint32_t sel)
{
    uint32_t h = __builtin_amdgcn_perm(0x64646464u, word, sel);
    asm("v_pk_add_f16 %0, %0, %1" : "+v"(h) : "s"(0xE440E440u));
    return __builtin_bit_cast(f16x2, h);
}

// grid: pairs * tiles blocks (pairs = Lc * H); tickets tile-major over the pairs as in
// k_decode, layer-fastest. Look-back slots: 2 * ticket + tensor (K = 0, V = 1).
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
    // ticket slot lc + Lc h: the kv heads of a layer (same kept positions, same rotary rows)
    // share a ticket class and so an XCD and its L2; `pair` is the storage index lc * H + h
    const int tp = ticket % pairs;
    const int Lcf = pairs / a.H;
    const int lc = tp % Lcf, h = tp / Lcf;
    const int pair = lc * a.H + h;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane_group(lane & 15), q = wave * 4 + (lane >> 4);
    const int n_keep = a.n_keep;
    const int t0 = tile * kFusedTile;
    const int nt = min(kFusedTile, n_keep - t0);
    const int jl0 = q * kFusedRun;                     // this lane group's first tile row
    const size_t row0 = (size_t)pair * n_keep + t0;    // chain row of the tile's first token

    // queries of this kv head in the key layout of decode_key_split (this lane's dims 4g..4g+3
    // and 64+4g..64+4g+3), times group_sign(g) / 256: the keys come out times
    // group_sign(g) * 2 sqrt(128), so q . x is the true score q . K / sqrt(128) (exact scaling)
    float qv[G][8];
    {
        const float f = group_sign(g) * (1.0f / 256.0f);
#pragma unroll
        for (int i = 0; i < G; i++) {
            const uint16_t *qp = a.Q + ((size_t)lc * a.Hq + h * G + i) * kHeadDim + 4 * g;
            const uint2 lo = *reinterpret_cast<const uint2 *>(qp);
            const uint2 hi = *reinterpret_cast<const uint2 *>(qp + 64);
            const uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                qv[i][2 * k] = h2f(w[k] & 0xffffu) * f;
                qv[i][2 * k + 1] = h2f(w[k] >> 16) * f;
            }
        }
    }

    // ---- keys: scores z[t][i] of the tile
    stage_tile<kFusedRun>(a.codes_k, a.scales_k, row0, nt, a.positions + (size_t)lc * n_keep + t0, a.T,
               sh.u.t.delta, sh.u.t.scale, sh.pos);
    {
        uint2 run = tile_run_base<kFusedRun, true>(sh.u.t.delta, nt, q, g, sh.tot, sh.excl,
                                                   a.lb_agg, a.lb_incl, 2 * (size_t)ticket,
                                                   2 * (size_t)pairs, tile,
                                                   a.lb_ticket + kTicketErr);
        const uint16_t *sl = reinterpret_cast<const uint16_t *>(sh.u.t.scale);
        // the rotary table through buffer resources: a row is 256 bytes at 32-bit offset
        // p * 256 (positions are below 2^23), the lane's 16 bytes at 16 g within it
        const __amdgpu_buffer_rsrc_t rcos = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.rope_cos), 0, a.T * 256, kBufWord3);
        const __amdgpu_buffer_rsrc_t rsin = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(a.rope_sin), 0, a.T * 256, kBufWord3);
        const uint32_t lane_rot = 16u * (uint32_t)g;
        auto load_rot = [&](int jrow, float c[4], float sn[4]) {
            const uint32_t o = ((uint32_t)sh.pos[jrow] << 8) | lane_rot;
            const u32x4 vc = __builtin_amdgcn_raw_buffer_load_b128(rcos, o, 0, 0);
            const u32x4 vs = __builtin_amdgcn_raw_buffer_load_b128(rsin, o, 0, 0);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                c[k] = __uint_as_float(vc[k]);
                sn[k] = __uint_as_float(vs[k]);
            }
        };
        // Every lane group walks kFusedRun rows. Rows past the tile's end (only in a chain's
        // last, partial tile) are computed on the last row's data and not reported, so the loop
        // has no branch around a load: the rotary rows of token i + kRotAhead are requested while
        // token i is computed, with exact waits.
        float rc[kRotAhead + 1][4], rs[kRotAhead + 1][4];
#pragma unroll
        for (int i = 0; i < kRotAhead; i++) load_rot(min(jl0 + i, nt - 1), rc[i], rs[i]);
#pragma unroll
        for (int i = 0; i < kFusedRun; i++) {
            const int jl = jl0 + i, jr = min(jl, nt - 1), cur = i % (kRotAhead + 1);
            if (i + kRotAhead < kFusedRun) {
                const int nx = (i + kRotAhead) % (kRotAhead + 1);
                load_rot(min(jl + kRotAhead, nt - 1), rc[nx], rs[nx]);
            }
            run = run_step(run, lane_delta<true>(sh.u.t.delta, jr, g));
            const uint32_t s_lo = sl[jr * kGroups + (g >> 1)];
            const uint32_t s_hi = sl[jr * kGroups + 8 + (g >> 1)];
            float x[8];
            decode_key_split(g, run, s_lo, s_hi, rc[cur], rs[cur], x);
            float d[G];
#pragma unroll
            for (int hq = 0; hq < G; hq++) {
                d[hq] = qv[hq][0] * x[0];
#pragma unroll
                for (int k = 1; k < 8; k++) d[hq] = __builtin_fmaf(qv[hq][k], x[k], d[hq]);
            }
            const float z = row_sums<G>(d, lane & 15);
            if (jl < nt && row_sum_reporter<G>(lane & 15)) sh.z[jl][row_sum_index<G>(lane & 15)] = z;
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
            sh.z[lane + 64 * r][hq] = pr;   // 0 past the tile's end
            l += pr;
        }
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) l += __shfl_xor(l, msk);
        if (lane == 0) { sh.ml[hq][0] = m; sh.ml[hq][1] = l; }
    }
    __syncthreads();   // also: every key row has been read, the staging area may be reused

    // ---- values: acc[i][k] = sum_t p_t,i * s_t * c_t,k (twice the dequantised sum; the merge
    //      halves it), on the codes themselves: each code is an exact fp16, and one
    //      v_fma_mix_f32 per (head, dim) multiplies it by the fp32 weight and adds to the fp32
    //      accumulator with one rounding
    stage_tile<kFusedRun>(a.codes_v, a.scales_v, row0, nt, nullptr, a.T, sh.u.t.delta, sh.u.t.scale,
               nullptr);
    float acc[G][8];
#pragma unroll
    for (int i = 0; i < G; i++)
#pragma unroll
        for (int k = 0; k < 8; k++) acc[i][k] = 0.0f;
    {
        uint2 run = tile_run_base<kFusedRun>(sh.u.t.delta, nt, q, g, sh.tot, sh.excl, a.lb_agg, a.lb_incl,
                                  2 * (size_t)ticket + 1, 2 * (size_t)pairs, tile,
                                  a.lb_ticket + kTicketErr);
        const uint2 *sd = reinterpret_cast<const uint2 *>(sh.u.t.delta) + g;
        const uint16_t *sl = reinterpret_cast<const uint16_t *>(sh.u.t.scale);
        // rows past the tile's end (as in the key loop) read the last row and carry weight 0
#pragma unroll
        for (int i = 0; i < kFusedRun; i++) {
            const int jl = jl0 + i, jr = min(jl, nt - 1);
            run = run_step(run, sd[jr * 16]);
            const float hs = h2f(sl[jr * kGroups + g]);   // s; the 1/2 is applied in the merge
            const f16x2 c01 = codes_f16(run.x, 0x04010400u), c23 = codes_f16(run.x, 0x04030402u);
            const f16x2 c45 = codes_f16(run.y, 0x04010400u), c67 = codes_f16(run.y, 0x04030402u);
            const float c[8] = {(float)c01.x, (float)c01.y, (float)c23.x, (float)c23.y,
                                (float)c45.x, (float)c45.y, (float)c67.x, (float)c67.y};
#pragma unroll
            for (int hq = 0; hq < G; hq++) {
                const float w = sh.z[jl][hq] * hs;
#pragma unroll
                for (int k = 0; k < 8; k++) acc[hq][k] = __builtin_fmaf(c[k], w, acc[hq][k]);
            }
        }
    }
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
    // the tiles summed p * s * c: the 1/2 of s / 2 and the 1/sqrt(128) of H (exact scalings)
    const float f = L > 0.0f ? group_sign(g) * (0.5f * kInvSqrt128) / L : 0.0f;
    float *o = a.out + ((size_t)lc * a.Hq + j) * kHeadDim + 8 * g;
#pragma unroll
    for (int k = 0; k < 8; k++) o[k] = x[k] * f;
}

}  // namespace nq
