// Encode and decode kernels: RoPE removal/restore, 128-point Hadamard rotation, per-group fp16
// scales, E8 nearest point, delta coding along the kept tokens and its running-sum inverse.
//
// Method: "Como comprimir o KV cache do seu LLM em 33x sem treino", section "Como funciona",
// steps 3-6 (RoPE removal, Hadamard rotation, E8 quantization of 8-float groups, delta coding);
// "NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破", sections "E8格点量化" and
// "技术实现细节" (keys 3-bit / values 2-bit; RoPE restored after quantization).
//
// Work decomposition (both directions). A chain is one (compressed layer, tensor K|V, kv head):
// the delta code runs along its kept tokens. A 256-thread workgroup owns a tile of 16*R
// consecutive kept tokens of one chain; each of its 16 lane groups walks R consecutive tokens
// in order, so the previous token's code is still in registers when the next token is coded.
#pragma once

#include "nq_common.hpp"

namespace nq {

constexpr int kCodecThreads = 256;
constexpr int kCodecRun = 16;                          // encode: tokens walked per lane group
constexpr int kCodecTile = 16 * kCodecRun;             // encode: tokens per workgroup tile
static_assert(kCodecTile == kCodecThreads, "encode stages one position per thread");
constexpr int kDecRun = 8;                             // decode: tokens per lane group
constexpr int kDecTile = 16 * kDecRun;                 // decode: tokens per workgroup tile

struct CodecArgs {
    const uint16_t *K, *V;         // fp16 [L][H][T][128]
    const int32_t *positions;      // [Lc][n_keep]
    const float *rope_cos, *rope_sin;  // [T][64]
    int8_t *codes_k, *codes_v;     // [Lc][H][n_keep][128]
    uint16_t *scales_k, *scales_v; // fp16 bits [Lc][H][n_keep][16]
    void *out_k, *out_v;           // decode outputs [Lc][H][n_keep][128]
    uint32_t *lb_agg, *lb_incl;    // decode look-back words [tiles][4][16 lanes] (see below)
    uint32_t *lb_ticket;           // kTicketWords: tile ticket counters, spin-limit error flag
    int32_t H, T, layer_begin, n_keep;
    int32_t tiles_per_chain;       // encode tiles (kCodecTile tokens) per chain
    int32_t dec_tiles_per_chain;   // decode tiles (kDecTile tokens) per chain
    float rho_k, rho_v;
    float rho_inv_k, rho_inv_v;    // fp32 nearest to 1/rho
    float rho_inv_lo_k, rho_inv_lo_v;   // fp32 nearest to 1/rho - rho_inv
    int32_t out_f32;
};

// Split-half rotary table: C[p][i] = fp32(cos(p * theta_i)), S[p][i] = fp32(sin(p * theta_i)),
// angles in fp64 from theta_i = base^(-i/64) computed on the host.
struct RopeTheta {
    double v[64];
};

__global__ __launch_bounds__(256) void k_rope_table(RopeTheta th, int T, float *__restrict__ C,
                                                   float *__restrict__ S)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * 64) return;
    const int i = (int)(idx & 63);
    const double phi = (double)(idx >> 6) * th.v[i];
    double sv, cv;
    sincos(phi, &sv, &cv);
    C[idx] = (float)cv;
    S[idx] = (float)sv;
}

// Which 8-dim group of a 128-dim row a lane holds: lane l of a 16-lane row holds dims
// 8 * lane_group(l) + j. The order (0 1 2 3 7 6 5 4 8 9 10 11 15 14 13 12) makes every
// butterfly partner one DPP step away: groups G and G ^ 1, G ^ 2, G ^ 4, G ^ 8 sit in lanes
// l ^ 1, l ^ 2, l ^ 7, l ^ 8 (quad_perm, quad_perm, row_half_mirror, row_ror:8). Loads and
// stores of a row still cover it whole with 16 lanes, so they stay coalesced.
__device__ __forceinline__ int lane_group(int l) { return l ^ ((l & 4) ? 3 : 0); }

// Hadamard butterflies of a row held as 8 values per lane (dims 8g + j, g = lane_group of the
// lane), in the order h = 1, 2, 4 (inside the lane) then 8, 16, 32, 64 (partner groups g ^ 1,
// g ^ 2, g ^ 4, g ^ 8); pair (a, b) -> (a + b, a - b). The normalisation by 1/sqrt(128) is left
// to the caller.
//
// Cross-lane stages keep a per-lane sign: each lane computes self + sgn * partner with one
// fused DPP multiply-add (sgn = +1 in the lower group of a pair, -1 in the upper one), so the
// upper lane holds -(a - b). By induction every lane ends holding group_sign(g) times the true
// value, group_sign(g) = (-1)^popcount(g); each value is one correctly rounded add or subtract
// of the same operands as in the sequential order, so |values| match it bit for bit.
__device__ __forceinline__ float group_sign(int g) { return (__popc(g & 15) & 1) ? -1.0f : 1.0f; }

// in-lane stages from h = H0 on
template <int H0 = 1>
__device__ __forceinline__ void hadamard_in_lane(float x[8])
{
#pragma unroll
    for (int h = H0; h < 8; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            if (!(j & h)) {
                const float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
        }
    }
}

__device__ __forceinline__ void hadamard_cross_lane(float x[8], int g)
{
    const float s1 = (g & 1) ? -1.0f : 1.0f, s2 = (g & 2) ? -1.0f : 1.0f;
    const float s4 = (g & 4) ? -1.0f : 1.0f, s8 = (g & 8) ? -1.0f : 1.0f;
    // x[j] += s * x[j] of the partner lane: v_fmac_f32 with a DPP-routed first operand (the
    // compiler does not fuse a DPP move into fmac by itself). s_nop 1 gives the two wait states
    // a DPP read needs after a VALU write of the same register.
#define NQ_FMAC_DPP(CTRL)                                                                      \
    "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"             \
    "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"             \
    "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"             \
    "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"             \
    "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"             \
    "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"             \
    "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"             \
    "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
#define NQ_X8 "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])
    asm("s_nop 1\n" NQ_FMAC_DPP("quad_perm:[1,0,3,2]") : NQ_X8 : "v"(s1));
    asm("s_nop 1\n" NQ_FMAC_DPP("quad_perm:[2,3,0,1]") : NQ_X8 : "v"(s2));
    asm("s_nop 1\n" NQ_FMAC_DPP("row_half_mirror") : NQ_X8 : "v"(s4));
    asm("s_nop 1\n" NQ_FMAC_DPP("row_ror:8") : NQ_X8 : "v"(s8));
#undef NQ_X8
#undef NQ_FMAC_DPP
}

__device__ __forceinline__ void hadamard_butterflies(float x[8], int g)
{
    hadamard_in_lane(x);
    hadamard_cross_lane(x, g);
}

// x[k] += sg * u[k] of the partner lane g ^ 8 (row_ror:8), rounded once: the cross term of a
// RoPE pair (i, i + 64), whose two lanes hold the same (C, S) so that each lane's own product
// u = x * S is the one its partner needs. One v_fmac_f32_dpp per value (written out: the
// compiler splits a DPP move from the multiply-add); s_nop 1 as in hadamard_cross_lane.
__device__ __forceinline__ void rope_cross(float x[8], const float u[8], float sg)
{
    asm("s_nop 1\n"
        "v_fmac_f32_dpp %0, %8, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %1, %9, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %2, %10, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %3, %11, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %4, %12, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %5, %13, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %6, %14, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        "v_fmac_f32_dpp %7, %15, %16 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
          "+v"(x[7])
        : "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(u[4]), "v"(u[5]), "v"(u[6]),
          "v"(u[7]), "v"(sg));
}

// Nearest E8 point of u (8 floats); returns the codes c = 2y as bytes c + 64 in two dwords.
// E8 = D8 u (D8 + 1/2) (Conway & Sloane). With f = rint(u), e = u - f, a = |e|:
//   coset D8:       squared distance sum(a^2), plus (1 - 2 max a) if sum(f) is odd, where the
//                   coordinate of largest a is re-rounded the other way;
//   coset D8 + 1/2: nearest half-integers f + sign(e)/2 at distance (1/2 - a) each, sum
//                   (2 - sum(a) + sum(a^2)), plus 2 min a if sum(f) - #(e < 0) is odd, where
//                   the coordinate of smallest a moves to the other neighbouring half-integer.
// The nearer coset wins (D8 on ties). Arg-max/min run on one key per coordinate, |e| with its
// 3 low bits replaced by the index; the index can only decide between coordinates whose
// errors differ by a few ulps, where the two candidate points are at (nearly) equal distance
// (a near-tie).
// Rounding: t = u + M with M = 1.5 * 2^23 + 32 lands where the fp32 spacing is 1, so the add
// rounds u to an integer with ties to even (M is even: the tie choice is rint's), t = rint(u) + M
// exactly for |u| < 2^21, and t's low mantissa byte is rint(u) + 32. g = M - t = -rint(u) and
// e = u + g are exact, with e = +0 whenever u is an integer (-0 included).
// Byte work: B = f + 32 per coordinate, gathered from the t words; N = [e < 0] per byte
// (gathered sign bytes); the D8 + 1/2 points are floor(u) + 1/2 = f - N + 1/2; parities come
// from byte sums / popcounts; the codes c + 64 are 2B (D8) or 2B + 1 (D8 + 1/2).
__device__ __forceinline__ void e8_nearest_code(const float u[8], uint32_t &w0, uint32_t &w1)
{
    constexpr float kMagic = 12582944.0f;   // 1.5 * 2^23 + 32
    float e[8];
    uint32_t tb[8];
    uint32_t kmax = 0u, kmin = 0xffffffffu;
    float Sa = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float t = u[i] + kMagic;
        e[i] = u[i] + (kMagic - t);
        tb[i] = __float_as_uint(t);
        // key: (eb & 0x7ffffff8) | i
        const uint32_t key = (uint32_t)__builtin_amdgcn_bitop3_b32(__float_as_uint(e[i]),
                                                                   0x7ffffff8u, (uint32_t)i, 0xEA);
        kmax = kmax > key ? kmax : key;
        kmin = kmin < key ? kmin : key;
        Sa += __builtin_fabsf(e[i]);
    }
    // B = f + 32 per byte: byte 0 of each t word
    uint32_t b0 = __builtin_amdgcn_perm(tb[1], tb[0], 0x0c0c0400u) |
                  __builtin_amdgcn_perm(tb[3], tb[2], 0x04000c0cu);
    uint32_t b1 = __builtin_amdgcn_perm(tb[5], tb[4], 0x0c0c0400u) |
                  __builtin_amdgcn_perm(tb[7], tb[6], 0x04000c0cu);
    // sign bytes of e (byte 3 of each float) gathered into two dwords, then [e < 0] per byte
    const uint32_t g0 = __builtin_amdgcn_perm(__float_as_uint(e[1]), __float_as_uint(e[0]), 0x0c0c0703u) |
                        __builtin_amdgcn_perm(__float_as_uint(e[3]), __float_as_uint(e[2]), 0x07030c0cu);
    const uint32_t g1 = __builtin_amdgcn_perm(__float_as_uint(e[5]), __float_as_uint(e[4]), 0x0c0c0703u) |
                        __builtin_amdgcn_perm(__float_as_uint(e[7]), __float_as_uint(e[6]), 0x07030c0cu);
    const uint32_t n0 = (g0 >> 7) & 0x01010101u, n1 = (g1 >> 7) & 0x01010101u;
    // sum of bytes = sum(f) + 256: bit 0 is the parity of sum(f)
    const uint32_t sb = __builtin_amdgcn_udot4(b0, 0x01010101u, __builtin_amdgcn_udot4(b1, 0x01010101u, 0u, false), false);
    const int P0 = (int)(sb & 1u);
    const int P1 = P0 ^ (int)((__popc(n0) + __popc(n1)) & 1u);
    const float amax = __uint_as_float(kmax & ~7u);
    const float amin = __uint_as_float(kmin & ~7u);
    // d1 - d0 = (2 - sum a + [P1] 2 min a) - [P0] (1 - 2 max a); sum(a^2) cancels
    float dd = 2.0f - Sa;
    if (P1) dd = __builtin_fmaf(2.0f, amin, dd);
    if (P0) dd = __builtin_fmaf(2.0f, amax, dd - 1.0f);
    const bool half = dd < 0.0f;
    const int jf = (int)((half ? kmin : kmax) & 7u);
    const int par = half ? P1 : P0;
    if (half) {
        b0 -= n0;   // floor(u) + 32 per byte (every byte >= 16: no borrow)
        b1 -= n1;
    }
    if (par) {
        // D8: re-round toward u (+sign(e)); D8 + 1/2: move away from u (-sign(e))
        const uint32_t neg = ((jf < 4 ? n0 : n1) >> (8 * (jf & 3))) & 1u;
        int d = neg ? -1 : 1;
        if (half) d = -d;
        const uint32_t add = (uint32_t)d << (8 * (jf & 3));
        if (jf < 4) b0 += add; else b1 += add;
    }
    // c + 64 = 2 (y + 32): 2B on D8, 2B + 1 on D8 + 1/2 (bytes stay below 128: no carry)
    const uint32_t hb = half ? 0x01010101u : 0u;
    w0 = (b0 << 1) | hb;
    w1 = (b1 << 1) | hb;
}

// The raw inputs of one kept token for this lane: its 8 fp16 dims and, for keys, the rotary
// table rows of its position.
struct TokenIn {
    u32x4 v;
    float c[8], s[8];
};

// this lane's 8 fp16 dims of the row at position p (each K/V row is read once: streamed)
__device__ __forceinline__ u32x4 load_row(const uint16_t *__restrict__ X, int p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(X + (size_t)p * kHeadDim));
}

__device__ __forceinline__ void load_rope(const float *__restrict__ rope_cos,
                                          const float *__restrict__ rope_sin, int p, int g,
                                          TokenIn &t)
{
    load_f32x8(rope_cos + (size_t)p * 64 + 8 * (g & 7), t.c);
    load_f32x8(rope_sin + (size_t)p * 64 + 8 * (g & 7), t.s);
}

template <bool IS_KEY>
__device__ __forceinline__ void load_token(const float *__restrict__ rope_cos,
                                           const float *__restrict__ rope_sin,
                                           const uint16_t *__restrict__ X, int p, int g,
                                           TokenIn &t)
{
    t.v = load_row(X, p);
    if (IS_KEY) load_rope(rope_cos, rope_sin, p, g, t);
}

// One chain's encode inputs and code output as buffer resources: a token's row and rotary rows
// sit at 32-bit byte offsets p * 256 (+ the lane's part) from the resource bases, which costs
// one shift per token instead of 64-bit address arithmetic for every pointer. Offsets past a
// resource's size read zeros and drop writes; every offset used here is in range.
constexpr int kBufWord3 = 0x00020000;   // raw 32-bit dword access, the gfx9 family's word 3
constexpr int kBufNt = 2;               // cache policy: non-temporal (streamed once)

struct ChainBuf {
    __amdgpu_buffer_rsrc_t x, cos, sin, codes;
};

template <bool IS_KEY>
__device__ __forceinline__ void load_token_buf(const ChainBuf &b, int p, int g, TokenIn &t)
{
    const uint32_t o = (uint32_t)p << 8;   // 128 fp16 dims or 64 fp32 rotary values per token
    t.v = __builtin_amdgcn_raw_buffer_load_b128(b.x, o | (uint32_t)(16 * g), 0, kBufNt);
    if (IS_KEY) {
        const uint32_t r = o | (uint32_t)(32 * (g & 7));
        const u32x4 c0 = __builtin_amdgcn_raw_buffer_load_b128(b.cos, r, 0, 0);
        const u32x4 c1 = __builtin_amdgcn_raw_buffer_load_b128(b.cos, r + 16, 0, 0);
        const u32x4 s0 = __builtin_amdgcn_raw_buffer_load_b128(b.sin, r, 0, 0);
        const u32x4 s1 = __builtin_amdgcn_raw_buffer_load_b128(b.sin, r + 16, 0, 0);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            t.c[k] = __uint_as_float(c0[k]);
            t.c[4 + k] = __uint_as_float(c1[k]);
            t.s[k] = __uint_as_float(s0[k]);
            t.s[4 + k] = __uint_as_float(s1[k]);
        }
    }
}

// The codec front end for one kept token loaded into t: the fp16 row, for keys the rotary
// embedding removed at the token's position, then the Hadamard butterflies. x = group_sign(g)
// times the unnormalised rotated row.
template <bool IS_KEY>
__device__ __forceinline__ void front_end(const TokenIn &t, int g, float x[8])
{
    const uint32_t w[4] = {t.v.x, t.v.y, t.v.z, t.v.w};
    if (!IS_KEY) {
        // stage h = 1 straight from the fp16 pairs: v_fma_mix_f32 a * 1 + (+-b) converts both
        // halves exactly and rounds the sum once, as the fp32 add of the converted values
#pragma unroll
        for (int k = 0; k < 4; k++) {
            asm("v_fma_mix_f32 %0, %2, 1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]\n"
                "v_fma_mix_f32 %1, %2, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
                : "=&v"(x[2 * k]), "=v"(x[2 * k + 1])
                : "v"(w[k]));
        }
        hadamard_in_lane<2>(x);
        hadamard_cross_lane(x, g);
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
        x[2 * k] = h2f(w[k] & 0xffffu);
        x[2 * k + 1] = h2f(w[k] >> 16);
    }
    {
        // RoPE removal, split-half pairs (i, i + 64) = lanes (g, g ^ 8):
        // x_i = a*C + b*S, x_{i+64} = b*C - a*S with (a, b) = (k_i, k_{i+64}). Both lanes of a
        // pair hold the same (C, S), so each lane's own product x*S is the one its partner needs:
        // it is formed in place and crosses over inside the final multiply-add.
        const float sg = g >= 8 ? -1.0f : 1.0f;
        float u[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            u[k] = x[k] * t.s[k];   // the partner's t2
            x[k] = x[k] * t.c[k];   // t1
        }
        rope_cross(x, u, sg);       // t1 +- t2, rounded once
    }
    hadamard_butterflies(x, g);
}

// Encodes one loaded token for this lane's 8 dims. Returns the absolute code bytes (offset
// +64) and the fp16 scale bits of this lane's group.
//
// Both divisions (amax / rho for the scale, xn / s for the lattice input) are a product with a
// two-part reciprocal h + l of the divisor d, h within an ulp of 1/d and l = (1 - d h) h (the
// bracket is exact in one fma): a / d is formed as fma(a, h, a * l), one rounded product and
// one fused multiply-add. h + l is within 2^-45 (relative) of 1/d, and with an 11-bit divisor
// significand (a binary16 s, rho <= 7) the quotient of any fp32 lies at least 2^-36 (relative)
// from a midpoint between fp32 neighbours, so the single rounding gives the correctly rounded
// quotient -- whenever a * l does not underflow, i.e. for every quotient above 2^-100; below,
// the result is within one ulp of it. Checked on the host: every fp32 significand against
// every binary16 significand and both candidate values of h, and every fp32 amax for the scale.
template <bool IS_KEY>
__device__ __forceinline__ uint2 encode_token(const TokenIn &t, int g, float rho, float rho_inv,
                                              float rho_inv_lo, uint32_t &s16)
{
    float x[8];
    front_end<IS_KEY>(t, g, x);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) amax = fmaxf(amax, __builtin_fabsf(x[k]));
    // the normalised row is x * fp32(1/sqrt(128)); rounding is monotone, so the group's
    // largest normalised magnitude is the rounded product of the largest raw one
    amax = amax * kInvSqrt128;
    // amax / rho correctly rounded (1/rho in two parts from the host); amax = 0 gives s = 0
    const float q = __builtin_fmaf(amax, rho_inv, amax * rho_inv_lo);
    // s = the smallest fp16 >= q, saturating at 65504. In the normal fp16 range, rounding q's
    // fp32 bits up at bit 13 gives s's fp32 bits (a mantissa carry moves into the exponent);
    // below 2^-14 (and for q = 0) fp16 steps are 2^-24 apart: s = ceil(q * 2^24) * 2^-24.
    uint32_t sb32 = min((__float_as_uint(q) + 0x1fffu) & 0xffffe000u, 0x477fe000u);
    s16 = (sb32 >> 13) - 0x1c000u;
    if (__builtin_expect(q < 0x1p-14f, 0)) {
        const float m = __builtin_ceilf(q * 0x1p24f);
        s16 = (uint32_t)m;
        sb32 = __float_as_uint(m * 0x1p-24f);
    }
    // u = xn / s, xn = the normalised rotated value (x times the lane sign and 1/sqrt(128),
    // rounded once), with h from v_rcp_f32 (within one ulp): the lattice step sees the
    // oracle's u (equal above 2^-100, where a one-ulp step moves no lattice distance by more
    // than 2^-99). A zero scale (an all-zero group, or one whose a / rho rounds to 0) takes
    // h = l = 0, which gives u = 0 as the oracle's.
    const float sf = __uint_as_float(sb32);
    const float rh = s16 ? __builtin_amdgcn_rcpf(sf) : 0.0f;
    const float rl = __builtin_fmaf(-sf, rh, 1.0f) * rh;
    const float cs = kInvSqrt128 * group_sign(g);   // exact: +-fp32(1/sqrt(128))
    float u[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const float xn = x[k] * cs;
        u[k] = __builtin_fmaf(xn, rh, xn * rl);
    }
    if (s16 == 0x7bffu) {   // saturated scale: |x / s| may exceed rho
#pragma unroll
        for (int k = 0; k < 8; k++) u[k] = fminf(fmaxf(u[k], -rho), rho);
    }
    uint2 c;
    e8_nearest_code(u, c.x, c.y);
    return c;
}

// Delta bytes (two's complement) from two offset-64 codes: per byte (a + 128) - b stays in
// [96, 160] for codes within +-16, so no carry or borrow crosses a byte; xor 0x80 recentres.
__device__ __forceinline__ uint2 delta_code(uint2 cur, uint2 prev)
{
    return make_uint2(((cur.x + 0x80808080u) - prev.x) ^ 0x80808080u,
                      ((cur.y + 0x80808080u) - prev.y) ^ 0x80808080u);
}

struct EncodeShared {
    uint2 last[17][16];                         // predecessor codes of each lane group
    uint4 scales[kCodecTile * kGroups * 2 / 16];   // the tile's fp16 scales, stored coalesced
    int32_t pos[kCodecTile + 1];                // positions of the tile and its predecessor
};

template <bool IS_KEY>
__device__ void encode_tile(const CodecArgs &a, int lc, int h, int tile, EncodeShared &sh)
{
    auto &s_last = sh.last;
    uint16_t *s_sc = reinterpret_cast<uint16_t *>(sh.scales);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane_group(lane & 15), q = wave * 4 + (lane >> 4);
    const int n_keep = a.n_keep;
    const size_t chain = (size_t)lc * a.H + h;
    ChainBuf b;
    b.x = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(IS_KEY ? a.K : a.V) +
            ((size_t)(a.layer_begin + lc) * a.H + h) * (size_t)a.T * kHeadDim,
        0, a.T * 256, kBufWord3);
    b.cos = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.rope_cos), 0, a.T * 256,
                                              kBufWord3);
    b.sin = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.rope_sin), 0, a.T * 256,
                                              kBufWord3);
    b.codes = __builtin_amdgcn_make_buffer_rsrc(
        (IS_KEY ? a.codes_k : a.codes_v) + chain * (size_t)n_keep * kHeadDim, 0, n_keep * 128,
        kBufWord3);
    const uint32_t lane_code = 8 * g;   // this lane's 8 code bytes of a 128-byte row
    const int t0 = tile * kCodecTile;
    const float rho = IS_KEY ? a.rho_k : a.rho_v;
    const float rho_inv = IS_KEY ? a.rho_inv_k : a.rho_inv_v;
    const float rho_inv_lo = IS_KEY ? a.rho_inv_lo_k : a.rho_inv_lo_v;
    const uint2 zero = make_uint2(0x40404040u, 0x40404040u);   // code 0 in offset form

    // positions of tokens t0 - 1 .. t0 + kCodecTile - 1 (clamped into the cache) to LDS
    {
        const int32_t *pos = a.positions + (size_t)lc * n_keep;
        const int jj = t0 - 1 + (int)threadIdx.x;
        if (jj >= 0 && jj < n_keep) sh.pos[threadIdx.x] = min(max(pos[jj], 0), a.T - 1);
        if (threadIdx.x == 0 && t0 + kCodecTile - 1 < n_keep)
            sh.pos[kCodecTile] = min(max(pos[t0 + kCodecTile - 1], 0), a.T - 1);
    }
    __syncthreads();
    const int32_t *s_pos = sh.pos + 1;   // s_pos[j - t0]

    // the tile's predecessor token, coded (not stored) by lane group 0
    if (q == 0) {
        uint2 hc = zero;
        if (t0 > 0) {
            uint32_t s16;
            TokenIn t;
            load_token_buf<IS_KEY>(b, s_pos[-1], g, t);
            hc = encode_token<IS_KEY>(t, g, rho, rho_inv, rho_inv_lo, s16);
        }
        s_last[0][g] = hc;
    }
    const int j0 = tile * kCodecTile + q * kCodecRun;
    uint2 first = zero, prev = zero;
    for (int i = 0; i < kCodecRun; i++) {
        const int j = j0 + i;
        if (j < n_keep) {
            TokenIn t;
            load_token_buf<IS_KEY>(b, s_pos[j - t0], g, t);
            uint32_t s16;
            const uint2 c = encode_token<IS_KEY>(t, g, rho, rho_inv, rho_inv_lo, s16);
            s_sc[(j - t0) * kGroups + g] = (uint16_t)s16;
            if (i == 0) {
                first = c;
            } else {
                const uint2 d = delta_code(c, prev);
                __builtin_amdgcn_raw_buffer_store_b64((u32x2){d.x, d.y}, b.codes,
                                                      (uint32_t)j * 128 + lane_code, 0, kBufNt);
            }
            prev = c;
        }
    }
    s_last[q + 1][g] = prev;
    __syncthreads();
    if (j0 < n_keep) {
        const uint2 d = delta_code(first, s_last[q][g]);
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){d.x, d.y}, b.codes,
                                              (uint32_t)j0 * 128 + lane_code, 0, kBufNt);
    }
    // the tile's scales: 32 bytes per token, written as 16-byte chunks past the caches
    const int nt = min(kCodecTile, n_keep - t0);
    uint4 *sc = reinterpret_cast<uint4 *>((IS_KEY ? a.scales_k : a.scales_v) +
                                          (chain * (size_t)n_keep + t0) * kGroups);
    for (int c = threadIdx.x; c < 2 * nt; c += kCodecThreads) {
        const uint4 v = sh.scales[c];
        const u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(sc + c));
    }
}

// grid: Lc * 2 * H * tiles_per_chain blocks in XCD-aware order: every head, tensor and layer of
// one tile index before the next tile index, so the blocks reading rotary rows of nearby
// positions share an L2
__global__ __launch_bounds__(kCodecThreads) void k_encode(CodecArgs a)
{
    const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t Lc = gridDim.x / (2u * a.H * a.tiles_per_chain);
    const int h = id % a.H;
    uint32_t r = id / a.H;
    const int tensor = r & 1;
    r >>= 1;
    const int lc = r % Lc;
    const int tile = r / Lc;
    __shared__ EncodeShared sh;
    if (tensor == 0)
        encode_tile<true>(a, lc, h, tile, sh);
    else
        encode_tile<false>(a, lc, h, tile, sh);
}

// ---------------------------------------------------------------------------------------------
// Decode. Each tile needs the running sum of all earlier deltas of its chain; tiles publish
// their own byte-wise sum and then their inclusive prefix (single-pass chained scan with
// decoupled look-back). Tiles take tickets from atomic counters in launch order
// (take_ticket), so every tile a tile waits for has already started and makes progress.
//
// Publication needs no memory fence: a tile's 128-byte value is written as 64 words of
// (tag << 16 | 16 payload bits) with relaxed device-scope atomic stores, tag 1 for the tile
// sum and 2 for the inclusive prefix, into buffers zeroed before the launch. A reader takes a
// value only once all 64 of its words carry the expected tag, so it can never combine a
// half-written value, whatever order the stores become visible in. (A release/acquire pair
// would write back and invalidate the whole L2 of the XCD on every publication.)
// ---------------------------------------------------------------------------------------------
constexpr uint32_t kSpinLimit = 1u << 26;

// Ticket words: kTicketClasses counters, counter k at word k * kTicketStride (one 128-byte
// line each), and the spin-limit error flag at word 1.
constexpr int kTicketClasses = 8;
constexpr int kTicketStride = 32;
constexpr int kTicketWords = kTicketClasses * kTicketStride;
constexpr int kTicketErr = 1;

// Zeroes n words and, when ticket is not null, the kTicketWords ticket words (a launch of at
// least kTicketWords threads).
// words must be 16-byte aligned: each thread clears 4 words with one 16-byte store (the last
// one clears what is left of n word by word).
__global__ void k_decode_reset(uint32_t *words, int64_t n, uint32_t *ticket)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t w = 4 * i;
    if (w + 4 <= n)
        *reinterpret_cast<uint4 *>(words + w) = make_uint4(0u, 0u, 0u, 0u);
    else
        for (int64_t k = w; k < n; k++) words[k] = 0u;
    if (ticket && i < kTicketWords) ticket[i] = 0u;
}

// threads of a k_decode_reset launch for n words (and the ticket words)
inline int64_t reset_threads(int64_t n) { return (n + 3) / 4 > kTicketWords ? (n + 3) / 4 : kTicketWords; }

// This block's ticket, taken by one thread. Tickets come from m counters, m the largest power
// of two <= kTicketClasses that divides `chains`; block b draws from counter b mod m, which
// deals the tickets congruent to b mod m in the order the blocks arrive (every residue class
// has as many blocks as tickets). A tile's predecessor, `chains` tickets earlier, is in the
// same class and was dealt before it, to a block that has started: the oldest unfinished
// ticket of each class can always proceed, so no wait is circular. A single counter would
// serialise every block start on one address.
__device__ __forceinline__ int take_ticket(uint32_t *tickets, uint32_t chains)
{
    const uint32_t m = min((uint32_t)kTicketClasses, chains & (0u - chains));
    const uint32_t k = blockIdx.x & (m - 1u);
    return (int)(k + m * atomicAdd(tickets + k * kTicketStride, 1u));
}

// One lane's 8 running bytes as 4 tagged words, word k at base + 16 k: the 16 lanes of a tile
// write one contiguous 64-byte segment per store instruction (device-scope stores go past the
// L2 to memory, where a segment written in part costs as much as a whole one).
__device__ __forceinline__ void lb_publish(uint32_t *base, uint2 v, uint32_t tag)
{
    const uint32_t t = tag << 16;
    __hip_atomic_store(base + 0, t | (v.x & 0xffffu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(base + 16, t | (v.x >> 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(base + 32, t | (v.y & 0xffffu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(base + 48, t | (v.y >> 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// reads one lane's part of a published value (layout as lb_publish); true if all four words
// carry the tag
__device__ __forceinline__ bool lb_read(const uint32_t *base, uint32_t tag, uint2 &v)
{
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
        w[k] = __hip_atomic_load(const_cast<uint32_t *>(base) + 16 * k, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    v.x = (w[0] & 0xffffu) | (w[1] << 16);
    v.y = (w[2] & 0xffffu) | (w[3] << 16);
    return (w[0] >> 16) == tag && (w[1] >> 16) == tag && (w[2] >> 16) == tag &&
           (w[3] >> 16) == tag;
}

// Running sums of the delta chain in offset-64 form: a byte holds v + 64. Every value the
// scans handle is a difference of two running codes or a running code (|c| <= 16), so it lies
// in [-32, 32] and every byte of every intermediate below stays inside [0, 255]: whole 32-bit
// adds act byte-wise, with no carry or borrow between bytes.
constexpr uint32_t kOff64 = 0x40404040u;   // zero in offset-64 form

// v + d per byte, d a two's complement delta: (v + 64) + (d + 128) - 128 (the intermediate
// (v + d) + 192 stays within [160, 224])
__device__ __forceinline__ uint2 run_step(uint2 run, uint2 d)
{
    return make_uint2(run.x + (d.x ^ 0x80808080u) + 0x7f7f7f80u,
                      run.y + (d.y ^ 0x80808080u) + 0x7f7f7f80u);
}

// a + b per byte, both offset-64: (a + 64) + (b + 64) - 64
__device__ __forceinline__ uint2 add_off(uint2 a, uint2 b)
{
    return make_uint2(a.x + b.x + 0xbfbfbfc0u, a.y + b.y + 0xbfbfbfc0u);
}

// a - b per byte, both offset-64: ((a + 64) + 64) - (b + 64)
__device__ __forceinline__ uint2 sub_off(uint2 a, uint2 b)
{
    return make_uint2(a.x + kOff64 - b.x, a.y + kOff64 - b.y);
}

// Decoupled look-back of one tile of a chain, run by the 16 lanes of one lane group (lane g
// carries group g's 8 running bytes, offset-64); they move together: a value is taken only when
// every lane's words are complete. slot: this tile's word slot; the chain's previous tile sits
// `step` slots earlier. Publishes this tile's aggregate (tile > 0) and inclusive prefix, and
// returns the exclusive prefix. A wait longer than kSpinLimit sets *err and gives up.
__device__ __forceinline__ uint2 chain_lookback(uint32_t *lb_agg, uint32_t *lb_incl, size_t slot,
                                                size_t step, int tile, uint2 agg, int g,
                                                uint32_t *err)
{
    uint2 excl = make_uint2(kOff64, kOff64);
    const size_t me = slot * 64 + g;
    if (tile == 0) {
        lb_publish(lb_incl + me, agg, 2u);
        return excl;
    }
    lb_publish(lb_agg + me, agg, 1u);
    size_t pred = slot - step;
    uint32_t spins = 0;
    while (true) {
        const size_t pw = pred * 64 + g;
        uint2 v;
        if (__ballot(!lb_read(lb_incl + pw, 2u, v)) == 0ull) {
            excl = add_off(excl, v);
            break;
        }
        if (__ballot(!lb_read(lb_agg + pw, 1u, v)) == 0ull) {
            excl = add_off(excl, v);
            pred -= step;
            spins = 0;
            continue;
        }
        if (++spins > kSpinLimit) {   // never expected: report and give up the wait
            if (g == 0) atomicOr(err, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    lb_publish(lb_incl + me, add_off(excl, agg), 2u);
    return excl;
}

// RoPE at a stored position on x = group_sign(g) times a rotated-back key row:
// k_i = x_i*C - x_{i+64}*S, k_{i+64} = x_{i+64}*C + x_i*S. The partner lane (group g ^ 8)
// carries the opposite lane sign, hence the flipped +-.
__device__ __forceinline__ void rope_redo(float x[8], int g, const float cr[8], const float sr[8])
{
    const float sg = g >= 8 ? -1.0f : 1.0f;
    float u[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        u[k] = x[k] * sr[k];   // the partner's product (both lanes hold the same S)
        x[k] = x[k] * cr[k];
    }
    rope_cross(x, u, sg);
}

// Reconstructs one token of one chain for this lane's 8 dims: x = group_sign(g) times the
// reconstructed row (dims 8g..8g+7). code: the token's absolute code bytes as c + 64, s16:
// this group's scale, (cr, sr): the rotary table row of the token's position (keys only).
template <bool IS_KEY>
__device__ __forceinline__ void decode_row(int g, uint2 code, uint32_t s16, const float cr[8],
                                           const float sr[8], float x[8])
{
    // The in-lane butterflies (h = 1, 2, 4) run on the integer codes in packed fp16, where
    // they are exact (|sums| <= 8 * 16): each code byte c + 64 becomes the fp16 1024 + (c + 64)
    // by placing it under the exponent byte 0x64, and one packed add removes the 1088. One
    // v_pk_add_f16 with op_sel / neg_hi gives a pair's sum in the low half and its difference
    // in the high half. Then x = (s / 2) * (1 / sqrt(128)) * (sum of codes), rounded once.
    const float hs = (0.5f * kInvSqrt128) * h2f(s16);
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
    // now q0 = (y0, y1), q1 = (y2, y3), q2 = (y4, y5), q3 = (y6, y7)
    asm("v_pk_add_f16 %0, %4, %5 op_sel:[0,0] op_sel_hi:[0,0] neg_hi:[0,1]\n"   // (z0, z2)
        "v_pk_add_f16 %1, %4, %5 op_sel:[1,1] op_sel_hi:[1,1] neg_hi:[0,1]\n"   // (z1, z3)
        "v_pk_add_f16 %2, %6, %7 op_sel:[0,0] op_sel_hi:[0,0] neg_hi:[0,1]\n"   // (z4, z6)
        "v_pk_add_f16 %3, %6, %7 op_sel:[1,1] op_sel_hi:[1,1] neg_hi:[0,1]\n"   // (z5, z7)
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(q0), "v"(q1), "v"(q2), "v"(q3));
    asm("v_pk_add_f16 %0, %4, %6 op_sel:[0,0] op_sel_hi:[0,0] neg_hi:[0,1]\n"   // (o0, o4)
        "v_pk_add_f16 %1, %4, %6 op_sel:[1,1] op_sel_hi:[1,1] neg_hi:[0,1]\n"   // (o2, o6)
        "v_pk_add_f16 %2, %5, %7 op_sel:[0,0] op_sel_hi:[0,0] neg_hi:[0,1]\n"   // (o1, o5)
        "v_pk_add_f16 %3, %5, %7 op_sel:[1,1] op_sel_hi:[1,1] neg_hi:[0,1]\n"   // (o3, o7)
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3)
        : "v"(r0), "v"(r1), "v"(r2), "v"(r3));
    // fp16 half times fp32 scale in one v_fma_mix_f32 (product rounded once, + 0)
    asm("v_fma_mix_f32 %0, %8, %12, 0 op_sel:[0,0,0] op_sel_hi:[1,0,0]\n"
        "v_fma_mix_f32 %4, %8, %12, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n"
        "v_fma_mix_f32 %2, %9, %12, 0 op_sel:[0,0,0] op_sel_hi:[1,0,0]\n"
        "v_fma_mix_f32 %6, %9, %12, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n"
        "v_fma_mix_f32 %1, %10, %12, 0 op_sel:[0,0,0] op_sel_hi:[1,0,0]\n"
        "v_fma_mix_f32 %5, %10, %12, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n"
        "v_fma_mix_f32 %3, %11, %12, 0 op_sel:[0,0,0] op_sel_hi:[1,0,0]\n"
        "v_fma_mix_f32 %7, %11, %12, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7])
        : "v"(q0), "v"(q1), "v"(q2), "v"(q3), "v"(hs));
    hadamard_cross_lane(x, g);   // x = group_sign(g) * (the reconstructed row)
    if (IS_KEY) rope_redo(x, g, cr, sr);
}

// Stores this lane's 8 dims of a reconstructed row (x = group_sign(g) times the row) as fp32
// or fp16 at row j of the chain starting at row_off.
__device__ __forceinline__ void store_row(void *out, bool out_f32, size_t row_off, int j, int g,
                                          float x[8])
{
    const uint32_t sbit = (__popc(g & 15) & 1) ? 0x80000000u : 0u;   // group_sign as a sign bit
    const size_t o = row_off + (size_t)j * kHeadDim + 8 * g;
    if (out_f32) {
        float *dst = (float *)out + o;
#pragma unroll
        for (int k = 0; k < 8; k++) x[k] = __uint_as_float(__float_as_uint(x[k]) ^ sbit);
        const u32x4 v0 = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                          __float_as_uint(x[3])};
        const u32x4 v1 = {__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                          __float_as_uint(x[7])};
        // the output is far larger than the caches: stream it past them
        __builtin_nontemporal_store(v0, reinterpret_cast<u32x4 *>(dst));
        __builtin_nontemporal_store(v1, reinterpret_cast<u32x4 *>(dst + 4));
    } else {
        // rounding to fp16 commutes with the sign, which is flipped on the packed halves
        uint16_t *dst = (uint16_t *)out + o;
        const uint32_t s2 = sbit | (sbit >> 16);
        u32x4 v;
        v.x = f2h_pack(x[0], x[1]) ^ s2;
        v.y = f2h_pack(x[2], x[3]) ^ s2;
        v.z = f2h_pack(x[4], x[5]) ^ s2;
        v.w = f2h_pack(x[6], x[7]) ^ s2;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
    }
}

// decode_row, then the row stored at row j of the chain starting at row_off
template <bool IS_KEY>
__device__ __forceinline__ void decode_store(const CodecArgs &a, size_t row_off, int j, int g,
                                             uint2 code, uint32_t s16, const float cr[8],
                                             const float sr[8])
{
    float x[8];
    decode_row<IS_KEY>(g, code, s16, cr, sr, x);
    store_row(IS_KEY ? a.out_k : a.out_v, a.out_f32, row_off, j, g, x);
}

struct DecodeShared {
    uint2 tot[4][16];                           // running-sum totals of the waves
    uint2 excl[16];                             // the tile's exclusive prefix
    int32_t pos[kDecTile];                      // the tile's positions
    uint4 scale[kDecTile * kGroups * 2 / 16];     // the tile's fp16 scales
    uint4 delta[kDecTile * kHeadDim / 16];        // the tile's delta codes
};

// Loads a tile of one chain into LDS: nt (<= 16 * RUN) rows of delta codes and scales starting
// at chain row `row0`, and, when pos is not null, the nt positions (clamped into [0, T)). Every
// load of a thread is issued before its first LDS store, so they are in flight together (one
// memory latency per tile, not one per chunk). The caller synchronises before reading.
template <int RUN>
__device__ __forceinline__ void stage_tile(const int8_t *codes, const uint16_t *scales,
                                           size_t row0, int nt, const int32_t *pos, int T,
                                           uint4 *s_delta, uint4 *s_scale, int32_t *s_pos)
{
    constexpr int kTile = 16 * RUN;
    constexpr int kDeltaChunks = kTile * kHeadDim / 16 / kCodecThreads;
    constexpr int kScaleChunks = (kTile * 2 + kCodecThreads - 1) / kCodecThreads;
    static_assert(kTile <= kCodecThreads, "one position per thread");
    const u32x4 *dc = reinterpret_cast<const u32x4 *>(codes + row0 * kHeadDim);
    const u32x4 *sc = reinterpret_cast<const u32x4 *>(scales + row0 * kGroups);
    const int tid = threadIdx.x;
    u32x4 d[kDeltaChunks], sv[kScaleChunks];
    int pv = 0;
#pragma unroll
    for (int k = 0; k < kDeltaChunks; k++)
        if (tid + k * kCodecThreads < 8 * nt)
            d[k] = __builtin_nontemporal_load(dc + tid + k * kCodecThreads);
#pragma unroll
    for (int k = 0; k < kScaleChunks; k++)
        if (tid + k * kCodecThreads < 2 * nt)
            sv[k] = __builtin_nontemporal_load(sc + tid + k * kCodecThreads);
    if (pos && tid < nt) pv = pos[tid];
#pragma unroll
    for (int k = 0; k < kDeltaChunks; k++)
        if (tid + k * kCodecThreads < 8 * nt)
            s_delta[tid + k * kCodecThreads] = make_uint4(d[k].x, d[k].y, d[k].z, d[k].w);
#pragma unroll
    for (int k = 0; k < kScaleChunks; k++)
        if (tid + k * kCodecThreads < 2 * nt)
            s_scale[tid + k * kCodecThreads] = make_uint4(sv[k].x, sv[k].y, sv[k].z, sv[k].w);
    if (pos && tid < nt) s_pos[tid] = min(max(pv, 0), T - 1);
}

// This lane's 8 delta bytes of staged tile row jl: dims 8g..8g+7 (one uint2), or with SPLIT
// dims 4g..4g+3 and 64+4g..64+4g+3 (two dwords of the 128-byte row)
template <bool SPLIT>
__device__ __forceinline__ uint2 lane_delta(const uint4 *s_delta, int jl, int g)
{
    if (SPLIT) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(s_delta) + jl * 32 + g;
        return make_uint2(w[0], w[16]);
    }
    return reinterpret_cast<const uint2 *>(s_delta)[jl * 16 + g];
}

// The running code of this lane's 8 dims (see lane_delta) just before lane group q's first
// token of a staged tile (q walks tile rows q * RUN ..), offset-64 (c + 64 per byte).
// Synchronises the block before reading the tile and after the look-back; slot/step/err as in
// chain_lookback. Every tile of a chain must use the same partition of the dims over lanes.
template <int RUN, bool SPLIT = false>
__device__ __forceinline__ uint2 tile_run_base(const uint4 *s_delta, int nt, int q, int g,
                                               uint2 (*s_tot)[16], uint2 *s_excl,
                                               uint32_t *lb_agg, uint32_t *lb_incl, size_t slot,
                                               size_t step, int tile, uint32_t *err)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // 1. the sum of this lane group's deltas (offset-64)
    __syncthreads();
    uint2 acc = make_uint2(kOff64, kOff64);
#pragma unroll
    for (int i = 0; i < RUN; i++) {
        const int jl = q * RUN + i;
        if (jl < nt) acc = run_step(acc, lane_delta<SPLIT>(s_delta, jl, g));
    }
    // 2. prefix over the lane groups before this one: across the 4 rows of a wave with lane
    //    shuffles, then across the 4 waves through LDS (one barrier); group 15's lanes then
    //    hold the tile total in gp + acc
    const int row = lane >> 4;
    uint2 incl = acc;
#pragma unroll
    for (int d = 1; d < 4; d <<= 1) {
        const uint2 t = make_uint2((uint32_t)__shfl_up((int)incl.x, 16 * d),
                                   (uint32_t)__shfl_up((int)incl.y, 16 * d));
        if (row >= d) incl = add_off(incl, t);
    }
    if (row == 3) s_tot[wave][g] = incl;
    __syncthreads();
    for (int w = 0; w < wave; w++) incl = add_off(incl, s_tot[w][g]);
    const uint2 gp = sub_off(incl, acc);
    // 3. decoupled look-back, done by lane group 15 (it holds the tile total)
    if (q == 15)
        s_excl[g] = chain_lookback(lb_agg, lb_incl, slot, step, tile, add_off(gp, acc), g, err);
    __syncthreads();
    return add_off(s_excl[g], gp);
}

template <bool IS_KEY>
__device__ void decode_tile(const CodecArgs &a, int lc, int h, int tile, int ticket, int chains,
                            DecodeShared &sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane_group(lane & 15), q = wave * 4 + (lane >> 4);
    const int n_keep = a.n_keep;
    const size_t chain = (size_t)lc * a.H + h;
    const int t0 = tile * kDecTile;
    const int nt = min(kDecTile, n_keep - t0);
    const int j0 = t0 + q * kDecRun;
    const int32_t *s_pos = sh.pos;

    stage_tile<kDecRun>(IS_KEY ? a.codes_k : a.codes_v, IS_KEY ? a.scales_k : a.scales_v,
               chain * (size_t)n_keep + t0, nt,
               IS_KEY ? a.positions + (size_t)lc * n_keep + t0 : nullptr, a.T, sh.delta,
               sh.scale, sh.pos);
    uint2 run = tile_run_base<kDecRun>(sh.delta, nt, q, g, sh.tot, sh.excl, a.lb_agg, a.lb_incl,
                              (size_t)ticket, (size_t)chains, tile, a.lb_ticket + kTicketErr);
    const uint2 *sd = reinterpret_cast<const uint2 *>(sh.delta) + g;   // [token][16 lanes]
    // 4. reconstruct every token of this lane group; the next token's rotary rows are requested
    //    before the current token is computed
    const size_t row_off = chain * (size_t)n_keep * kHeadDim;
    const uint16_t *sl = reinterpret_cast<const uint16_t *>(sh.scale);
    const int jend = min(n_keep, j0 + kDecRun);
    float rc[2][8], rs[2][8];   // rotary rows of the current and the next token
    if (IS_KEY && j0 < jend) {
        const size_t p = (size_t)s_pos[j0 - t0] * 64 + 8 * (g & 7);
        load_f32x8(a.rope_cos + p, rc[0]);
        load_f32x8(a.rope_sin + p, rs[0]);
    }
#pragma unroll
    for (int i = 0; i < kDecRun; i++) {
        const int j = j0 + i, cur = i & 1;
        if (j < jend) {
            if (IS_KEY && j + 1 < jend) {
                const size_t p = (size_t)s_pos[j + 1 - t0] * 64 + 8 * (g & 7);
                load_f32x8(a.rope_cos + p, rc[cur ^ 1]);
                load_f32x8(a.rope_sin + p, rs[cur ^ 1]);
            }
            run = run_step(run, sd[(j - t0) * 16]);
            decode_store<IS_KEY>(a, row_off, j, g, run, sl[(j - t0) * kGroups + g], rc[cur],
                                 rs[cur]);
        }
    }
}

// grid: Lc * 2 * H * dec_tiles_per_chain blocks; the logical tile comes from the ticket, ordered
// tile-major over the chains: tile k of a chain holds ticket k * chains + chain, so its
// predecessor started `chains` tickets earlier and has usually published its inclusive prefix
// by the time it is looked up (a chain-major order would start a chain's tiles together and
// make the last ones walk back through many tile sums). Chain index = lc + Lc (tensor + 2 h):
// a ticket's class, and with it the block's XCD, follows the layer (chains = 2 Lc H), so the
// kv heads of one layer -- which share its kept positions -- read their rotary rows through
// the same L2 instead of one XCD per head.
__global__ __launch_bounds__(kCodecThreads) void k_decode(CodecArgs a)
{
    __shared__ int s_ticket;
    const int chains = (int)(gridDim.x / (uint32_t)a.dec_tiles_per_chain);
    if (threadIdx.x == 0) s_ticket = take_ticket(a.lb_ticket, (uint32_t)chains);
    __syncthreads();
    const int ticket = s_ticket;
    const int tile = ticket / chains;
    uint32_t r = ticket % chains;
    const uint32_t Lc = (uint32_t)chains / (2u * (uint32_t)a.H);
    const int lc = r % Lc;
    r /= Lc;
    const int tensor = r & 1;
    const int h = r >> 1;
    __shared__ DecodeShared sh;
    if (tensor == 0)
        decode_tile<true>(a, lc, h, tile, ticket, chains, sh);
    else
        decode_tile<false>(a, lc, h, tile, ticket, chains, sh);
}

}  // namespace nq
