// Device helpers shared by the gfx950 kernels of libnq.
//
// Lane layout used by every row kernel: a 128-float head row is spread over 16 consecutive
// lanes, each holding one group of 8 consecutive dims -- one 16-byte fp16 load per lane, a
// fully coalesced 256-byte row per 16 lanes, and one E8 group per lane. Lane l (= lane & 15)
// holds group l in the scoring and attention kernels and group lane_group(l) (a fixed
// permutation that suits the Hadamard butterflies) in the codec kernels. A wave64 therefore
// works on 4 rows at once ("lane groups" 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nq {

constexpr int kHeadDim = 128;
constexpr int kGroups = 16;                       // 8-float groups per row
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;    // fp32 nearest to 1/sqrt(128)

__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t f2h_bits(float x)   // round to nearest even
{
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed fp16 pair (lo, hi), rounded to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t f2h_pack(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

// 8 fp16 values (one 16-byte load) -> fp32
__device__ __forceinline__ void load_f16x8(const uint16_t *__restrict__ p, float x[8])
{
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        x[2 * k] = h2f(w[k] & 0xffffu);
        x[2 * k + 1] = h2f(w[k] >> 16);
    }
}

// the same for data read once: a non-temporal load does not keep the line in the caches
// 8 bytes stored past the caches (outputs written once and not read back by the kernel)
__device__ __forceinline__ void store_stream(void *p, uint2 v)
{
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p));
}

__device__ __forceinline__ void load_f16x8_stream(const uint16_t *__restrict__ p, float x[8])
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        x[2 * k] = h2f(w[k] & 0xffffu);
        x[2 * k + 1] = h2f(w[k] >> 16);
    }
}

__device__ __forceinline__ void load_f32x8(const float *__restrict__ p, float x[8])
{
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Cross-lane moves inside a 16-lane row with DPP (no LDS traffic): row_ror:8 = lane ^ 8
// within the row.
constexpr int kDppRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float lane_xor8(float v) { return dpp<kDppRor8>(v); }

// One transpose-reduce level across lane partners l ^ m (DPP control CTRL): lanes whose
// selecting bit is clear keep a + a(partner), the others b + b(partner).
template <int CTRL>
__device__ __forceinline__ float tr_level(float a, float b, bool hi)
{
    return (hi ? b : a) + dpp<CTRL>(hi ? a : b);
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
        float v = d[0] + dpp<kRor8>(d[0]);
        v += dpp<kHm>(v);
        v += dpp<kX2>(v);
        return v + dpp<kX1>(v);
    } else if constexpr (G == 2) {
        float v = tr_level<kRor8>(d[0], d[1], b3);
        v += dpp<kHm>(v);
        v += dpp<kX2>(v);
        return v + dpp<kX1>(v);
    } else if constexpr (G == 4) {
        const float v01 = tr_level<kRor8>(d[0], d[1], b3);
        const float v23 = tr_level<kRor8>(d[2], d[3], b3);
        float v = tr_level<kHm>(v01, v23, b2);
        v += dpp<kX2>(v);
        return v + dpp<kX1>(v);
    } else {
        static_assert(G == 8, "G in {1, 2, 4, 8}");
        const float v01 = tr_level<kRor8>(d[0], d[1], b3);
        const float v23 = tr_level<kRor8>(d[2], d[3], b3);
        const float v45 = tr_level<kRor8>(d[4], d[5], b3);
        const float v67 = tr_level<kRor8>(d[6], d[7], b3);
        const float v03 = tr_level<kHm>(v01, v23, b2);
        const float v47 = tr_level<kHm>(v45, v67, b2);
        const float v = tr_level<kX2>(v03, v47, b1);
        return v + dpp<kX1>(v);
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

// Workgroup-to-XCD aware block order. The dispatcher hands consecutive workgroup ids to the 8
// XCDs round robin; this maps the hardware id to a logical id so that logically consecutive
// blocks (which share cached rows, e.g. the rotary table of one token tile) run on one XCD and
// share its L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t n)
{
    const uint32_t per = n >> 3, rem = n & 7u, x = b & 7u;
    return x * per + (x < rem ? x : rem) + (b >> 3);
}

}  // namespace nq
