// Key-key proxy scoring and eviction (steps 1-2).
//
// "NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破", sections "Token淘汰机制" (drop the
// least important tokens, always keep BOS and a recent sliding window) and "技术实现细节"
// (key-key proxy scorer, no extra computation); "Como comprimir o KV cache do seu LLM em 33x sem
// treino", "Como funciona" steps 1-2 (cross-head inner product).
//
// The recent window's keys stand in for queries: qbar_h = sum of the last W keys of head h
// (fp64: exact for fp16 inputs), and a candidate's score is s_t = sum_h <qbar_h, k_{h,t}>
// (fp64). The scorer is a GEMV over all of K -- HBM bound, no matrix cores.
#pragma once

#include "nq_common.hpp"

namespace nq {

// ---- window sums: one block per (compressed layer, head) ----------------------------------
__global__ __launch_bounds__(256) void k_window_sum(const uint16_t *__restrict__ K, int H, int T,
                                                   int W, int layer_begin,
                                                   double *__restrict__ qbar)
{
    __shared__ double red[16][kHeadDim];
    const int lh = blockIdx.x;
    const int lc = lh / H, h = lh % H;
    const int g = threadIdx.x & 15, slot = threadIdx.x >> 4;
    const uint16_t *base = K + ((size_t)(layer_begin + lc) * H + h) * (size_t)T * kHeadDim + 8 * g;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // 8 rows per thread in flight at once, then their sums (exact in fp64 in any order)
    for (int w0 = max(0, T - W) + slot; w0 < T; w0 += 16 * 8) {
        u32x4 v[8];
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const int w = w0 + 16 * r;
            v[r] = w < T ? *reinterpret_cast<const u32x4 *>(base + (size_t)w * kHeadDim)
                         : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const uint32_t wd[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                acc[2 * k] += (double)h2f(wd[k] & 0xffffu);
                acc[2 * k + 1] += (double)h2f(wd[k] >> 16);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 8; k++) red[slot][8 * g + k] = acc[k];
    __syncthreads();
    if (threadIdx.x < kHeadDim) {
        double s = 0.0;
        for (int r = 0; r < 16; r++) s += red[r][threadIdx.x];   // exact: fp16 sums fit fp64
        qbar[(size_t)lh * kHeadDim + threadIdx.x] = s;
    }
}

// ---- scores: block = 64 tokens of one compressed layer; lane group per row -----------------
constexpr int kScoreTile = 64;

__global__ __launch_bounds__(256) void k_scores(const uint16_t *__restrict__ K,
                                                const double *__restrict__ qbar, int H, int T,
                                                int W, int layer_begin, int tiles,
                                                double *__restrict__ scores)
{
    // (no XCD-aware order here: nothing is shared between blocks, and plain order measured
    // faster)
    const int lc = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 15, r4 = lane >> 4;
    const int c_end = T - W;                        // candidates: [1, c_end)
    const uint16_t *Kl = K + (size_t)(layer_begin + lc) * H * (size_t)T * kHeadDim + 8 * g;
    const double *qb = qbar + (size_t)lc * H * kHeadDim + 8 * g;
    int t[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
        t[u] = tile * kScoreTile + wave * 16 + u * 4 + r4;
        ok[u] = t[u] >= 1 && t[u] < c_end;
    }
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int h = 0; h < H; h++) {
        double q[8];
#pragma unroll
        for (int k = 0; k < 8; k++) q[k] = qb[(size_t)h * kHeadDim + k];
        const uint16_t *Kh = Kl + (size_t)h * T * kHeadDim;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            if (ok[u]) {
                float x[8];
                load_f16x8_stream(Kh + (size_t)t[u] * kHeadDim, x);
#pragma unroll
                for (int k = 0; k < 8; k++) acc[u] = __builtin_fma(q[k], (double)x[k], acc[u]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) acc[u] += __shfl_xor(acc[u], m);
        if (g == 0 && ok[u]) scores[(size_t)lc * T + t[u]] = acc[u];
    }
}

// ---- selection: one 1024-thread block per compressed layer ---------------------------------
// Keeps the m best candidates by (score desc, position asc): an MSB-first radix select over
// order-preserving 64-bit keys finds the m-th best key exactly, then one ordered pass emits BOS,
// the window, the candidates above that key and the lowest-positioned ones equal to it.
constexpr int kSelThreads = 1024;
constexpr int kHistCopies = 16;   // LDS histogram copies of the radix passes (lane mod 16)
constexpr int kSelCompact = 4096; // bucket size up to which k_select_mem gathers it into LDS

__device__ __forceinline__ uint64_t order_key(double d)
{
    uint64_t b = (uint64_t)__double_as_longlong(d);
    if (d == 0.0) b = 0ull;                               // -0 and +0 are one key
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// exclusive block scan of one uint32 per thread (1024 threads = 16 waves)
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *s_wave, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < kSelThreads / 64; w++) {
        const uint32_t x = s_wave[w];
        if (w < wave) before += x;
        all += x;
    }
    __syncthreads();
    total = all;
    return before + incl - v;
}

// LDS state of one layer's selection. The radix histograms come in kHistCopies copies, copy =
// lane mod kHistCopies: keys crowd into a few digits on the first passes (sign and exponent
// bits), and a wave's 64 lanes adding to one LDS word serialise; with 16 copies at most 4
// lanes of an instruction share a word.
struct SelectShared {
    uint32_t hist[kHistCopies][256];
    uint32_t wave_sum[kSelThreads / 64];
    uint64_t wave_min[kSelThreads / 64], wave_max[kSelThreads / 64];
    uint64_t prefix, mask;   // bits of the m-th best key resolved so far
    int krem;                // rank of that key among the keys matching prefix/mask
    uint32_t bucket;         // number of keys matching prefix/mask
    int all;                 // the whole matching bucket is kept
    int bits;                // bits left to resolve
};

// Radix state from every thread's smallest and largest candidate key: the bits shared by all
// candidates (the common prefix of the extremes) need no pass. Ends with a barrier.
__device__ __forceinline__ void sel_init_prefix(SelectShared &sh, uint64_t kmin, uint64_t kmax)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t a = __shfl_xor(kmin, d), b = __shfl_xor(kmax, d);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    if (lane == 0) { sh.wave_min[wave] = kmin; sh.wave_max[wave] = kmax; }
    __syncthreads();
    if (tid == 0) {
        uint64_t lo = sh.wave_min[0], hi = sh.wave_max[0];
        for (int w = 1; w < kSelThreads / 64; w++) {
            lo = sh.wave_min[w] < lo ? sh.wave_min[w] : lo;
            hi = sh.wave_max[w] > hi ? sh.wave_max[w] : hi;
        }
        const int common = lo == hi ? 64 : __clzll((long long)(lo ^ hi));
        sh.bits = 64 - common;
        sh.mask = common == 64 ? ~0ull : (common == 0 ? 0ull : ~0ull << (64 - common));
        sh.prefix = lo & sh.mask;
    }
    __syncthreads();
}

// Clears the histogram copies. Ends with a barrier.
__device__ __forceinline__ void sel_clear_hist(SelectShared &sh)
{
    for (int i = threadIdx.x; i < kHistCopies * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0u;
    __syncthreads();
}

// One radix digit: key k (matching the pass's prefix/mask) counted in its lane's copy
__device__ __forceinline__ void sel_count(SelectShared &sh, uint64_t k, int shift, uint32_t dmask)
{
    atomicAdd(&sh.hist[(threadIdx.x & 63) % kHistCopies][(uint32_t)(k >> shift) & dmask], 1u);
}

// After a pass has counted its keys: sums the copies, finds the digit that holds the krem-th
// largest key and narrows prefix/mask/krem to it (all = 1 when the whole bucket is kept).
// Starts and ends with a barrier.
__device__ __forceinline__ void sel_pick_digit(SelectShared &sh, int shift, uint32_t dmask,
                                               uint64_t prefix, uint64_t mask)
{
    const int tid = threadIdx.x;
    __syncthreads();
    if (tid < 256) {
        uint32_t c = 0;
        for (int w = 0; w < kHistCopies; w++) c += sh.hist[w][tid];
        sh.hist[0][tid] = c;
    }
    __syncthreads();
    if (tid < 64) {
        // lane L covers digits 255-4L .. 252-4L (descending)
        const int krem = sh.krem;
        uint32_t c[4], loc = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) { c[i] = sh.hist[0][255 - 4 * tid - i]; loc += c[i]; }
        uint32_t incl = loc;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(incl, d);
            if (tid >= d) incl += o;
        }
        uint32_t above = incl - loc;               // keys in higher digits
        if (above < (uint32_t)krem && incl >= (uint32_t)krem) {
            for (int i = 0; i < 4; i++) {
                if (above + c[i] >= (uint32_t)krem) {
                    const uint32_t dgt = 255 - 4 * tid - i;
                    sh.prefix = prefix | ((uint64_t)dgt << shift);
                    sh.mask = mask | ((uint64_t)dmask << shift);
                    sh.krem = krem - (int)above;
                    sh.bucket = c[i];
                    if (c[i] == (uint32_t)(krem - (int)above)) sh.all = 1;
                    break;
                }
                above += c[i];
            }
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void k_select(const double *__restrict__ scores, int T,
                                                        int W, int n_keep,
                                                        int32_t *__restrict__ positions)
{
    __shared__ SelectShared sh;
    const int lc = blockIdx.x;
    const double *s = scores + (size_t)lc * T;
    int32_t *out = positions + (size_t)lc * n_keep;
    const int tid = threadIdx.x;
    const int c_end = T - W;
    const int n_cand = c_end > 1 ? c_end - 1 : 0;
    const int m = n_keep - (T - n_cand);
    const bool partial = m > 0 && m < n_cand;

    if (tid == 0) { sh.prefix = 0ull; sh.mask = 0ull; sh.krem = m; sh.all = 0; sh.bits = 64; }
    if (partial) {
        uint64_t kmin = ~0ull, kmax = 0ull;
        for (int t0 = 1 + tid; t0 < c_end; t0 += 8 * kSelThreads) {
            double v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int t = t0 + u * kSelThreads;
                v[u] = t < c_end ? s[t] : 0.0;
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                if (t0 + u * kSelThreads < c_end) {
                    const uint64_t k = order_key(v[u]);
                    kmin = k < kmin ? k : kmin;
                    kmax = k > kmax ? k : kmax;
                }
            }
        }
        sel_init_prefix(sh, kmin, kmax);
    }
    __syncthreads();
    if (partial) {
        for (int top = sh.bits; top > 0; top -= 8) {
            const int shift = top >= 8 ? top - 8 : 0;
            const uint32_t dmask = top >= 8 ? 255u : ((1u << top) - 1u);
            sel_clear_hist(sh);
            const uint64_t prefix = sh.prefix, mask = sh.mask;
            // 8 independent loads in flight per thread, then their histogram updates
            for (int t0 = 1 + tid; t0 < c_end; t0 += 8 * kSelThreads) {
                double v[8];
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const int t = t0 + u * kSelThreads;
                    v[u] = t < c_end ? s[t] : 0.0;
                }
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const uint64_t k = order_key(v[u]);
                    if (t0 + u * kSelThreads < c_end && (k & mask) == prefix)
                        sel_count(sh, k, shift, dmask);
                }
            }
            sel_pick_digit(sh, shift, dmask, prefix, mask);
            if (sh.all) break;                             // the whole bucket is kept
        }
    }
    const uint64_t prefix = sh.prefix, mask = sh.mask;
    const int krem = sh.krem;
    const bool take_all_eq = sh.all != 0;
    // ordered emission: chunks of 4 consecutive positions per thread
    uint32_t eq_base = 0, out_base = 0;
    for (int t0 = 0; t0 < T; t0 += 4 * kSelThreads) {
        const int tb = t0 + 4 * tid;
        uint32_t keepf = 0, eqf = 0;
        uint32_t gt4 = 0;
        double v[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = tb + i;
            v[i] = (partial && t >= 1 && t < c_end) ? s[t] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = tb + i;
            if (t >= T) continue;
            const bool cand = t >= 1 && t < c_end;
            if (!cand) { keepf |= 1u << i; continue; }
            if (!partial) { if (m > 0) keepf |= 1u << i; continue; }
            const uint64_t k = order_key(v[i]) & mask;
            if (k > prefix) gt4 |= 1u << i;
            else if (k == prefix) eqf |= 1u << i;
        }
        uint32_t eq_tot;
        const uint32_t eq_before = block_excl_scan(__builtin_popcount(eqf), sh.wave_sum, eq_tot);
        uint32_t r = eq_base + eq_before;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (gt4 & (1u << i)) keepf |= 1u << i;
            if (eqf & (1u << i)) {
                if (take_all_eq || r < (uint32_t)krem) keepf |= 1u << i;
                r++;
            }
        }
        eq_base += eq_tot;
        uint32_t k_tot;
        uint32_t o = out_base + block_excl_scan(__builtin_popcount(keepf), sh.wave_sum, k_tot);
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (keepf & (1u << i)) {
                if (o < (uint32_t)n_keep) out[o] = tb + i;   // never past the caller's row
                o++;
            }
        out_base += k_tot;
    }
}

// ---- selection with the candidate keys held in registers -------------------------------------
// The same selection as k_select for layers of at most KPT * 1024 candidates: every thread
// loads its KPT candidates once (positions 1 + tid + 1024 u, u < KPT) and keeps their keys in
// registers, so the radix passes and the ordered emission read no memory. The emission ranks
// the kept positions with wave ballots: per chunk u of 1024 consecutive positions, each wave's
// count goes to LDS, one block scan over the (chunk, wave) counts gives every wave its offset,
// and a lane adds the kept lanes below it. Ties at the selected key are ranked the same way
// first (the lowest-positioned ones are kept).
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void k_select_reg(const double *__restrict__ scores,
                                                            int T, int W, int n_keep,
                                                            int32_t *__restrict__ positions)
{
    constexpr int kWaves = kSelThreads / 64;
    static_assert(KPT * kWaves <= kSelThreads, "one (chunk, wave) count per thread");
    __shared__ SelectShared sh;
    __shared__ uint32_t s_cnt[KPT * kWaves];
    const int lc = blockIdx.x;
    const double *s = scores + (size_t)lc * T;
    int32_t *out = positions + (size_t)lc * n_keep;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c_end = T - W;
    const int n_cand = c_end > 1 ? c_end - 1 : 0;
    const int m = n_keep - (T - n_cand);
    const bool partial = m > 0 && m < n_cand;

    uint64_t key[KPT];
    {
        double v[KPT];
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            const int t = 1 + tid + u * kSelThreads;
            v[u] = t < c_end ? s[t] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < KPT; u++) key[u] = order_key(v[u]);
    }
    if (tid == 0) { sh.prefix = 0ull; sh.mask = 0ull; sh.krem = m; sh.all = 0; sh.bits = 64; }
    if (partial) {
        uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            if (1 + tid + u * kSelThreads < c_end) {
                kmin = key[u] < kmin ? key[u] : kmin;
                kmax = key[u] > kmax ? key[u] : kmax;
            }
        }
        sel_init_prefix(sh, kmin, kmax);
    }
    __syncthreads();
    if (partial) {
        for (int top = sh.bits; top > 0; top -= 8) {
            const int shift = top >= 8 ? top - 8 : 0;
            const uint32_t dmask = top >= 8 ? 255u : ((1u << top) - 1u);
            sel_clear_hist(sh);
            const uint64_t prefix = sh.prefix, mask = sh.mask;
#pragma unroll
            for (int u = 0; u < KPT; u++)
                if (1 + tid + u * kSelThreads < c_end && (key[u] & mask) == prefix)
                    sel_count(sh, key[u], shift, dmask);
            sel_pick_digit(sh, shift, dmask, prefix, mask);
            if (sh.all) break;
        }
    }
    const uint64_t prefix = sh.prefix, mask = sh.mask;
    const int krem = sh.krem;
    const bool take_all_eq = sh.all != 0;
    const uint64_t below = (1ull << lane) - 1ull;      // lanes under this one
    // bit u: chunk u's candidate is above the selected key (gt) or equal to it (eq)
    uint32_t gt = 0u, eq = 0u;
    static_assert(KPT <= 32, "one flag bit per chunk");
#pragma unroll
    for (int u = 0; u < KPT; u++) {
        const int t = 1 + tid + u * kSelThreads;
        if (t < c_end) {
            if (!partial) {
                if (m > 0) gt |= 1u << u;
            } else {
                const uint64_t k = key[u] & mask;
                if (k > prefix) gt |= 1u << u;
                else if (k == prefix) eq |= 1u << u;
            }
        }
    }
    // rank the ties in position order, keep the first krem of them (or all)
    if (partial && !take_all_eq) {
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            const uint64_t b = __ballot((eq >> u) & 1u);
            if (lane == 0) s_cnt[u * kWaves + wave] = (uint32_t)__popcll(b);
        }
        __syncthreads();
        uint32_t tot;
        const uint32_t off = block_excl_scan(tid < KPT * kWaves ? s_cnt[tid] : 0u, sh.wave_sum, tot);
        if (tid < KPT * kWaves) s_cnt[tid] = off;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            const uint64_t b = __ballot((eq >> u) & 1u);
            const uint32_t r = s_cnt[u * kWaves + wave] + (uint32_t)__popcll(b & below);
            if (((eq >> u) & 1u) && r < (uint32_t)krem) gt |= 1u << u;
        }
        __syncthreads();
    } else {
        gt |= eq;
    }
    // output ranks of the kept candidates; BOS first, the window after the candidates
#pragma unroll
    for (int u = 0; u < KPT; u++) {
        const uint64_t b = __ballot((gt >> u) & 1u);
        if (lane == 0) s_cnt[u * kWaves + wave] = (uint32_t)__popcll(b);
    }
    __syncthreads();
    uint32_t kept;
    const uint32_t off = block_excl_scan(tid < KPT * kWaves ? s_cnt[tid] : 0u, sh.wave_sum, kept);
    if (tid < KPT * kWaves) s_cnt[tid] = off;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < KPT; u++) {
        const uint64_t b = __ballot((gt >> u) & 1u);
        if ((gt >> u) & 1u) {
            const uint32_t o = 1u + s_cnt[u * kWaves + wave] + (uint32_t)__popcll(b & below);
            if (o < (uint32_t)n_keep) out[o] = 1 + tid + u * kSelThreads;
        }
    }
    if (tid == 0 && T > 0 && n_keep > 0) out[0] = 0;
    const int ws = c_end > 1 ? c_end : 1;               // first window position after BOS
    for (int t = ws + tid; t < T; t += kSelThreads) {
        const uint32_t o = 1u + kept + (uint32_t)(t - ws);
        if (o < (uint32_t)n_keep) out[o] = t;
    }
}

// ---- selection for long layers, candidate flags in LDS ----------------------------------------
// The same selection for layers of at most KPT * 1024 candidates whose keys do not fit in
// registers: the radix passes re-read the scores (L2-resident) as k_select does, but the
// candidates' outcome -- above the selected key, or equal to it -- is kept as one bit per chunk
// and thread in LDS after a single further pass, and the ordered emission ranks kept positions with
// wave ballots and one block scan over the (chunk, wave) counts, as k_select_reg does (k_select
// instead scans the whole position range in 4096-position steps, two block scans per step).
// Chunk u of thread tid is position 1 + tid + 1024 u.

// exclusive scan of n counts in LDS, kPer per thread (n <= kPer * 1024); returns the total
template <int kPer>
__device__ __forceinline__ uint32_t scan_counts(uint32_t *cnt, int n, uint32_t *s_wave)
{
    const int tid = threadIdx.x;
    uint32_t loc[kPer], sum = 0;
#pragma unroll
    for (int e = 0; e < kPer; e++) {
        const int idx = tid * kPer + e;
        loc[e] = idx < n ? cnt[idx] : 0u;
        sum += loc[e];
    }
    uint32_t tot;
    uint32_t base = block_excl_scan(sum, s_wave, tot);   // its barriers order the reads above
#pragma unroll
    for (int e = 0; e < kPer; e++) {
        const int idx = tid * kPer + e;
        if (idx < n) cnt[idx] = base;
        base += loc[e];
    }
    __syncthreads();
    return tot;
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void k_select_mem(const double *__restrict__ scores,
                                                            int T, int W, int n_keep,
                                                            int32_t *__restrict__ positions)
{
    constexpr int kWaves = kSelThreads / 64;
    constexpr int kWords = (KPT + 31) / 32;
    constexpr int kCnt = KPT * kWaves;
    constexpr int kPer = (kCnt + kSelThreads - 1) / kSelThreads;
    // loads in flight per thread on every pass (16 or 32 measured no faster)
    constexpr int kBatch = 8;
    static_assert(KPT % kBatch == 0 && 32 % kBatch == 0, "whole batches of loads");
    __shared__ SelectShared sh;
    __shared__ uint32_t s_cnt[kCnt];
    __shared__ uint32_t s_gt[kWords][kSelThreads], s_eq[kWords][kSelThreads];
    __shared__ uint64_t s_ck[kSelCompact];   // the chosen bucket's keys, once it is small,
    __shared__ int32_t s_cp[kSelCompact];    // and their positions
    __shared__ uint32_t s_nck;
    __shared__ uint32_t s_above, s_match;
    __shared__ int s_retry;
    const int lc = blockIdx.x;
    const double *s = scores + (size_t)lc * T;
    int32_t *out = positions + (size_t)lc * n_keep;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c_end = T - W;
    const int n_cand = c_end > 1 ? c_end - 1 : 0;
    const int m = n_keep - (T - n_cand);
    const bool partial = m > 0 && m < n_cand;

    // The radix passes start below the bits that every candidate shares. Those are guessed from
    // the extremes of a sample (kBatch chunks spread over the layer): the first pass then also
    // counts the candidates above the guessed range and checks that the m-th best key lies in
    // it; if it does not (or the sample is flat), the extremes of every candidate are taken as
    // usual and the passes start over. A correct guess saves one read of the scores.
    if (tid == 0) {
        sh.prefix = 0ull; sh.mask = 0ull; sh.krem = m; sh.all = 0; sh.bits = 64;
        s_above = 0u; s_match = 0u; s_retry = 0;
    }
    bool guessed = false;
    if (partial) {
        uint64_t kmin = ~0ull, kmax = 0ull;
        double v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            const int t = 1 + tid + b * (KPT / kBatch) * kSelThreads;
            v[b] = t < c_end ? s[t] : 0.0;
        }
#pragma unroll
        for (int b = 0; b < kBatch; b++) {
            if (1 + tid + b * (KPT / kBatch) * kSelThreads < c_end) {
                const uint64_t k = order_key(v[b]);
                kmin = k < kmin ? k : kmin;
                kmax = k > kmax ? k : kmax;
            }
        }
        sel_init_prefix(sh, kmin, kmax);
        guessed = sh.bits > 0;
    }
    auto extremes_pass = [&]() {
        uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll 1
        for (int u0 = 0; u0 < KPT; u0 += kBatch) {
            double v[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; b++) {
                const int t = 1 + tid + (u0 + b) * kSelThreads;
                v[b] = t < c_end ? s[t] : 0.0;
            }
#pragma unroll
            for (int b = 0; b < kBatch; b++) {
                if (1 + tid + (u0 + b) * kSelThreads < c_end) {
                    const uint64_t k = order_key(v[b]);
                    kmin = k < kmin ? k : kmin;
                    kmax = k > kmax ? k : kmax;
                }
            }
        }
        if (tid == 0) { sh.krem = m; sh.all = 0; }
        sel_init_prefix(sh, kmin, kmax);
    };
    if (partial && !guessed) extremes_pass();
    __syncthreads();
    // Once the chosen bucket holds at most kSelCompact keys, they are gathered into LDS with
    // their positions and the remaining passes count only them, instead of re-reading every
    // score per pass. The same read marks the candidates above the bucket (kept whatever the
    // remaining passes decide), so the flags of the rest come from the gathered keys alone.
    bool compact = false;
    if (partial) {
        bool first = guessed;
        for (int top = sh.bits; top > 0; top -= 8) {
            const int shift = top >= 8 ? top - 8 : 0;
            const uint32_t dmask = top >= 8 ? 255u : ((1u << top) - 1u);
            sel_clear_hist(sh);
            const uint64_t prefix = sh.prefix, mask = sh.mask;
            if (compact) {
                const int nck = (int)s_nck;
                for (int i = tid; i < nck; i += kSelThreads) {
                    const uint64_t k = s_ck[i];
                    if ((k & mask) == prefix) sel_count(sh, k, shift, dmask);
                }
            } else {
                uint32_t above = 0u, match = 0u;
#pragma unroll 1
                for (int u0 = 0; u0 < KPT; u0 += kBatch) {
                    double v[kBatch];
#pragma unroll
                    for (int b = 0; b < kBatch; b++) {
                        const int t = 1 + tid + (u0 + b) * kSelThreads;
                        v[b] = t < c_end ? s[t] : 0.0;
                    }
#pragma unroll
                    for (int b = 0; b < kBatch; b++) {
                        const uint64_t k = order_key(v[b]);
                        if (1 + tid + (u0 + b) * kSelThreads < c_end) {
                            if ((k & mask) == prefix) {
                                sel_count(sh, k, shift, dmask);
                                match++;
                            } else if ((k & mask) > prefix) {
                                above++;
                            }
                        }
                    }
                }
                if (first) {
                    // the guessed range: candidates above it are kept, the m-th best must be in it
                    first = false;
                    atomicAdd(&s_above, above);
                    atomicAdd(&s_match, match);
                    __syncthreads();
                    if (tid == 0) {
                        const uint32_t a = s_above;
                        if (a < (uint32_t)m && (uint32_t)m - a <= s_match) sh.krem = m - (int)a;
                        else s_retry = 1;
                    }
                    __syncthreads();
                    if (s_retry) {
                        extremes_pass();
                        top = sh.bits + 8;   // start over below the true common prefix
                        continue;
                    }
                }
            }
            sel_pick_digit(sh, shift, dmask, prefix, mask);
            if (sh.all) break;
            if (!compact && shift > 0 && sh.bucket <= (uint32_t)kSelCompact) {
                const uint64_t p2 = sh.prefix, m2 = sh.mask;
                if (tid == 0) s_nck = 0u;
                __syncthreads();
                for (int w = 0; w < kWords; w++) {
                    uint32_t g1 = 0u;
#pragma unroll 1
                    for (int u0 = 0; u0 < 32; u0 += kBatch) {
                        double v[kBatch];
#pragma unroll
                        for (int b = 0; b < kBatch; b++) {
                            const int t = 1 + tid + (32 * w + u0 + b) * kSelThreads;
                            v[b] = t < c_end ? s[t] : 0.0;
                        }
#pragma unroll
                        for (int b = 0; b < kBatch; b++) {
                            const int t = 1 + tid + (32 * w + u0 + b) * kSelThreads;
                            if (t < c_end) {
                                const uint64_t k = order_key(v[b]);
                                if ((k & m2) > p2) {
                                    g1 |= 1u << (u0 + b);
                                } else if ((k & m2) == p2) {
                                    const uint32_t i = atomicAdd(&s_nck, 1u);
                                    s_ck[i] = k;
                                    s_cp[i] = t;
                                }
                            }
                        }
                    }
                    s_gt[w][tid] = g1;
                    s_eq[w][tid] = 0u;
                }
                __syncthreads();
                compact = true;
            }
        }
    }
    const uint64_t prefix = sh.prefix, mask = sh.mask;
    const int krem = sh.krem;
    const bool take_all_eq = sh.all != 0;
    const uint64_t below = (1ull << lane) - 1ull;
    // bit u of word u / 32: chunk u's candidate is above the selected key (gt) or equal (eq)
    // per-thread flag words in LDS ([word][thread]: conflict-free), so no register array is
    // indexed by a loop variable. After a compaction only the gathered keys are left to flag
    // (the candidate at position t is chunk (t - 1) / kSelThreads of thread (t - 1) %
    // kSelThreads).
    if (compact) {
        const int nck = (int)s_nck;
        for (int i = tid; i < nck; i += kSelThreads) {
            const uint64_t k = s_ck[i] & mask;
            const int t1 = s_cp[i] - 1, th = t1 % kSelThreads, u = t1 / kSelThreads;
            if (k > prefix) atomicOr(&s_gt[u >> 5][th], 1u << (u & 31));
            else if (k == prefix) atomicOr(&s_eq[u >> 5][th], 1u << (u & 31));
        }
        __syncthreads();
    }
    for (int w = 0; w < kWords && !compact; w++) {
        uint32_t g1 = 0u, e1 = 0u;
#pragma unroll 1
        for (int u0 = 0; u0 < 32; u0 += kBatch) {
            double v[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; b++) {
                const int t = 1 + tid + (32 * w + u0 + b) * kSelThreads;
                v[b] = (partial && t < c_end) ? s[t] : 0.0;
            }
#pragma unroll
            for (int b = 0; b < kBatch; b++) {
                const uint32_t f = 1u << (u0 + b);
                if (1 + tid + (32 * w + u0 + b) * kSelThreads < c_end) {
                    if (!partial) {
                        if (m > 0) g1 |= f;
                    } else {
                        const uint64_t k = order_key(v[b]) & mask;
                        if (k > prefix) g1 |= f;
                        else if (k == prefix) e1 |= f;
                    }
                }
            }
        }
        s_gt[w][tid] = g1;
        s_eq[w][tid] = e1;
    }
    // rank the ties in position order, keep the first krem of them (or all)
    if (partial && !take_all_eq) {
        for (int u = 0; u < KPT; u++) {
            const uint64_t b = __ballot((s_eq[u >> 5][tid] >> (u & 31)) & 1u);
            if (lane == 0) s_cnt[u * kWaves + wave] = (uint32_t)__popcll(b);
        }
        __syncthreads();
        scan_counts<kPer>(s_cnt, kCnt, sh.wave_sum);
        for (int w = 0; w < kWords; w++) {
            const uint32_t e1 = s_eq[w][tid];
            uint32_t add = 0u;
            for (int bb = 0; bb < 32; bb++) {
                const uint32_t bit = (e1 >> bb) & 1u;
                const uint64_t b = __ballot(bit);
                const uint32_t r = s_cnt[(32 * w + bb) * kWaves + wave] + (uint32_t)__popcll(b & below);
                if (bit && r < (uint32_t)krem) add |= 1u << bb;
            }
            s_gt[w][tid] |= add;
        }
        __syncthreads();
    } else {
        for (int w = 0; w < kWords; w++) s_gt[w][tid] |= s_eq[w][tid];
    }
    // output ranks of the kept candidates; BOS first, the window after the candidates
    for (int u = 0; u < KPT; u++) {
        const uint64_t b = __ballot((s_gt[u >> 5][tid] >> (u & 31)) & 1u);
        if (lane == 0) s_cnt[u * kWaves + wave] = (uint32_t)__popcll(b);
    }
    __syncthreads();
    const uint32_t kept = scan_counts<kPer>(s_cnt, kCnt, sh.wave_sum);
    for (int u = 0; u < KPT; u++) {
        const uint32_t bit = (s_gt[u >> 5][tid] >> (u & 31)) & 1u;
        const uint64_t b = __ballot(bit);
        if (bit) {
            const uint32_t o = 1u + s_cnt[u * kWaves + wave] + (uint32_t)__popcll(b & below);
            if (o < (uint32_t)n_keep) out[o] = 1 + tid + u * kSelThreads;
        }
    }
    if (tid == 0 && T > 0 && n_keep > 0) out[0] = 0;
    const int ws = c_end > 1 ? c_end : 1;               // first window position after BOS
    for (int t = ws + tid; t < T; t += kSelThreads) {
        const uint32_t o = 1u + kept + (uint32_t)(t - ws);
        if (o < (uint32_t)n_keep) out[o] = t;
    }
}

}  // namespace nq
