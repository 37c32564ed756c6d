// device_common.h -- device helpers shared by the step kernels (one copy per
// translation unit): candidate keys, element loads, reductions, block scan and
// the LDS radix select.
#pragma once

#include <math.h>

#include "internal.h"

namespace gr {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;  // fp32 nearest to log2(e)
constexpr double kLn2 = 0.693147180559945309417232121458;
constexpr float kFarBelow = -3.0e38f;  // finite start of the running log2 reference

__device__ __forceinline__ uint32_t ord_f32(float f) {
    const uint32_t b = __float_as_uint(f + 0.0f);  // -0 -> +0: they compare equal
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t k) {
    const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(b);
}

__device__ __forceinline__ uint64_t cand_key(uint32_t ord, uint32_t flat) {
    return ((uint64_t)ord << 32) | (uint32_t)(~flat);
}

__device__ __forceinline__ float ex2(float y) { return __builtin_amdgcn_exp2f(y); }

template <typename DT>
__device__ __forceinline__ float load_elem(const DT* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}

// ------------------------------------------------------------- reductions
//
// Wave-wide reductions on the DPP path: each step is a VALU lane move (no
// LDS round trip, unlike a shuffle).  GFX9 DPP controls: lanes i^1 and i^2
// (quad_perm [1,0,3,2] and [2,3,0,1]), the two quads of every 8 lanes (row
// half mirror), the two halves of every row of 16 (row mirror); then lane 15
// of rows 0 and 2 into rows 1 and 3 (row_bcast:15, row mask 0xA) and lane 31
// into rows 2 and 3 (row_bcast:31, row mask 0xC), which leaves the wave's
// result in lane 63, read out as a wave-uniform value.  Lanes that a masked
// move does not write take `idle`, the operation's identity.  Every lane of
// the wave must be active.
namespace dpp {
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;
}  // namespace dpp

template <int Ctrl, int RowMask, typename T>
__device__ __forceinline__ T dpp_move(T v, T idle) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, idle),
                                                                 __builtin_bit_cast(int, v), Ctrl, RowMask,
                                                                 0xF, false));
    } else {
        const uint64_t x = __builtin_bit_cast(uint64_t, v), y = __builtin_bit_cast(uint64_t, idle);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)y, (int)(uint32_t)x, Ctrl,
                                                                  RowMask, 0xF, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(y >> 32),
                                                                  (int)(uint32_t)(x >> 32), Ctrl, RowMask,
                                                                  0xF, false);
        return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    }
}

template <typename T>
__device__ __forceinline__ T read_lane(T v, int lane) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
    } else {
        const uint64_t x = __builtin_bit_cast(uint64_t, v);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
        return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    }
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, T idle, Op op) {
    v = op(v, dpp_move<dpp::kXor1, 0xF>(v, idle));
    v = op(v, dpp_move<dpp::kXor2, 0xF>(v, idle));
    v = op(v, dpp_move<dpp::kHalfMirror, 0xF>(v, idle));
    v = op(v, dpp_move<dpp::kMirror, 0xF>(v, idle));
    v = op(v, dpp_move<dpp::kBcast15, 0xA>(v, idle));
    v = op(v, dpp_move<dpp::kBcast31, 0xC>(v, idle));
    return read_lane(v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, -INFINITY, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ double wave_sum(double v) {
    return wave_reduce(v, 0.0, [](double x, double y) { return x + y; });
}
__device__ __forceinline__ long long wave_sum_ll(long long v) {
    return wave_reduce(v, 0ll, [](long long x, long long y) { return x + y; });
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    return wave_reduce(v, (uint64_t)0, [](uint64_t x, uint64_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
    return wave_reduce(v, ~(uint64_t)0, [](uint64_t x, uint64_t y) { return x < y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce(v, ~0u, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}

// Inclusive prefix sum over the wave's lanes: shifts by 1, 2, 4 and 8
// within each row of 16 (lanes without a source add 0), then the row totals
// forward by row_bcast:15 and row_bcast:31.  Every lane must be active.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    v += dpp_move<0x111, 0xF>(v, 0u);  // row_shr:1
    v += dpp_move<0x112, 0xF>(v, 0u);  // row_shr:2
    v += dpp_move<0x114, 0xF>(v, 0u);  // row_shr:4
    v += dpp_move<0x118, 0xF>(v, 0u);  // row_shr:8
    v += dpp_move<dpp::kBcast15, 0xA>(v, 0u);
    v += dpp_move<dpp::kBcast31, 0xC>(v, 0u);
    return v;
}

// Lanes below this one whose bit is set in the wave mask m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide reductions; every thread gets the result.  `sh` holds one
// entry per wave and is reused, so each call starts with a barrier.
template <int NT>
__device__ float block_max(float v, float* sh) {
    v = wave_max(v);
    if constexpr (NT == 64) return v;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, sh[i]);
    return r;
}
template <int NT>
__device__ double block_sum(double v, double* sh) {
    v = wave_sum(v);
    if constexpr (NT == 64) return v;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) r += sh[i];
    return r;
}
template <int NT>
__device__ long long block_sum_ll(long long v, long long* sh) {
    v = wave_sum_ll(v);
    if constexpr (NT == 64) return v;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    long long r = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) r += sh[i];
    return r;
}

// The s-th largest (ties counted) of the wave's values v[0..E) per lane
// (0 = none), or 0 when fewer than s are nonzero (s >= 1): a bitwise search
// for the largest h with at least s values >= h, one compare and ballot
// count per value and bit.  As soon as exactly s values reach the candidate,
// the answer is the least of them (one wave minimum) and the search stops.
// Every lane must be active.
template <int E>
__device__ uint32_t wave_kth_u32(const uint32_t* v, int s) {
    uint32_t h = 0;
#pragma unroll 4
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = h | (1u << bit);
        int n = 0;
#pragma unroll
        for (int q = 0; q < E; ++q) n += __popcll(__ballot(v[q] >= c));
        if (n >= s) {
            h = c;
            if (n == s) {
                uint32_t m = ~0u;
#pragma unroll
                for (int q = 0; q < E; ++q) m = v[q] >= c && v[q] < m ? v[q] : m;
                return wave_min_u32(m);
            }
        }
    }
    return h;
}

// The s-th largest of the wave's keys k[0..E) per lane (unique, 0 = none),
// or 0 when the wave holds fewer than s (s >= 1): the s-th largest score half
// h (above), then among the keys whose score half is h the index half the
// same way -- or, when all of them are needed, their smallest index half
// (one wave minimum).  Every lane must be active.
template <int E>
__device__ uint64_t wave_kth_key(const uint64_t* k, int s) {
    uint32_t hi[E], lo[E];
#pragma unroll
    for (int q = 0; q < E; ++q) {
        hi[q] = (uint32_t)(k[q] >> 32);
        lo[q] = (uint32_t)k[q];
    }
    auto count_ge = [&](uint32_t c) {
        int n = 0;
#pragma unroll
        for (int q = 0; q < E; ++q) n += __popcll(__ballot(hi[q] >= c));
        return n;
    };
    // a key's score half is never 0 (the order bits of a finite or -inf fp32)
    const uint32_t h = wave_kth_u32<E>(hi, s);
    if (h == 0) return 0;
    const int need = s - (h == ~0u ? 0 : count_ge(h + 1));  // >= 1
    int eq = 0;
#pragma unroll
    for (int q = 0; q < E; ++q) eq += __popcll(__ballot(hi[q] == h));
    uint32_t l = 0;
    if (eq == need) {
        uint32_t m = ~0u;
#pragma unroll
        for (int q = 0; q < E; ++q) m = hi[q] == h && lo[q] < m ? lo[q] : m;
        l = wave_min_u32(m);
    } else {
#pragma unroll 1  // (an early exit and ballots: the compiler keeps it rolled)
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = l | (1u << bit);
            int n = 0;
#pragma unroll
            for (int q = 0; q < E; ++q) n += __popcll(__ballot(hi[q] == h && lo[q] >= c));
            if (n >= need) {
                l = c;
                if (n == need) {  // exactly `need` reach c: the least of them
                    uint32_t m = ~0u;
#pragma unroll
                    for (int q = 0; q < E; ++q) m = hi[q] == h && lo[q] >= c && lo[q] < m ? lo[q] : m;
                    l = wave_min_u32(m);
                    break;
                }
            }
        }
    }
    return ((uint64_t)h << 32) | l;
}

// ------------------------------------------------------------- sampling

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011) of one counter block c[0..3] under key (k0, k1),
// in place: ten rounds, each multiplying c0 and c2 by 0xD2511F53 and
// 0xCD9E8D57 into 64-bit products whose high words are xored with the other
// counter words and the key; the key gains 0x9E3779B9 / 0xBB67AE85 before
// every round after the first.
__device__ __forceinline__ void philox4x32_10(uint32_t* c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // each 32 x 32 -> 64-bit product in one multiply (both halves)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        const uint32_t y0 = hi1 ^ c[1] ^ k0, y2 = hi0 ^ c[3] ^ k1;
        c[0] = y0;
        c[1] = lo1;
        c[2] = y2;
        c[3] = lo0;
    }
}

// The standard Gumbel variate of one Philox word r: u = (r + 1/2) 2^-32,
// g = -log(-log(u)) in fp64, rounded to fp32.
__device__ __forceinline__ float gumbel_of_word(uint32_t r) {
    const double u = ((double)r + 0.5) * 0x1p-32;
    return (float)(-log(-log(u)));
}

// The standard Gumbel variate of candidate `flat` (= parent slot * V + token)
// of request b at step t: word flat mod 4 of the Philox block at counter
// (flat / 4, b, t, 0) and key (seed low, seed high), u = (r + 1/2) 2^-32,
// g = -log(-log(u)) in fp64, rounded to fp32.  Out of line: inlined into
// the candidate loops, its fp64 temporaries would push the loops' live
// values to scratch even when nothing is sampled.
__device__ __attribute__((noinline)) float gumbel_noise(uint64_t seed, int b, int t, uint32_t flat) {
    uint32_t c[4] = {flat >> 2, (uint32_t)b, (uint32_t)t, 0u};
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const uint32_t w = flat & 3u;
    return gumbel_of_word(w == 0 ? c[0] : (w == 1 ? c[1] : (w == 2 ? c[2] : c[3])));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The Gumbel variates (as gumbel_noise) of the four consecutive candidates
// flat0 .. flat0+3 of request b at step t: they share one Philox block, or
// two when the run straddles a block boundary.  Out of line for the same
// reason as gumbel_noise.
__device__ __attribute__((noinline)) f32x4 gumbel_run4(uint64_t seed, int b, int t, uint32_t flat0) {
    uint32_t c0[4] = {flat0 >> 2, (uint32_t)b, (uint32_t)t, 0u};
    uint32_t c1[4] = {(flat0 >> 2) + 1u, (uint32_t)b, (uint32_t)t, 0u};
    philox4x32_10(c0, (uint32_t)seed, (uint32_t)(seed >> 32));
    if (flat0 & 3u) philox4x32_10(c1, (uint32_t)seed, (uint32_t)(seed >> 32));
    f32x4 g;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w = (flat0 & 3u) + (uint32_t)q;  // word of the run's first block, or of the next
        const uint32_t r = w < 4 ? (w == 0 ? c0[0] : w == 1 ? c0[1] : w == 2 ? c0[2] : c0[3])
                                 : (w == 4 ? c1[0] : w == 5 ? c1[1] : c1[2]);
        g[q] = gumbel_of_word(r);
    }
    return g;
}

// Fast estimates of the same variates, for bounds only.  From Philox word r:
// L = -ln u comes from u itself, or, where u lies within 2^-6 of one, from
// the series w + w^2/2 + w^3/3 + w^4/4 in w = 1 - u (relative error below
// 2^-26 there), so that L keeps its relative accuracy as it tends to zero;
// then g = -ln L.  Both logarithms are the hardware base-2 logarithm in fp32.
// |gumbel_fast(r) - exact variate| <= kDrawErr for every r (gr_probe_draw_error
// measures all 2^32 words); the estimates never rank a candidate, they only
// bound which candidates can rank among a row's best.
constexpr float kDrawErr = 0x1p-12f;

__device__ __forceinline__ float gumbel_fast(uint32_t r) {
    constexpr float ln2 = 0.693147182f;
    const float u = fmaf((float)r, 0x1p-32f, 0x1p-33f);
    const float w = fmaf((float)~r, 0x1p-32f, 0x1p-33f);  // 1 - u
    const float ls = w * fmaf(w, fmaf(w, fmaf(w, 0.25f, 0.333333343f), 0.5f), 1.0f);
    const float L = w < 0x1p-6f ? ls : -__builtin_amdgcn_logf(u) * ln2;
    return -__builtin_amdgcn_logf(L) * ln2;
}

// The Philox block of request b, step t at counter word blk: four words.
__device__ __forceinline__ void philox_block(uint64_t seed, int b, int t, uint32_t blk, uint32_t* w) {
    w[0] = blk;
    w[1] = (uint32_t)b;
    w[2] = (uint32_t)t;
    w[3] = 0u;
    philox4x32_10(w, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Fast estimates of the N consecutive candidates flat0 .. flat0+N-1 (N a
// multiple of 4): N/4 Philox blocks, one more when flat0 is not a multiple
// of 4.  The misaligned run picks its words with masks (flat0 mod 4 is the
// same for every vector of a row: a select chain on it would become branches).
template <int N>
__device__ __forceinline__ void gumbel_fast_run(uint64_t seed, int b, int t, uint32_t flat0, float* g) {
    static_assert(N % 4 == 0, "runs of whole blocks");
    const uint32_t sh = flat0 & 3u;
    uint32_t w[N + 4];
#pragma unroll
    for (int k = 0; k < N / 4; ++k) philox_block(seed, b, t, (flat0 >> 2) + (uint32_t)k, w + 4 * k);
    if (sh == 0) {
#pragma unroll
        for (int q = 0; q < N; ++q) g[q] = gumbel_fast(w[q]);
        return;
    }
    philox_block(seed, b, t, (flat0 >> 2) + (uint32_t)(N / 4), w + N);
    const uint32_t m1 = sh == 1 ? ~0u : 0u, m2 = sh == 2 ? ~0u : 0u, m3 = sh == 3 ? ~0u : 0u;
#pragma unroll
    for (int q = 0; q < N; ++q) g[q] = gumbel_fast((w[q + 1] & m1) | (w[q + 2] & m2) | (w[q + 3] & m3));
}

__device__ __forceinline__ float gumbel_fast_one(uint64_t seed, int b, int t, uint32_t flat) {
    uint32_t w[4];
    philox_block(seed, b, t, flat >> 2, w);
    const uint32_t q = flat & 3u;
    return gumbel_fast(q == 0 ? w[0] : q == 1 ? w[1] : q == 2 ? w[2] : w[3]);
}

// ------------------------------------------------------- LDS bitonic sort

// Sort the P 64-bit keys v[0..P) in LDS in place (P a power of two),
// descending when Desc, else ascending, with a bitonic network: log2(P)
// (log2(P) + 1) / 2 stages of P/2 compare-exchanges, one barrier after each.
// Every thread of the workgroup calls it once v is complete (after a
// barrier); it ends with a barrier.
template <int NT, bool Desc>
__device__ void block_bitonic_sort(uint64_t* v, int P) {
    for (int k = 2; k <= P; k <<= 1) {
        for (int h = k >> 1; h > 0; h >>= 1) {
            for (int i = threadIdx.x; i < P / 2; i += NT) {
                const int lo = ((i & ~(h - 1)) << 1) | (i & (h - 1));  // the pair (lo, lo + h)
                const uint64_t x = v[lo], y = v[lo + h];
                // runs of length k alternate direction; the last run (k = P) is the result
                if ((Desc ? x < y : x > y) == ((lo & k) == 0)) {
                    v[lo] = y;
                    v[lo + h] = x;
                }
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------ wave-aggregated atomics

// A slot from the LDS counter *ctr for every active lane with pred: one
// atomic per wave instead of one per lane (same-address LDS atomics
// serialise).  Returns -1 where !pred.
__device__ __forceinline__ int wave_claim(int* ctr, bool pred) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return -1;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((unsigned long long)m) - 1;
    int base = 0;
    if (lane == leader) base = atomicAdd(ctr, __popcll(m));
    base = __builtin_amdgcn_readlane(base, leader);
    return pred ? base + lanes_below(m) : -1;
}

// hist[d] += 1 from every active lane; the lanes sharing the first active
// lane's digit add together (the common case in the top digits of keys whose
// scores lie close together).
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t d) {
    const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
    const uint64_t m = __ballot(d == d0);
    if (d == d0) {
        if ((int)(threadIdx.x & 63) == __ffsll((unsigned long long)m) - 1)
            atomicAdd(&hist[d0], (uint32_t)__popcll(m));
    } else {
        atomicAdd(&hist[d], 1u);
    }
}

// Three block-wide sums at once (one exchange), left in out[0..2] of LDS for
// every thread to read after the closing barrier.  sh holds 3 entries per
// wave.  (Returning the sums in registers lets the compiler defer the
// additions to the sums' last use and keep every wave's partial live.)
template <int NT>
__device__ void block_sum3_ll(long long x, long long y, long long z, long long* sh, long long* out) {
    x = wave_sum_ll(x);
    y = wave_sum_ll(y);
    z = wave_sum_ll(z);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        const int w = threadIdx.x >> 6;
        sh[3 * w] = x;
        sh[3 * w + 1] = y;
        sh[3 * w + 2] = z;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        long long a = 0, b = 0, c = 0;
        for (int i = 0; i < NT / 64; ++i) {
            a += sh[3 * i];
            b += sh[3 * i + 1];
            c += sh[3 * i + 2];
        }
        out[0] = a;
        out[1] = b;
        out[2] = c;
    }
    __syncthreads();
}

// ---------------------------------------------------------- radix select
//
// Threshold of the `need` largest keys (32 or 64 bits) among those visited
// by for_each (every thread visits its share).  MSB-first, 8-bit digits:
// each pass histograms the next digit of the keys that share the prefix
// fixed so far, wave 0 finds the digit bin holding the need-th largest, and
// the pass ends early once that bin holds exactly the keys still needed.
// Returns P <= the need-th largest key with at least `need` keys >= P
// (exactly `need` when keys are unique), or 0 -- every key -- when fewer
// than `need` keys are visited.  Requires need >= 1.  Uses hist[256] and
// misc[0..2].  Stopping after the digit at bit
// min_shift (a multiple of 8) returns that prefix with the lower bits zero:
// still a value <= the need-th largest with at least `need` keys >= it.
template <int NT, typename KeyT = uint64_t, typename ForEach>
__device__ KeyT radix_threshold(ForEach for_each, uint32_t need, uint32_t* hist, int* misc, int min_shift = 0) {
    const int tid = threadIdx.x;
    KeyT prefix = 0, mask = 0;
    for (int shift = 8 * (int)sizeof(KeyT) - 8; shift >= min_shift; shift -= 8) {
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        if (tid == 0) misc[0] = -1;  // stays -1 when no bin holds the need-th key
        __syncthreads();
        for_each([&](KeyT k) {
            if ((k & mask) == prefix) hist_add(hist, (uint32_t)(k >> shift) & 255u);
        });
        __syncthreads();
        if (tid < 64) {
            // lane l owns bins 255-4l .. 252-4l (descending)
            const uint32_t h0 = hist[255 - 4 * tid], h1 = hist[254 - 4 * tid];
            const uint32_t h2 = hist[253 - 4 * tid], h3 = hist[252 - 4 * tid];
            const uint32_t loc = h0 + h1 + h2 + h3;
            const uint32_t inc = wave_inclusive_scan(loc);
            const uint32_t exc = inc - loc;
            if (exc < need && need <= inc) {
                uint32_t acc = exc;
                int d;
                uint32_t hd;
                if (acc + h0 >= need) {
                    d = 255 - 4 * tid; hd = h0;
                } else {
                    acc += h0;
                    if (acc + h1 >= need) {
                        d = 254 - 4 * tid; hd = h1;
                    } else {
                        acc += h1;
                        if (acc + h2 >= need) {
                            d = 253 - 4 * tid; hd = h2;
                        } else {
                            acc += h2; d = 252 - 4 * tid; hd = h3;
                        }
                    }
                }
                misc[0] = d;
                misc[1] = (int)acc;
                misc[2] = (int)hd;
            }
        }
        __syncthreads();
        if (misc[0] < 0) {  // fewer than `need` keys (first pass only: later ones count a found bin's keys)
            __syncthreads();
            return 0;
        }
        const uint32_t d = (uint32_t)misc[0], above = (uint32_t)misc[1], hd = (uint32_t)misc[2];
        need -= above;
        prefix |= (KeyT)d << shift;
        mask |= (KeyT)0xFF << shift;
        __syncthreads();  // misc and hist are rewritten next
        if (hd == need) break;
    }
    return prefix;
}

// Keep only the keys >= th of buf[0..n) (n <= NT * PER), packed at the
// front; returns how many (every thread gets it).  Ends with a barrier.
template <int NT, int PER>
__device__ __forceinline__ int compact_ge(uint64_t* buf, int n, uint64_t th, int* ctr) {
    const int tid = threadIdx.x;
    uint64_t r[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int i = tid + q * NT;
        r[q] = i < n ? buf[i] : 0ull;
    }
    if (tid == 0) *ctr = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (q * NT < n) {  // (the same for every thread)
            const bool keep = r[q] != 0ull && r[q] >= th;
            const int p = wave_claim(ctr, keep);
            if (keep) buf[p] = r[q];
        }
    }
    __syncthreads();
    const int m = *ctr;
    __syncthreads();
    return m;
}

// A cut P for the K best of the n > K keys of buf: P is at most the K-th
// largest key and at least K keys are >= P (the K-th key's bucket mates
// come too: *kept of them in all).  The keys' range [min, max] is split
// into 256 buckets of 2^sh keys; P is the lower edge of the bucket that
// holds the K-th largest.  One counting pass where a radix select takes
// several.  Uses hist[256], misc[0..1] and wmm[0 .. 2 * NT / 64); ends with a
// barrier.
template <int NT>
__device__ __forceinline__ uint64_t bucket_cut(const uint64_t* buf, int n, int K, uint32_t* hist, int* misc, uint64_t* wmm,
                               int* kept) {
    const int tid = threadIdx.x;
    uint64_t lo = ~0ull, hi = 0ull;
    for (int i = tid; i < n; i += NT) {
        const uint64_t k = buf[i];
        lo = k < lo ? k : lo;
        hi = k > hi ? k : hi;
    }
    lo = wave_min_u64(lo);
    hi = wave_max_u64(hi);
    if ((tid & 63) == 0) {
        wmm[2 * (tid >> 6)] = lo;
        wmm[2 * (tid >> 6) + 1] = hi;
    }
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    lo = wmm[0];
    hi = wmm[1];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
        lo = wmm[2 * w] < lo ? wmm[2 * w] : lo;
        hi = wmm[2 * w + 1] > hi ? wmm[2 * w + 1] : hi;
    }
    const uint64_t span = hi - lo;
    const int sh = span < 256 ? 0 : 56 - __clzll((long long)span);  // (span >> sh) < 256
    for (int i = tid; i < n; i += NT) hist_add(hist, (uint32_t)((buf[i] - lo) >> sh));
    __syncthreads();
    if (tid < 64) {  // lane l owns buckets 255-4l .. 252-4l (descending)
        const uint32_t h0 = hist[255 - 4 * tid], h1 = hist[254 - 4 * tid];
        const uint32_t h2 = hist[253 - 4 * tid], h3 = hist[252 - 4 * tid];
        const uint32_t loc = h0 + h1 + h2 + h3;
        const uint32_t inc = wave_inclusive_scan(loc);
        const uint32_t exc = inc - loc, need = (uint32_t)K;
        if (exc < need && need <= inc) {
            int d = 252 - 4 * tid;
            if (exc + h0 >= need) d = 255 - 4 * tid;
            else if (exc + h0 + h1 >= need) d = 254 - 4 * tid;
            else if (exc + h0 + h1 + h2 >= need) d = 253 - 4 * tid;
            misc[0] = d;
            misc[1] = (int)(exc + (d == 255 - 4 * tid   ? h0
                                   : d == 254 - 4 * tid ? h0 + h1
                                   : d == 253 - 4 * tid ? h0 + h1 + h2
                                                        : loc));
        }
    }
    __syncthreads();
    const uint64_t cut = lo + ((uint64_t)misc[0] << sh);
    *kept = misc[1];
    __syncthreads();  // (misc and hist are reused)
    return cut;
}

// Ranks, best first, of the n <= Q * NT unique keys of a[0..n): thread tid
// holds key[q] = a[tid + q * NT] (any value past n), read before the call.
// The keys are bucketed by (key - min) >> sh into 256 buckets over their
// range (a monotone map), counted, scanned and scattered back into a in
// bucket order; then thread tid takes the keys at positions tid + q * NT of
// that order: key[q] becomes that key (0 past n), at(q, key[q]) is called
// for it (say, to issue its loads), and rk[q] gets its rank: the number of
// keys in higher buckets plus the greater ones in its own bucket (-1 past
// n).  The lanes of a wave then count in the same one or two buckets:
// their LDS reads coincide and their loops run alike.  A few barriers,
// where counting every pair costs n^2 LDS reads and a sorting network a
// barrier per stage.  Uses hist[256], cur[256] and wmm[0 .. 2 * NT / 64);
// rewrites a[0..n); ends with a barrier.
template <int NT, int Q, typename At>
__device__ __forceinline__ void bucket_ranks(uint64_t* a, int n, uint64_t* key, int* rk, uint32_t* hist, int* cur,
                                             uint64_t* wmm, At&& at) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x;
    uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
    for (int q = 0; q < Q; ++q)
        if (tid + q * NT < n) {
            kmin = key[q] < kmin ? key[q] : kmin;
            kmax = key[q] > kmax ? key[q] : kmax;
        }
    kmin = wave_min_u64(kmin);
    kmax = wave_max_u64(kmax);
    if ((tid & 63) == 0) {
        wmm[2 * (tid >> 6)] = kmin;
        wmm[2 * (tid >> 6) + 1] = kmax;
    }
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();  // (the caller's reads of a are done: it is rewritten below)
    kmin = wmm[0];
    kmax = wmm[1];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        kmin = wmm[2 * w] < kmin ? wmm[2 * w] : kmin;
        kmax = wmm[2 * w + 1] > kmax ? wmm[2 * w + 1] : kmax;
    }
    const uint64_t span = kmax - kmin;
    const int sh = span < 256 ? 0 : 56 - __clzll((long long)span);  // (span >> sh) < 256
    int bk[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        bk[q] = (int)((key[q] - kmin) >> sh);
        if (tid + q * NT < n) atomicAdd(&hist[bk[q]], 1u);
    }
    __syncthreads();
    if (tid < 64) {  // bucket starts: an inclusive scan, lane l holding buckets 4l .. 4l+3
        const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2], h3 = hist[4 * tid + 3];
        const uint32_t inc = wave_inclusive_scan(h0 + h1 + h2 + h3);
        const uint32_t e0 = inc - (h0 + h1 + h2 + h3);
        cur[4 * tid] = (int)e0;
        cur[4 * tid + 1] = (int)(e0 + h0);
        cur[4 * tid + 2] = (int)(e0 + h0 + h1);
        cur[4 * tid + 3] = (int)(e0 + h0 + h1 + h2);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < Q; ++q)
        if (tid + q * NT < n) a[atomicAdd(&cur[bk[q]], 1)] = key[q];
    __syncthreads();  // cur[] now holds each bucket's end
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int p = tid + q * NT;
        key[q] = p < n ? a[p] : 0ull;
        if (p < n) at(q, key[q]);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        rk[q] = -1;
        if (tid + q * NT < n) {
            const int bq = (int)((key[q] - kmin) >> sh);
            const int end = cur[bq];
            int m = end - (int)hist[bq], r = n - end;
            for (; m + 3 < end; m += 4)  // four independent LDS reads per round
                r += (a[m] > key[q] ? 1 : 0) + (a[m + 1] > key[q] ? 1 : 0) + (a[m + 2] > key[q] ? 1 : 0) +
                     (a[m + 3] > key[q] ? 1 : 0);
            for (; m < end; ++m) r += a[m] > key[q] ? 1 : 0;
            rk[q] = r;
        }
    }
    __syncthreads();  // (hist, cur and a are free again)
}

// Exclusive prefix sum of arr[0..n) in place (LDS), arr[n] = total; returns
// the total to every thread.  wsum holds one int per wave.  Each thread scans
// a contiguous range, which other threads may have written: the first barrier
// orders those writes before the reads.
template <int NT>
__device__ int block_exclusive_scan(int* arr, int n, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    __syncthreads();
    const int per = (n + NT - 1) / NT;
    const int beg = tid * per;
    const int end = beg + per < n ? beg + per : n;
    int local = 0;
    for (int i = beg; i < end; ++i) local += arr[i];
    const int inc = (int)wave_inclusive_scan((uint32_t)local);
    __syncthreads();
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int wpre = 0, total = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        wpre += i < w ? wsum[i] : 0;
        total += wsum[i];
    }
    int run = wpre + inc - local;
    for (int i = beg; i < end; ++i) {
        const int v = arr[i];
        arr[i] = run;
        run += v;
    }
    __syncthreads();
    if (tid == 0) arr[n] = total;
    __syncthreads();
    return total;
}

}  // namespace
}  // namespace gr
