// row_stream.h -- streaming one row of logits and its log-sum-exp, shared by
// the row kernel and the fused short-row step kernel (one copy per
// translation unit, like device_common.h).
#pragma once

#include <type_traits>

#include "device_common.h"

namespace gr {
namespace {

// Unpack one 16-byte vector into VEC fp32 values (bf16 widened exactly).
template <typename DT>
__device__ __forceinline__ void unpack(const u32x4& w, float* x) {
    if constexpr (sizeof(DT) == 4) {
        x[0] = __uint_as_float(w.x);
        x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z);
        x[3] = __uint_as_float(w.w);
    } else {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            x[2 * q] = __uint_as_float(ws[q] << 16);
            x[2 * q + 1] = __uint_as_float(ws[q] & 0xFFFF0000u);
        }
    }
}

// Fold n values into the running (max mx, log2 reference Rr, sum s): one max
// and at most one rescale per call, then s += sum 2^(x*sc - Rr), sc = log2(e)
// over the temperature.
template <int N>
__device__ __forceinline__ float fold(const float* x, float& mx, float& Rr, float& s, float sc) {
    static_assert((N & (N - 1)) == 0, "fold sums a power-of-two count");
    float vm = x[0];
#pragma unroll
    for (int q = 1; q < N; ++q) vm = fmaxf(vm, x[q]);
    if (vm > mx) {
        const float nr = vm * sc;
        s *= ex2(Rr - nr);
        Rr = nr;
        mx = vm;
    }
    const float nR = -Rr;
    float e[N];
#pragma unroll
    for (int q = 0; q < N; ++q) e[q] = ex2(fmaf(x[q], sc, nR));
#pragma unroll
    for (int h = N / 2; h > 0; h >>= 1) {
#pragma unroll
        for (int r = 0; r < h; ++r) e[r] += e[r + h];
    }
    s += e[0];
    return vm;
}

// Stream one row: every thread (tid in [0, NT): its index among the NT
// threads sharing the row) folds its share of the V logits into
// (Rr, s).  Full batches of U vectors per thread are loaded unconditionally
// and software-pipelined -- the next batch is in flight while the current
// one is folded -- then the remaining vectors and the unaligned head and tail
// elements are folded one by one.  early() runs once the first batch is in
// flight: loads it issues overlap the rest of the stream.  EarlyRest: the
// row has at most one full batch per thread (nfull <= 1), and the rest is
// loaded with it.
// Mode kBound: also count the -inf logits (ninf), leave the thread's maximum
// in tmax and the maximum of each of its batches in gmax[k*NT + tid] (batch
// nfull = the remaining vectors; the head and tail elements belong to none).
// Mode kDrawn: the same for the estimates y = x q + g~ in place of the
// logits x (g~ = gumbel_fast of the element's Philox word), and the range
// [xlo, xhi] of the thread's finite logits in the DrawCtx.
enum StreamMode { kPlain = 0, kBound = 1, kDrawn = 2 };

struct DrawCtx {
    uint64_t seed;
    int b, t;
    uint32_t flat0;  // flat index j*V + v of the row's first streamed token
    float q;         // 1/T, over the live length penalty when it applies
    float xlo, xhi;
};

// 16-byte vectors per stream batch of a one-wave (short) row, the same in
// the row kernel and the fused step so that both fold a row alike (bf16:
// two, so that the 32 unpacked values of a batch fit the fused kernel's
// registers)
template <typename DT>
constexpr int short_row_batch() {
    return sizeof(DT) == 2 ? 2 : kStreamBatch;
}

template <typename DT>
__device__ __forceinline__ int row_head(const DT* row, int V) {
    const int h = (int)(((16u - (uint32_t)((uintptr_t)row & 15u)) & 15u) / sizeof(DT));
    return h < V ? h : V;
}

template <typename DT, int NT, int U, int Mode, bool EarlyRest = false, typename Early>
__device__ __forceinline__ void stream_row(const DT* row, int V, int tid, float sc, float& Rr, float& s,
                                           Early&& early, float* gmax, int& ninf, float& tmax,
                                           DrawCtx& dc) {
    constexpr int VEC = 16 / (int)sizeof(DT);
    float mx = -INFINITY, ymax = -INFINITY;
    Rr = kFarBelow;
    s = 0.0f;
    auto count_inf = [&](const float* x, int n) {
        if constexpr (Mode != kPlain)
            for (int q = 0; q < n; ++q) ninf += x[q] == -INFINITY ? 1 : 0;
    };
    // estimates of n consecutive elements (flat0 .. flat0 + n - 1): their maximum
    auto draw_max = [&](const float* x, const float* g, int n) {
        float ym = -INFINITY;
        for (int q = 0; q < n; ++q) {
            ym = fmaxf(ym, __fadd_rn(__fmul_rn(x[q], dc.q), g[q]));
            dc.xlo = fminf(dc.xlo, x[q] == -INFINITY ? dc.xlo : x[q]);
        }
        return ym;
    };
    auto one = [&](int64_t i) {  // a head or tail element
        const float x = load_elem<DT>(row, i);
        count_inf(&x, 1);
        fold<1>(&x, mx, Rr, s, sc);
        if constexpr (Mode == kDrawn) {
            const float g = gumbel_fast_one(dc.seed, dc.b, dc.t, dc.flat0 + (uint32_t)i);
            ymax = fmaxf(ymax, draw_max(&x, &g, 1));
        }
    };
    const int head = row_head(row, V);
    if (tid < head) one(tid);
    const int64_t nvec = (int64_t)(V - head) / VEC;
    const u32x4* vp = reinterpret_cast<const u32x4*>(row + head);
    constexpr int64_t per = (int64_t)U * NT;
    const int64_t nfull = nvec / per;
    auto load_batch = [&](int64_t k, u32x4* w) {
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = __builtin_nontemporal_load(vp + k * per + u * NT + tid);
    };
    // fold n vectors; their first is vector v0, the next ones NT apart
    // (drawn: vector by vector, so that only one vector's values and draws
    // are live at a time)
    auto fold_vecs = [&](const u32x4* w, int64_t v0, auto n_c) {
        constexpr int N = decltype(n_c)::value;
        if constexpr (Mode == kDrawn) {
            float vm = -INFINITY;
#pragma unroll
            for (int u = 0; u < N; ++u) {
                float x[VEC], g[VEC];
                unpack<DT>(w[u], x);
                count_inf(x, VEC);
                fold<VEC>(x, mx, Rr, s, sc);
                gumbel_fast_run<VEC>(dc.seed, dc.b, dc.t,
                                     dc.flat0 + (uint32_t)head + (uint32_t)((v0 + (int64_t)u * NT) * VEC), g);
                vm = fmaxf(vm, draw_max(x, g, VEC));
            }
            ymax = fmaxf(ymax, vm);
            return vm;
        } else {
            float x[N * VEC];
#pragma unroll
            for (int u = 0; u < N; ++u) unpack<DT>(w[u], x + u * VEC);
            count_inf(x, N * VEC);
            return fold<N * VEC>(x, mx, Rr, s, sc);
        }
    };
    auto fold_batch = [&](const u32x4* w, int64_t k) {
        const float vm = fold_vecs(w, k * per + tid, std::integral_constant<int, U>{});
        if constexpr (Mode != kPlain) gmax[k * NT + tid] = vm;
    };
    float rmax = -INFINITY;
    if constexpr (EarlyRest) {
        // a row of at most one batch and the rest (the caller guarantees
        // nfull <= 1): the rest's loads are issued with the batch, before it
        // is folded -- the whole row costs one round trip; the folds run in
        // the same order as below
        static_assert(Mode == kPlain, "early rest loads: plain rows");
        u32x4 wa[U], w[U];
        int64_t vi[U];
        auto load_rest = [&] {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                vi[u] = nfull * per + (int64_t)u * NT + tid;
                if (vi[u] < nvec) w[u] = __builtin_nontemporal_load(vp + vi[u]);
            }
        };
        if (nfull == 0) {
            load_rest();
            early();
        } else {
            load_batch(0, wa);
            early();
            load_rest();
            fold_batch(wa, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (vi[u] < nvec) fold_vecs(&w[u], vi[u], std::integral_constant<int, 1>{});
    } else {
        if (nfull > 0) {
            u32x4 wa[U], wb[U];
            load_batch(0, wa);
            early();
            int64_t k = 1;
            for (; k + 1 < nfull; k += 2) {
                load_batch(k, wb);
                fold_batch(wa, k - 1);
                load_batch(k + 1, wa);
                fold_batch(wb, k);
            }
            if (k < nfull) {
                load_batch(k, wb);
                fold_batch(wa, k - 1);
                fold_batch(wb, k);
            } else {
                fold_batch(wa, k - 1);
            }
        } else {
            early();
        }
        // the remaining vectors (fewer than a batch per thread): all of a
        // thread's loads are issued before any is folded -- one round trip,
        // not one per vector
        u32x4 w[U];
        int64_t vi[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vi[u] = nfull * per + (int64_t)u * NT + tid;
            if (vi[u] < nvec) w[u] = __builtin_nontemporal_load(vp + vi[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (vi[u] < nvec) rmax = fmaxf(rmax, fold_vecs(&w[u], vi[u], std::integral_constant<int, 1>{}));
    }
    if constexpr (Mode != kPlain)
        if (nvec > nfull * per) gmax[nfull * NT + tid] = rmax;
    const int64_t tail0 = head + nvec * VEC;
    if (tail0 + tid < V) one(tail0 + tid);
    tmax = Mode == kDrawn ? ymax : mx;
    dc.xhi = mx;
}

// Row normaliser from every thread's (Rr, s), s = sum of 2^(x*log2e - Rr)
// over the thread's elements: each wave combines in fp64 by shuffles, the
// waves through LDS (one barrier); lse = ln2 * (R + log2 S), rounded once.
// s 2^(Rr - Rw) in fp64, and (R + log2 S) ln 2 rounded to fp32, out of line:
// called from a loop over rows, the fp64 routines' constants would otherwise
// be hoisted into the loop's registers (the same arithmetic as inline)
__device__ __attribute__((noinline)) double rescale_part_ool(float s, float Rr, float Rw) {
    return s > 0.0f ? (double)s * exp2((double)Rr - (double)Rw) : 0.0;
}
__device__ __attribute__((noinline)) float lse_of_ool(double R, double S) {
    return (float)((R + log2(S)) * kLn2);
}

template <int NT, bool OutOfLine = false>
__device__ float block_lse(float Rr, float s, double* red, double& Rtop) {
    const float Rw = wave_max(Rr);
    double part;
    if constexpr (OutOfLine) part = rescale_part_ool(s, Rr, Rw);
    else part = s > 0.0f ? (double)s * exp2((double)Rr - (double)Rw) : 0.0;
    part = wave_sum(part);
    constexpr int W = NT / 64;
    double R = (double)Rw, S = part;
    if constexpr (W > 1) {
        if ((threadIdx.x & 63) == 0) {
            red[2 * (threadIdx.x >> 6)] = (double)Rw;
            red[2 * (threadIdx.x >> 6) + 1] = part;
        }
        __syncthreads();
        R = red[0];
#pragma unroll
        for (int i = 1; i < W; ++i) R = fmax(R, red[2 * i]);
        S = 0.0;
#pragma unroll
        for (int i = 0; i < W; ++i)
            S += red[2 * i + 1] > 0.0 ? red[2 * i + 1] * exp2(red[2 * i] - R) : 0.0;
    }
    Rtop = S > 0.0 ? R : 0.0;
    if constexpr (OutOfLine) return S > 0.0 ? lse_of_ool(R, S) : -INFINITY;
    return S > 0.0 ? (float)((R + log2(S)) * kLn2) : -INFINITY;
}

// The normaliser of a row whose largest scaled logit is so large in
// magnitude (|max x/T| log2 e >= 2^30) that the residual of the stream's
// fused reference, fl(max x sc), leaves exp2's range: the maximum of the
// tempered values fl32(x/T) first, then the fp64 sum of exp(value - max),
// one rounding at the end.  for_each(f) calls f(x) on each of the thread's
// logits; two passes over them.
template <int NT, typename ForEach>
__device__ float exact_lse(ForEach&& for_each, float inv_t, double* red) {
    float m = -INFINITY;
    for_each([&](float x) { m = fmaxf(m, __fmul_rn(x, inv_t)); });
    m = block_max<NT>(m, reinterpret_cast<float*>(red));
    if (m == -INFINITY) return -INFINITY;
    double sum = 0.0;
    for_each([&](float x) { sum += exp((double)__fmul_rn(x, inv_t) - (double)m); });
    sum = block_sum<NT>(sum, red);
    return (float)((double)m + log(sum));
}

}  // namespace
}  // namespace gr
