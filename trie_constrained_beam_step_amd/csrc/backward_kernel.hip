// backward_kernel.hip -- surrogate backward of a search (beamgrad README,
// "How it works": with the selection held fixed, the gradient of final beam
// k's ranked score with respect to log_probs[t, p, v] is 1 / penalty(length_k)
// for each (t, p, v) on k's path and zero elsewhere; "Features": each step is
// handed only its own path gradient, never a dense [B, T, K, V] array).
//
//   backward_paths_kernel: one thread per final slot (b, k) walks the stored
//     backpointers from the last step to the first, writing the slot and
//     token of k's path at every step (token -1 where the beam was carried:
//     that step added no log-probability) and k's weight
//     grad[b][k] / pen(len_k), len_k = the tokens of k's final sequence.
//   backward_scatter_kernel: one workgroup per request adds step t's gradient
//     into a [B, K, V] buffer.  Final beams sharing (p, v) at step t share
//     the target: the (target, k) pairs are sorted in LDS, so each target's
//     beams are adjacent in ascending k, and the first of them (lowest k)
//     sums all their weights in that order and adds once -- every target has
//     one writer and the result does not depend on scheduling.
#include <math.h>

#include "backward.h"
#include "device_common.h"

namespace gr {
namespace {

__global__ __launch_bounds__(256) void backward_paths_kernel(BackwardArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)a.B * a.K;
    if (gid >= n) return;
    const int b = (int)(gid / a.K), k = (int)(gid - (int64_t)b * a.K);
    const bool live = a.score[gid] != -INFINITY;
    int i = live ? k : -1;
    for (int t = a.steps - 1; t >= 0; --t) {
        int p = -1, v = -1;
        if (i >= 0) {
            const int64_t h = (int64_t)t * n + (int64_t)b * a.K + i;
            p = a.parents[h];
            v = a.tokens[h];
            if (p >= a.K) p = -1;  // outside the history's range: the walk ends
        }
        a.path_slot[(int64_t)t * n + gid] = p;
        a.path_token[(int64_t)t * n + gid] = v;
        i = p;
    }
    float w = 0.0f;
    if (live) {
        int len = 0;
        for (int q = 0; q < a.T; ++q) len += a.seq[gid * a.T + q] != -1 ? 1 : 0;
        w = __fdiv_rn(a.grad[gid], a.pen[len]);
    }
    a.weight[gid] = w;
}

__global__ __launch_bounds__(kScatterThreads) void backward_scatter_kernel(ScatterArgs a) {
    extern __shared__ __align__(16) uint64_t sm64[];
    constexpr int NT = kScatterThreads;
    const int K = a.K;
    const int P = scatter_width(K);
    // entries (target << 32) | k, target = p*V + v (K*V < 2^32) or ~0 for no
    // entry; sorted ascending, each target's beams are adjacent in ascending k
    uint64_t* ent = sm64;
    float* w = reinterpret_cast<float*>(ent + P);  // [K] the beams' weights
    const int b = blockIdx.x;
    const int64_t n = (int64_t)a.B * K;
    const int64_t row0 = (int64_t)a.t * n + (int64_t)b * K;
    for (int k = threadIdx.x; k < P; k += NT) {
        uint64_t e = ~0ull;  // padding: sorts last
        if (k < K) {
            const int p = a.path_slot[row0 + k], v = a.path_token[row0 + k];
            const bool ok = v >= 0 && v < a.V && p >= 0 && p < K;
            const uint32_t target = ok ? (uint32_t)p * (uint32_t)a.V + (uint32_t)v : ~0u;
            e = ((uint64_t)target << 32) | (uint32_t)k;
            w[k] = a.weight[(int64_t)b * K + k];
        }
        ent[k] = e;
    }
    __syncthreads();
    block_bitonic_sort<NT, false>(ent, P);
    // the first beam of each target sums the weights of all beams through it,
    // in ascending k, and adds once
    for (int i = threadIdx.x; i < K; i += NT) {
        const uint32_t e = (uint32_t)(ent[i] >> 32);
        if (e == ~0u) continue;
        if (i > 0 && (uint32_t)(ent[i - 1] >> 32) == e) continue;
        float acc = 0.0f;
        for (int q = i; q < K && (uint32_t)(ent[q] >> 32) == e; ++q) acc = __fadd_rn(acc, w[(uint32_t)ent[q]]);
        const uint32_t p = e / (uint32_t)a.V, v = e - p * (uint32_t)a.V;
        float* g = a.grad + ((int64_t)b * K + p) * a.stride + v;
        *g = __fadd_rn(*g, acc);
    }
}

}  // namespace

hipError_t launch_backward_paths(const BackwardArgs& a, hipStream_t st) {
    const int64_t n = (int64_t)a.B * a.K;
    backward_paths_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_backward_scatter(const ScatterArgs& a, hipStream_t st) {
    const size_t lds = (size_t)scatter_width(a.K) * sizeof(uint64_t) + (size_t)a.K * sizeof(float);
    backward_scatter_kernel<<<dim3((unsigned)a.B), kScatterThreads, lds, st>>>(a);
    return hipGetLastError();
}

}  // namespace gr
