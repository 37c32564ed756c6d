// backward.h -- the surrogate backward's kernels (host launch interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gr {

// Paths and weights of every final slot of a search of `steps` steps.
struct BackwardArgs {
    int32_t B, K, T, steps;
    const int32_t* parents;  // [T, B, K] history (rows < steps are read)
    const int32_t* tokens;   // [T, B, K]
    const float* score;      // [B, K] final scores (-inf = empty slot)
    const int32_t* seq;      // [B, K, T] final sequences
    const float* grad;       // [B, K] upstream gradient of each final ranked score
    const float* pen;        // [T + 1] length penalty table
    int32_t* path_slot;      // [steps, B, K] out
    int32_t* path_token;     // [steps, B, K] out
    float* weight;           // [B, K] out
};

// One step's log-probability gradient, added to grad.
struct ScatterArgs {
    int32_t B, K, V, t;
    int64_t stride;            // elements between rows of grad
    const int32_t* path_slot;  // [steps, B, K]
    const int32_t* path_token;
    const float* weight;       // [B, K]
    float* grad;               // row (b, p) at (b*K + p) * stride
};

constexpr int kScatterThreads = 1024;

// Width of the scatter's sorting network: the power of two at or above K.
__host__ __device__ inline int scatter_width(int K) {
    int P = 1;
    while (P < K) P <<= 1;
    return P;
}

hipError_t launch_backward_paths(const BackwardArgs& a, hipStream_t st);
hipError_t launch_backward_scatter(const ScatterArgs& a, hipStream_t st);

}  // namespace gr
