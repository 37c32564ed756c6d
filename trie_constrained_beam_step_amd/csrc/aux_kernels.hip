// aux_kernels.hip -- state reset and the bandwidth probes.
#include "device_common.h"

namespace gr {
namespace {

__global__ void reset_kernel(float* score, int32_t* node, uint8_t* fin, int32_t* seq,
                             int32_t* parents, int32_t* tokens, float* lse, int B, int K, int T,
                             int root) {
    const size_t n = (size_t)B * K;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n * T; i += stride) {
        seq[i] = -1;
        parents[i] = -1;
        tokens[i] = -1;
        if (i < n) {
            const bool first = (i % K) == 0;
            score[i] = first ? 0.0f : -INFINITY;
            node[i] = first ? root : -1;
            fin[i] = 0;
            lse[i] = __uint_as_float(0x7FC00000u);
        }
    }
}

// 1 + the last slot of any request whose score is not -inf (0 when none)
// to *out: one workgroup.
constexpr int kLiveThreads = 1024;
__global__ __launch_bounds__(kLiveThreads) void live_bound_kernel(const float* score, int B, int K, int* out) {
    __shared__ int wbest[kLiveThreads / 64];
    const int64_t n = (int64_t)B * K;
    int best = 0;
    for (int64_t i = threadIdx.x; i < n; i += kLiveThreads)
        if (score[i] != -INFINITY) best = max(best, (int)(i % K) + 1);
    best = wave_reduce(best, 0, [](int x, int y) { return x > y ? x : y; });
    if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kLiveThreads / 64; ++w) best = max(best, wbest[w]);
        *out = best;
    }
}

// Streaming read probe: each workgroup reads one contiguous chunk of
// kProbeChunk 16-byte vectors (64 KB) with non-temporal loads, kProbeLoads in
// flight per thread -- the fastest plain read of a sweep over chunk sizes,
// loads in flight, workgroup sizes and grid-stride layouts on MI355X.
constexpr size_t kProbeChunk = 4096;
constexpr int kProbeLoads = 8;

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* src, size_t n16, uint32_t* sink) {
    const size_t beg = (size_t)blockIdx.x * kProbeChunk;
    const size_t end = beg + kProbeChunk < n16 ? beg + kProbeChunk : n16;
    uint32_t acc = 0;
    for (size_t i0 = beg + threadIdx.x; i0 < end; i0 += kProbeLoads * 256) {
        u32x4 v[kProbeLoads];
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) {
            const size_t i = i0 + (size_t)u * 256;
            v[u] = i < end ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    acc = (uint32_t)wave_sum_ll((long long)acc);
    if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x & 65535u], acc);
}

__global__ void probe_copy_kernel(u32x4* dst, const u32x4* src, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

// The dense table of one trie level: every entry -1, then each node's
// children at their codes (token - tbase), one thread per node.
__global__ void dense_fill_kernel(int32_t* dense, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dense[i] = -1;
}

__global__ void dense_scatter_kernel(const int64_t* off, const int32_t* tok, const int32_t* child, int64_t nnodes,
                                     int32_t tbase, int32_t span, int32_t* dense) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < nnodes; n += stride)
        for (int64_t e = off[n]; e < off[n + 1]; ++e) dense[n * span + (tok[e] - tbase)] = child[e];
}

// Largest |gumbel_fast(r) - gumbel_of_word(r)| over the Philox words r0 ..
// r0 + count - 1, as the bit pattern of an fp64 (non-negative doubles order
// as their bits), into *out with one atomic per wave; *out starts at zero.
__global__ void probe_zero_kernel(unsigned long long* out) { *out = 0ull; }

__global__ __launch_bounds__(256) void probe_draw_error_kernel(uint32_t r0, uint64_t count, unsigned long long* out) {
    const uint64_t stride = (uint64_t)gridDim.x * 256u;
    double m = 0.0;
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < count; i += stride) {
        const uint32_t r = r0 + (uint32_t)i;
        m = fmax(m, fabs((double)gumbel_fast(r) - (double)gumbel_of_word(r)));
    }
    m = wave_reduce(m, 0.0, [](double x, double y) { return fmax(x, y); });
    if ((threadIdx.x & 63) == 0) atomicMax(out, (unsigned long long)__double_as_longlong(m));
}

}  // namespace

hipError_t launch_probe_draw_error(uint32_t r0, uint64_t count, double* out, hipStream_t st) {
    unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
    probe_zero_kernel<<<1, 1, 0, st>>>(o);
    const uint64_t blocks = (count + 255) / 256;
    if (blocks > 0) probe_draw_error_kernel<<<(unsigned)(blocks < 8192 ? blocks : 8192), 256, 0, st>>>(r0, count, o);
    return hipGetLastError();
}

float draw_error_bound() { return kDrawErr; }

hipError_t launch_trie_densify(const int64_t* off, const int32_t* tok, const int32_t* child, int64_t nnodes,
                               int32_t tbase, int32_t span, int32_t* dense, hipStream_t st) {
    const int64_t n = nnodes * span;
    if (n == 0) return hipSuccess;
    dense_fill_kernel<<<4096, 256, 0, st>>>(dense, n);
    const int64_t blocks = (nnodes + 255) / 256;
    dense_scatter_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, st>>>(off, tok, child, nnodes, tbase,
                                                                                  span, dense);
    return hipGetLastError();
}

hipError_t launch_reset(float* score, int32_t* node, uint8_t* fin, int32_t* seq, int32_t* parents,
                        int32_t* tokens, float* lse, int B, int K, int T, int root,
                        hipStream_t st) {
    const size_t n = (size_t)B * K * T;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    reset_kernel<<<blocks, 256, 0, st>>>(score, node, fin, seq, parents, tokens, lse, B, K, T, root);
    return hipGetLastError();
}

hipError_t launch_live_bound(const float* score, int B, int K, int* out, hipStream_t st) {
    live_bound_kernel<<<1, kLiveThreads, 0, st>>>(score, B, K, out);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t n16, uint32_t* sink, hipStream_t st) {
    const size_t blocks = (n16 + kProbeChunk - 1) / kProbeChunk;
    if (blocks == 0) return hipSuccess;
    probe_read_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(reinterpret_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t n16, hipStream_t st) {
    probe_copy_kernel<<<4096, 256, 0, st>>>(reinterpret_cast<u32x4*>(dst),
                                            reinterpret_cast<const u32x4*>(src), n16);
    return hipGetLastError();
}

}  // namespace gr
