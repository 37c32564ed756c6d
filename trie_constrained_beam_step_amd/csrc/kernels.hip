// kernels.hip -- gfx950 kernels of one trie-constrained beam step.
//
// Two kernels per step, both on the caller's stream:
//
//   row_kernel      one workgroup per possibly-live beam row (b, j):
//                   (1) streams the row of V logits once from HBM with 16-byte
//                       non-temporal loads, keeping a per-thread running max and
//                       a sum of exp2 terms in fp32, combined across the
//                       workgroup in fp64 into the row's log-sum-exp (the
//                       log-softmax normaliser over the full row);
//                   (2) walks the candidates of the row -- the CSR children of
//                       the slot's trie node (FlashRec README, "Decoding"), or
//                       every token when unconstrained -- gathering their
//                       logits (cache-hot) and forming c = S_j + (x_v - lse)
//                       in fp32, and keeps the row's best R = min(K, fan-out)
//                       candidates exactly, by admission into an LDS buffer
//                       with radix-select compaction;
//                   (3) writes those keys to the row's pool segment and its best
//                       s keys to a small per-row summary.
//   select_kernel   one workgroup per request: takes the K-th best summary key
//                   as a lower bound on the request's K-th best candidate,
//                   gathers the pool keys at or above it into LDS, selects the
//                   exact top K by radix select, ranks them (best first) and
//                   writes the new state: backpointers, tokens, scores, next
//                   trie nodes, finished flags and reordered sequences.
//
// A candidate is ordered by a 64-bit key: the order-preserving bit pattern of
// its fp32 score in the high word and the complement of its flat index
// j*V + v in the low word, so a larger key is a better candidate under
// "higher score, then lower flat index" (beamgrad README, "Features": a strict
// total order on candidates).  Keys are unique, so every selection is exact
// and the result does not depend on scheduling.
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
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

// ---------------------------------------------------------- radix select
//
// Threshold of the `need` largest 64-bit keys among those visited by
// for_each (every thread visits its share).  MSB-first, 8-bit digits: each
// pass histograms the next digit of the keys that share the prefix fixed so
// far, wave 0 finds the digit bin holding the need-th largest, and the pass
// ends early once that bin holds exactly the keys still needed.  Returns P
// such that exactly `need` keys are >= P (keys are unique).  Requires
// 1 <= need <= number of keys.  Uses hist[256] and misc[0..2].
template <int NT, typename ForEach>
__device__ uint64_t radix_threshold(ForEach for_each, uint32_t need, uint32_t* hist, int* misc) {
    const int tid = threadIdx.x;
    uint64_t prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        for_each([&](uint64_t k) {
            if ((k & mask) == prefix) atomicAdd(&hist[(uint32_t)(k >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            // lane l owns bins 255-4l .. 252-4l (descending)
            const uint32_t h0 = hist[255 - 4 * tid], h1 = hist[254 - 4 * tid];
            const uint32_t h2 = hist[253 - 4 * tid], h3 = hist[252 - 4 * tid];
            const uint32_t loc = h0 + h1 + h2 + h3;
            uint32_t inc = loc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(inc, o);
                if (tid >= o) inc += y;
            }
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
        const uint32_t d = (uint32_t)misc[0], above = (uint32_t)misc[1], hd = (uint32_t)misc[2];
        need -= above;
        prefix |= (uint64_t)d << shift;
        mask |= (uint64_t)0xFF << shift;
        __syncthreads();  // misc and hist are rewritten next
        if (hd == need) break;
    }
    return prefix;
}

// ------------------------------------------------------------- row kernel

// LDS layout of the row kernel (bytes): red (16 doubles), misc (16 ints),
// hist (256 u32), then the candidate buffer (cap keys, cap token ids) and
// the compaction staging area (stg keys, stg ids).
enum { kCount = 4, kStage = 5, kPoolW = 6, kSumW = 7 };

template <typename DT, int NT, int U>
__device__ __forceinline__ void stream_row(const DT* row, int V, float& Rr, float& s) {
    constexpr int VEC = 16 / (int)sizeof(DT);
    const int tid = threadIdx.x;
    float mx = -INFINITY;
    Rr = kFarBelow;
    s = 0.0f;
    // scalar element: running max in x, sum of 2^(x*log2e - Rr)
    auto take = [&](float x) {
        if (x > mx) {
            const float nr = x * kLog2e;
            s *= ex2(Rr - nr);
            Rr = nr;
            mx = x;
        }
        s += ex2(fmaf(x, kLog2e, -Rr));
    };
    const uintptr_t addr = (uintptr_t)row;
    int head = (int)(((16u - (uint32_t)(addr & 15u)) & 15u) / sizeof(DT));
    if (head > V) head = V;
    if (tid < head) take(load_elem<DT>(row, tid));
    const int64_t nvec = (int64_t)(V - head) / VEC;
    const u32x4* vp = reinterpret_cast<const u32x4*>(row + head);
    for (int64_t i0 = tid; i0 < nvec; i0 += (int64_t)U * NT) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * NT;
            if (i < nvec) w[u] = __builtin_nontemporal_load(vp + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * NT;
            if (i >= nvec) break;
            float x[VEC];
            if constexpr (VEC == 4) {
                x[0] = __uint_as_float(w[u].x);
                x[1] = __uint_as_float(w[u].y);
                x[2] = __uint_as_float(w[u].z);
                x[3] = __uint_as_float(w[u].w);
            } else {
                const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    x[2 * q] = __uint_as_float(ws[q] << 16);
                    x[2 * q + 1] = __uint_as_float(ws[q] & 0xFFFF0000u);
                }
            }
            float vm = x[0];
#pragma unroll
            for (int q = 1; q < VEC; ++q) vm = fmaxf(vm, x[q]);
            if (vm > mx) {
                const float nr = vm * kLog2e;
                s *= ex2(Rr - nr);
                Rr = nr;
                mx = vm;
            }
            const float nR = -Rr;
            float e[VEC];
#pragma unroll
            for (int q = 0; q < VEC; ++q) e[q] = ex2(fmaf(x[q], kLog2e, nR));
#pragma unroll
            for (int q = VEC / 2; q > 0; q >>= 1) {
#pragma unroll
                for (int r = 0; r < q; ++r) e[r] += e[r + q];
            }
            s += e[0];
        }
    }
    const int64_t tail0 = head + nvec * VEC;
    if (tail0 + tid < V) take(load_elem<DT>(row, tail0 + tid));
}

template <typename DT, int NT>
__global__ __launch_bounds__(NT) void row_kernel(StepArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    double* red = reinterpret_cast<double*>(lds);
    int* misc = reinterpret_cast<int*>(lds + 16 * sizeof(double));
    uint32_t* hist = reinterpret_cast<uint32_t*>(misc + 16);
    uint32_t* bk = hist + 256;
    uint32_t* bi = bk + a.cap;
    uint32_t* sk = bi + a.cap;
    uint32_t* si = sk + a.stg;

    const int tid = threadIdx.x;
    const int rowid = blockIdx.x;
    const int b = rowid / a.L;
    const int j = rowid - b * a.L;
    const int slot = b * a.K + j;
    if (rowid == 0 && tid < 4) a.stats[tid] = 0ull;  // the request kernel adds after us

    const float S = a.score[slot];
    if (S == -INFINITY) {  // empty slot: no candidate, row not read
        if (tid == 0) {
            a.cnt[rowid] = 0;
            a.ncand[rowid] = 0;
            a.lse_o[slot] = __uint_as_float(0x7FC00000u);
        }
        return;
    }
    if (a.fin[slot]) {  // finished: carried forward unchanged, row not read
        if (a.eos < 0) {  // no EOS in this search: a stray flag makes the slot empty
            if (tid == 0) {
                a.cnt[rowid] = 0;
                a.ncand[rowid] = 0;
                a.lse_o[slot] = __uint_as_float(0x7FC00000u);
            }
            return;
        }
        if (tid == 0) {
            const uint64_t key = cand_key(ord_f32(S), (uint32_t)j * (uint32_t)a.V + (uint32_t)a.eos);
            a.pool[(size_t)rowid * a.R] = key;
            a.summ[(size_t)rowid * a.s] = key;
            a.cnt[rowid] = 1;
            a.ncand[rowid] = 1;
            a.lse_o[slot] = __uint_as_float(0x7FC00000u);
        }
        return;
    }

    const DT* row = reinterpret_cast<const DT*>(a.logits) + (size_t)(b * a.K + j) * (size_t)a.stride;

    // (1) normaliser over the full row
    float Rr, sp;
    stream_row<DT, NT, 4>(row, a.V, Rr, sp);
    const float Rb = block_max<NT>(Rr, reinterpret_cast<float*>(red));
    const double part = sp > 0.0f ? (double)sp * exp2((double)Rr - (double)Rb) : 0.0;
    const double Sb = block_sum<NT>(part, red);
    const float lse = Sb > 0.0 ? (float)(((double)Rb + log2(Sb)) * kLn2) : -INFINITY;

    // (2) candidates: CSR children of the node, or every token
    int64_t e0 = 0, ncands = a.V;
    if (a.off) {
        const int32_t n = a.node[slot];
        if (n >= 0 && n < a.nnodes) {
            e0 = a.off[n];
            ncands = a.off[n + 1] - e0;
        } else {
            ncands = 0;  // not a node of this level: no valid continuation
        }
    }
    if (lse == -INFINITY) ncands = 0;  // no finite logit: no finite candidate
    if (tid == 0) misc[kCount] = 0;
    __syncthreads();

    const uint32_t R = (uint32_t)a.R;
    uint64_t theta = 0;  // admission bound: keys below it cannot make the row's top R
    long long nfin = 0;
    auto for_buf = [&](int n) {
        return [=](auto&& f) {
            for (int i = tid; i < n; i += NT) f(((uint64_t)bk[i] << 32) | (uint32_t)~bi[i]);
        };
    };
    constexpr int E = kAdmitPerThread;
    for (int64_t base = 0; base < ncands; base += (int64_t)E * NT) {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int64_t ci = base + (int64_t)k * NT + tid;
            if (ci < ncands) {
                const int32_t v = a.off ? a.tok[e0 + ci] : (int32_t)ci;
                const float x = load_elem<DT>(row, v);
                const float c = __fadd_rn(S, __fsub_rn(x, lse));
                if (c != -INFINITY) {
                    ++nfin;
                    const uint32_t o = ord_f32(c);
                    const uint64_t comp = ((uint64_t)o << 32) | (uint32_t)~(uint32_t)v;
                    if (comp >= theta) {
                        const int p = atomicAdd(&misc[kCount], 1);
                        bk[p] = o;
                        bi[p] = (uint32_t)v;
                    }
                }
            }
        }
        __syncthreads();
        const int cnt = misc[kCount];
        const int64_t rem = ncands - (base + (int64_t)E * NT);
        const int64_t nxt = rem < (int64_t)E * NT ? rem : (int64_t)E * NT;
        __syncthreads();
        if (rem > 0 && cnt + nxt > a.cap) {
            // keep the R best so far; later candidates must beat the R-th
            theta = radix_threshold<NT>(for_buf(cnt), R, hist, misc);
            if (tid == 0) misc[kStage] = 0;
            __syncthreads();
            for (int i = tid; i < cnt; i += NT) {
                const uint64_t comp = ((uint64_t)bk[i] << 32) | (uint32_t)~bi[i];
                if (comp >= theta) {
                    const int p = atomicAdd(&misc[kStage], 1);
                    sk[p] = bk[i];
                    si[p] = bi[i];
                }
            }
            __syncthreads();
            for (int i = tid; i < (int)R; i += NT) {
                bk[i] = sk[i];
                bi[i] = si[i];
            }
            if (tid == 0) misc[kCount] = (int)R;
            __syncthreads();
        }
    }

    // (3) the row's best R to the pool, its best s to the summary
    __syncthreads();
    const int n = misc[kCount];
    const int keep = n < (int)R ? n : (int)R;
    uint64_t thR = 0, thS = 0;
    if (n > (int)R) thR = radix_threshold<NT>(for_buf(n), R, hist, misc);
    if (keep > a.s) thS = radix_threshold<NT>(for_buf(n), (uint32_t)a.s, hist, misc);
    if (tid == 0) {
        misc[kPoolW] = 0;
        misc[kSumW] = 0;
    }
    __syncthreads();
    uint64_t* pseg = a.pool + (size_t)rowid * a.R;
    uint64_t* sseg = a.summ + (size_t)rowid * a.s;
    const uint32_t jV = (uint32_t)j * (uint32_t)a.V;
    for (int i = tid; i < n; i += NT) {
        const uint64_t comp = ((uint64_t)bk[i] << 32) | (uint32_t)~bi[i];
        if (comp >= thR) {
            const uint64_t key = cand_key(bk[i], jV + bi[i]);
            pseg[atomicAdd(&misc[kPoolW], 1)] = key;
            if (comp >= thS) sseg[atomicAdd(&misc[kSumW], 1)] = key;
        }
    }
    const long long nf = block_sum_ll<NT>(nfin, reinterpret_cast<long long*>(red));
    if (tid == 0) {
        a.cnt[rowid] = keep;
        a.ncand[rowid] = (int32_t)nf;
        a.lse_o[slot] = lse;
    }
}

// ---------------------------------------------------------- select kernel

enum { kSelN = 4, kSurv = 5 };

__global__ __launch_bounds__(kSelectThreads) void select_kernel(StepArgs a) {
    constexpr int NT = kSelectThreads;
    extern __shared__ __align__(16) uint8_t lds[];
    long long* red = reinterpret_cast<long long*>(lds);            // 16
    int* misc = reinterpret_cast<int*>(lds + 16 * sizeof(long long)); // 16
    uint32_t* hist = reinterpret_cast<uint32_t*>(misc + 16);        // 256
    uint64_t* buf = reinterpret_cast<uint64_t*>(hist + 256);        // sb
    uint64_t* sel = buf + a.sb;                                     // K

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int NW = NT / 64;
    const int b = blockIdx.x;
    const int L = a.L, K = a.K;
    const int32_t* cnt = a.cnt + (size_t)b * L;
    const uint64_t* pool = a.pool + (size_t)b * L * a.R;
    const uint64_t* summ = a.summ + (size_t)b * L * a.s;

    long long tot = 0, totc = 0, nsum = 0, rows = 0;
    for (int j = tid; j < L; j += NT) {
        const int c = cnt[j];
        tot += c;
        nsum += c < a.s ? c : a.s;
        totc += a.ncand[(size_t)b * L + j];
        rows += isnan(a.lse_o[(size_t)b * K + j]) ? 0 : 1;
    }
    tot = block_sum_ll<NT>(tot, red);
    nsum = block_sum_ll<NT>(nsum, red);
    totc = block_sum_ll<NT>(totc, red);
    rows = block_sum_ll<NT>(rows, red);

    // visit every pool key of the request: one wave per row
    auto for_pool = [&](auto&& f) {
        for (int j = w; j < L; j += NW) {
            const int c = cnt[j];
            const uint64_t* seg = pool + (size_t)j * a.R;
            for (int i = lane; i < c; i += 64) f(seg[i]);
        }
    };
    auto for_lds = [&](const uint64_t* p, int n) {
        return [=](auto&& f) {
            for (int i = tid; i < n; i += NT) f(p[i]);
        };
    };

    int nsel;
    long long nsurv = tot;
    int slow = 0;
    if (tid == 0) misc[kSelN] = 0;
    __syncthreads();
    if (tot <= K) {
        for_pool([&](uint64_t k) { sel[atomicAdd(&misc[kSelN], 1)] = k; });
        nsel = (int)tot;
    } else {
        uint64_t tau = 0;
        if (nsum >= K && nsum <= a.sb) {
            if (tid == 0) misc[kSurv] = 0;
            __syncthreads();
            for (int j = w; j < L; j += NW) {
                const int c = cnt[j] < a.s ? cnt[j] : a.s;
                const uint64_t* seg = summ + (size_t)j * a.s;
                for (int i = lane; i < c; i += 64) buf[atomicAdd(&misc[kSurv], 1)] = seg[i];
            }
            __syncthreads();
            tau = radix_threshold<NT>(for_lds(buf, (int)nsum), (uint32_t)K, hist, misc);
        }
        if (tid == 0) misc[kSurv] = 0;
        __syncthreads();
        for_pool([&](uint64_t k) {
            if (k >= tau) {
                const int p = atomicAdd(&misc[kSurv], 1);
                if (p < a.sb) buf[p] = k;
            }
        });
        __syncthreads();
        nsurv = misc[kSurv];
        uint64_t theta;
        if (nsurv <= a.sb) {
            theta = radix_threshold<NT>(for_lds(buf, (int)nsurv), (uint32_t)K, hist, misc);
            for (int i = tid; i < (int)nsurv; i += NT)
                if (buf[i] >= theta) sel[atomicAdd(&misc[kSelN], 1)] = buf[i];
        } else {
            // too many survivors for LDS: select straight from the pool
            slow = 1;
            theta = radix_threshold<NT>(for_pool, (uint32_t)K, hist, misc);
            for_pool([&](uint64_t k) {
                if (k >= theta) sel[atomicAdd(&misc[kSelN], 1)] = k;
            });
        }
        nsel = K;
    }
    __syncthreads();

    // rank (keys are unique), decode and write the new state
    const int T = a.T, t = a.t, V = a.V;
    for (int i = tid; i < nsel; i += NT) {
        const uint64_t key = sel[i];
        int r = 0;
        for (int m = 0; m < nsel; ++m) r += sel[m] > key ? 1 : 0;
        const uint32_t flat = ~(uint32_t)key;
        const int j = (int)(flat / (uint32_t)V);
        const int v = (int)(flat - (uint32_t)j * (uint32_t)V);
        const size_t ps = (size_t)b * K + j;
        int tokn, nd;
        uint8_t f;
        if (a.fin[ps]) {
            tokn = -1; nd = -1; f = 1;
        } else if (a.off) {
            const int32_t n = a.node[ps];
            int64_t lo = a.off[n], hi = a.off[n + 1];
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if (a.tok[mid] < v) lo = mid + 1; else hi = mid;
            }
            const bool found = lo < a.off[n + 1] && a.tok[lo] == v;
            tokn = v; nd = found ? a.child[lo] : -1; f = 0;
        } else {
            tokn = v; nd = -1; f = (uint8_t)(v == a.eos);
        }
        const size_t o = (size_t)b * K + r;
        a.score_o[o] = unord_f32((uint32_t)(key >> 32));
        a.node_o[o] = nd;
        a.fin_o[o] = f;
        a.parent_o[o] = j;
        a.token_o[o] = tokn;
        const int32_t* sp = a.seq + ps * T;
        int32_t* so = a.seq_o + o * T;
        for (int q = 0; q < T; ++q) so[q] = q < t ? sp[q] : (q == t ? tokn : -1);
    }
    for (int r = nsel + tid; r < K; r += NT) {
        const size_t o = (size_t)b * K + r;
        a.score_o[o] = -INFINITY;
        a.node_o[o] = -1;
        a.fin_o[o] = 0;
        a.parent_o[o] = -1;
        a.token_o[o] = -1;
        for (int q = 0; q < T; ++q) a.seq_o[o * T + q] = -1;
    }
    for (int j = L + tid; j < K; j += NT) a.lse_o[(size_t)b * K + j] = __uint_as_float(0x7FC00000u);
    if (tid == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)rows);
        atomicAdd(&a.stats[1], (unsigned long long)totc);
        atomicAdd(&a.stats[2], (unsigned long long)nsurv);
        atomicAdd(&a.stats[3], (unsigned long long)slow);
    }
}

// ------------------------------------------------------------ small kernels

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

__global__ void probe_read_kernel(const u32x4* src, size_t n16, uint32_t* sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc = (uint32_t)wave_sum_ll((long long)acc);
    if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x & 65535u], acc);
}

__global__ void probe_copy_kernel(u32x4* dst, const u32x4* src, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

}  // namespace

size_t row_lds_bytes(int cap, int stg) {
    return 16 * sizeof(double) + 16 * sizeof(int) + 256 * sizeof(uint32_t) +
           (size_t)(2 * cap + 2 * stg) * sizeof(uint32_t);
}

size_t select_lds_bytes(int sb, int K) {
    return 16 * sizeof(long long) + 16 * sizeof(int) + 256 * sizeof(uint32_t) +
           (size_t)(sb + K) * sizeof(uint64_t);
}

hipError_t launch_rows(const StepArgs& a, int bf16, hipStream_t st) {
    const int NT = row_threads(a.V);
    const size_t lds = row_lds_bytes(a.cap, a.stg);
    const dim3 grid((unsigned)(a.B * a.L));
    if (bf16) {
        if (NT == 64) row_kernel<uint16_t, 64><<<grid, 64, lds, st>>>(a);
        else row_kernel<uint16_t, 256><<<grid, 256, lds, st>>>(a);
    } else {
        if (NT == 64) row_kernel<float, 64><<<grid, 64, lds, st>>>(a);
        else row_kernel<float, 256><<<grid, 256, lds, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_select(const StepArgs& a, hipStream_t st) {
    select_kernel<<<dim3((unsigned)a.B), kSelectThreads, select_lds_bytes(a.sb, a.K), st>>>(a);
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

hipError_t launch_probe_read(const void* src, size_t n16, uint32_t* sink, hipStream_t st) {
    probe_read_kernel<<<4096, 256, 0, st>>>(reinterpret_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t n16, hipStream_t st) {
    probe_copy_kernel<<<4096, 256, 0, st>>>(reinterpret_cast<u32x4*>(dst),
                                            reinterpret_cast<const u32x4*>(src), n16);
    return hipGetLastError();
}

hipError_t set_lds_limits(int row_bytes, int select_bytes) {
    hipError_t e = hipSuccess;
    hipError_t r;
    r = hipFuncSetAttribute((const void*)row_kernel<float, 64>, hipFuncAttributeMaxDynamicSharedMemorySize, row_bytes);
    if (r != hipSuccess) e = r;
    r = hipFuncSetAttribute((const void*)row_kernel<float, 256>, hipFuncAttributeMaxDynamicSharedMemorySize, row_bytes);
    if (r != hipSuccess) e = r;
    r = hipFuncSetAttribute((const void*)row_kernel<uint16_t, 64>, hipFuncAttributeMaxDynamicSharedMemorySize, row_bytes);
    if (r != hipSuccess) e = r;
    r = hipFuncSetAttribute((const void*)row_kernel<uint16_t, 256>, hipFuncAttributeMaxDynamicSharedMemorySize, row_bytes);
    if (r != hipSuccess) e = r;
    r = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, select_bytes);
    if (r != hipSuccess) e = r;
    return e;
}

}  // namespace gr
