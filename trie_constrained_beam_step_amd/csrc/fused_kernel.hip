// fused_kernel.hip -- one trie-constrained beam step in one launch, for
// short rows (a few KB of logits per beam).
//
// The step computes what the row kernel and the request kernel compute
// together (log-softmax normaliser over each live row, the CSR children of
// the row's trie node as candidates, c = S_j + (x_v - lse_j) in fp32, the K
// best of each request under (higher c, lower j*V + v), and the new state;
// FlashRec README, "Decoding"; beamgrad README, "How it works"), organised
// for rows too short to keep a 256-thread workgroup busy:
//   1. the L rows of request b are split over fw workgroups (rpw rows each);
//      each wave of a workgroup takes whole rows: it streams the row, folds
//      its log-sum-exp in registers, gathers the children's logits (their
//      token ids are fetched before the stream, their logits as soon as the
//      stream's first loads are in flight) and appends every finite
//      candidate's 64-bit key to the workgroup's LDS buffer -- no per-row
//      selection and no per-row summary;
//   2. the workgroup keeps its K best keys (a radix select over the buffer),
//      raises the request's running bound (64-bit atomic maximum) with its
//      own K-th best key -- every workgroup's K-th best is at most the
//      request's -- and writes its keys at or above that bound;
//   3. it counts itself done on the request's counter, and the last
//      workgroup to finish merges the kept keys (admitting those at or above
//      the final bound, compacting back to the K best whenever the next
//      chunk might not fit), ranks the K best and decodes them into the new
//      state.  It resets the counter and the bound for the next step.  No
//      workgroup waits for another.
// Every value one workgroup hands to another (kept keys, their counts, the
// per-workgroup counters) is stored and loaded with device-scope atomic
// accesses, which the GPU keeps coherent across its XCDs' L2 caches, and
// each wave waits for its stores to complete before the workgroup counts
// itself done; nothing needs a device-wide fence (an L2 write-back).
// The keys are those of the two-kernel step (ordered fp32 score, then the
// complement of j*F + i, i the candidate's edge ordinal in its node), so the
// results are identical to it.  The host takes this path only for CSR trie
// levels, unperturbed ranking (no sampling, length penalty or masks), the
// full-row normaliser, K <= kFusedCap / 2, rows of at most kFusedMaxRowBytes
// and rpw x (the level's largest fan-out) <= kFusedCap, so no buffer can
// overflow.
#include "row_stream.h"

namespace gr {
namespace {

// LDS ints: candidate count, last-workgroup flag, kept count, rows, finite
// candidates, merge chunk bookkeeping; [16..18] the radix select's scratch
enum { fCount = 0, fLast = 1, fKept = 2, fRows = 3, fFin = 4, fMisc = 16 };
constexpr int kFusedCountRankMax = 512;  // larger selections are sorted to rank them
constexpr int kCompactPerThread = kFusedCap / kFusedThreads;

// Device-scope (cross-XCD coherent) store and load of a value handed to
// another workgroup.
template <typename T>
__device__ __forceinline__ void store_dev(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_dev(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Keep only the keys >= th of buf[0..n) (n <= kFusedCap), packed at the
// front; returns how many (every thread gets it).  Ends with a barrier.
template <int NT>
__device__ int compact_ge(uint64_t* buf, int n, uint64_t th, int* ctr) {
    const int tid = threadIdx.x;
    uint64_t r[kCompactPerThread];
#pragma unroll
    for (int q = 0; q < kCompactPerThread; ++q) {
        const int i = tid + q * NT;
        r[q] = i < n ? buf[i] : 0ull;
    }
    if (tid == 0) *ctr = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCompactPerThread; ++q) {
        const bool keep = r[q] != 0ull && r[q] >= th;
        const int p = wave_claim(ctr, keep);
        if (keep) buf[p] = r[q];
    }
    __syncthreads();
    const int m = *ctr;
    __syncthreads();
    return m;
}

template <typename DT>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(4))) void fused_kernel(StepArgs a) {
    constexpr int NT = kFusedThreads, NW = NT / 64, E = kAdmitPerThread;
    extern __shared__ __align__(16) uint8_t lds[];
    double* red = reinterpret_cast<double*>(lds);                   // 16
    int* misc = reinterpret_cast<int*>(red + 16);                    // 32
    uint32_t* hist = reinterpret_cast<uint32_t*>(misc + 32);         // 256
    int* pre = reinterpret_cast<int*>(hist + 256);                   // kFusedMaxW + 1
    uint64_t* buf = reinterpret_cast<uint64_t*>(pre + kFusedMaxW + 2);  // fcap keys (8-byte aligned)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fw = a.fw;
    const int b = blockIdx.x / fw, w = blockIdx.x - b * fw;
    const int K = a.K, L = a.L, T = a.T, t = a.t;
    const int j0 = w * a.rpw, j1 = min(L, j0 + a.rpw);
    const float kNaN = __uint_as_float(0x7FC00000u);
    const DT* logits = reinterpret_cast<const DT*>(a.logits);
    if (tid < 16) misc[tid] = 0;
    __syncthreads();

    // 1. the workgroup's rows, one per wave at a time
    int rows = 0;
    long long nfin = 0;
    for (int j = j0 + wave; j < j1; j += NW) {
        const int slot = b * K + j;
        const float S = a.score[slot];
        if (S == -INFINITY || a.fin[slot]) {  // empty (a finished flag has no EOS to carry here)
            if (lane == 0) a.lse_o[slot] = kNaN;
            continue;
        }
        const DT* row = logits + (size_t)slot * (size_t)a.stride;
        const int32_t n = a.node[slot];
        int64_t e0 = 0, f = 0;
        if (n >= 0 && n < a.nnodes) {
            e0 = a.off[n];
            f = a.off[n + 1] - e0;
        }
        int32_t cv[E];
        float xv[E];
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int ci = lane + 64 * k;
            cv[k] = ci < f ? a.tok[e0 + ci] : -1;
        }
        float Rr = kFarBelow, sp = 0.0f, tmax = -INFINITY;
        int ninf = 0;
        DrawCtx dc;
        // (bf16 rows: two 16-byte vectors per batch, so their 32 unpacked values fit)
        stream_row<DT, 64, sizeof(DT) == 2 ? 2 : kStreamBatch, kPlain>(
            row, a.V, lane, kLog2e, Rr, sp,
            [&] {
#pragma unroll
                for (int k = 0; k < E; ++k) xv[k] = cv[k] >= 0 ? load_elem<DT>(row, cv[k]) : 0.0f;
            },
            nullptr, ninf, tmax, dc);
        double Rtop;
        float lse = block_lse<64>(Rr, sp, red, Rtop);
        if (fabs(Rtop) >= 0x1p30)  // rare: logits beyond the fused reference's range
            lse = exact_lse<64>(
                [&](auto&& g) {
                    for (int64_t i = lane; i < a.V; i += 64) g(load_elem<DT>(row, i));
                },
                1.0f, red);
        if (lane == 0) a.lse_o[slot] = lse;
        ++rows;
        if (lse == -INFINITY) continue;  // no finite logit: no finite candidate
        const uint32_t jF = (uint32_t)j * (uint32_t)a.F;
        for (int64_t c0 = 0; c0 < f; c0 += (int64_t)E * 64) {
            if (c0 > 0) {  // candidates past the first E*64 (wide nodes): gathered here
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int64_t ci = c0 + lane + 64 * k;
                    cv[k] = ci < f ? a.tok[e0 + ci] : -1;
                }
#pragma unroll
                for (int k = 0; k < E; ++k) xv[k] = cv[k] >= 0 ? load_elem<DT>(row, cv[k]) : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < E; ++k) {
                uint64_t key = 0;
                if (cv[k] >= 0) {
                    const float c = __fadd_rn(S, __fsub_rn(xv[k], lse));
                    if (c != -INFINITY) key = cand_key(ord_f32(c), jF + (uint32_t)(c0 + lane + 64 * k));
                }
                nfin += key != 0 ? 1 : 0;
                const int p = wave_claim(&misc[fCount], key != 0);
                if (key != 0 && p < a.fcap) buf[p] = key;
            }
        }
    }
    // the workgroup's counts
    nfin = wave_sum_ll(nfin);
    if (lane == 0) {
        atomicAdd(&misc[fRows], rows);
        atomicAdd(&misc[fFin], (int)nfin);
    }
    __syncthreads();
    int n = min(misc[fCount], a.fcap);

    // 2. its K best, and the request's running bound
    if (fw > 1) {
        uint64_t th = 0;
        if (n > K)
            th = radix_threshold<NT>(
                [&](auto&& g) {
                    for (int i = tid; i < n; i += NT) g(buf[i]);
                },
                (uint32_t)K, hist, misc + fMisc);
        if (tid == 0) {
            const unsigned long long old = atomicMax(&a.req_theta[b], (unsigned long long)th);
            const uint64_t cut = old > th ? old : th;
            red[8] = __longlong_as_double((long long)cut);
            misc[fKept] = 0;
        }
        __syncthreads();
        const uint64_t cut = (uint64_t)__double_as_longlong(red[8]);
        uint64_t* dst = a.part + ((size_t)b * fw + w) * K;
        for (int i = tid; i < n; i += NT) {
            const bool keep = buf[i] >= cut;
            const int p = wave_claim(&misc[fKept], keep);
            if (keep) store_dev(&dst[p], buf[i]);
        }
        __syncthreads();
        if (tid == 0) {
            const size_t pw = (size_t)b * fw + w;
            store_dev(&a.part_n[pw], misc[fKept]);
            store_dev(&a.part_stats[2 * pw], (long long)misc[fRows]);
            store_dev(&a.part_stats[2 * pw + 1], (long long)misc[fFin]);
        }
        // 3. every wave's hand-over stores complete before the workgroup
        //    counts itself done; the last to count merges
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) misc[fLast] = atomicAdd(&a.req_done[b], 1u) == (unsigned)(fw - 1);
        __syncthreads();
        if (!misc[fLast]) return;
        if (tid == 0) {
            // the final bound; then reset the request's bound and counter
            red[8] = __longlong_as_double((long long)atomicExch(&a.req_theta[b], 0ull));
            atomicExch(&a.req_done[b], 0u);
            long long rsum = 0, fsum = 0, ksum = 0;
            int tot = 0;
            for (int q = 0; q < fw; ++q) {
                const size_t pw = (size_t)b * fw + q;
                pre[q] = tot;
                tot += load_dev(&a.part_n[pw]);
                const long long rq = load_dev(&a.part_stats[2 * pw]), fq = load_dev(&a.part_stats[2 * pw + 1]);
                rsum += rq;
                fsum += fq;
                ksum += min((long long)K, fq);
            }
            pre[fw] = tot;
            red[9] = __longlong_as_double(rsum);
            red[10] = __longlong_as_double(fsum);
            red[11] = __longlong_as_double(ksum);
            misc[fCount] = 0;
        }
        __syncthreads();
        uint64_t bound = (uint64_t)__double_as_longlong(red[8]);
        const int N = pre[fw];
        // merge: chunks of kFusedCap - K keys, compacting back to the K best
        // whenever the next chunk might not fit
        const int chunk = a.fcap - K;
        n = 0;
        for (int g0 = 0; g0 < N; g0 += chunk) {
            const int g1 = min(N, g0 + chunk);
            for (int g = g0 + tid; g < g1; g += NT) {
                int lo = 0, hi = fw;  // pre[lo] <= g < pre[hi]
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (pre[mid] <= g) lo = mid; else hi = mid;
                }
                const uint64_t key = load_dev(&a.part[((size_t)b * fw + lo) * K + (g - pre[lo])]);
                const bool keep = key >= bound;
                const int p = wave_claim(&misc[fCount], keep);
                if (keep && p < a.fcap) buf[p] = key;  // (the chunks keep p below fcap)
            }
            __syncthreads();
            n = misc[fCount];
            if (g1 < N && n > K) {
                const uint64_t th = radix_threshold<NT>(
                    [&](auto&& g) {
                        for (int i = tid; i < n; i += NT) g(buf[i]);
                    },
                    (uint32_t)K, hist, misc + fMisc);
                bound = th > bound ? th : bound;
                n = compact_ge<NT>(buf, n, th, &misc[fKept]);
                if (tid == 0) misc[fCount] = n;
                __syncthreads();
            }
        }
        if (tid == 0) {
            misc[fRows] = (int)__double_as_longlong(red[9]);
            misc[fFin] = (int)__double_as_longlong(red[10]);
            // the workgroups' K best (not what the running bound let
            // through: that depends on the order they finished)
            misc[fKept] = (int)__double_as_longlong(red[11]);
        }
        __syncthreads();
    } else if (tid == 0) {
        misc[fKept] = min(n, K);  // one workgroup per request: its buffer is the request's
    }
    __syncthreads();
    const int survivors = misc[fKept];

    // 4. the K best, ranked (keys are unique) and decoded into the new state
    if (n > K) {
        const uint64_t th = radix_threshold<NT>(
            [&](auto&& g) {
                for (int i = tid; i < n; i += NT) g(buf[i]);
            },
            (uint32_t)K, hist, misc + fMisc);
        n = compact_ge<NT>(buf, n, th, &misc[fKept]);
    }
    const int nsel = n;
    auto decode = [&](uint64_t key, int r) {
        const uint32_t flat = ~(uint32_t)key;
        const int j = (int)(flat / (uint32_t)a.F);
        const int ci = (int)(flat - (uint32_t)j * (uint32_t)a.F);
        const int64_t base = a.off[a.node[(size_t)b * K + j]];  // the parent's first edge
        const int32_t tokn = a.tok[base + ci], nd = a.child[base + ci];
        const size_t o = (size_t)b * K + r;
        a.score_o[o] = unord_f32((uint32_t)(key >> 32));
        a.node_o[o] = nd;
        a.fin_o[o] = 0;
        a.parent_o[o] = j;
        a.token_o[o] = tokn;
        const int32_t* sp = a.seq + ((size_t)b * K + j) * T;
        int32_t* so = a.seq_o + o * T;
        for (int q = 0; q < T; ++q) so[q] = q < t ? sp[q] : (q == t ? tokn : -1);
    };
    if (nsel > kFusedCountRankMax) {
        int P = 1;
        while (P < nsel) P <<= 1;
        for (int i = nsel + tid; i < P; i += NT) buf[i] = 0ull;  // padding sorts last
        __syncthreads();
        block_bitonic_sort<NT, true>(buf, P);
        for (int i = tid; i < nsel; i += NT) decode(buf[i], i);
    } else {
        int G = 1;
        while (G < 64 && 2 * G * nsel <= NT) G *= 2;
        for (int i0 = 0; i0 < nsel; i0 += NT / G) {
            const int i = i0 + tid / G, part = tid % G;
            const uint64_t key = i < nsel ? buf[i] : 0ull;
            int r = 0;
            if (i < nsel) {
                int m = part;
                for (; m + 3 * G < nsel; m += 4 * G)
                    r += (buf[m] > key ? 1 : 0) + (buf[m + G] > key ? 1 : 0) + (buf[m + 2 * G] > key ? 1 : 0) +
                         (buf[m + 3 * G] > key ? 1 : 0);
                for (; m < nsel; m += G) r += buf[m] > key ? 1 : 0;
            }
            for (int o = 1; o < G; o <<= 1) r += __shfl_xor(r, o);
            if (i < nsel && part == 0) decode(key, r);
        }
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
    for (int j = L + tid; j < K; j += NT) a.lse_o[(size_t)b * K + j] = kNaN;
    if (tid == 0) {
        unsigned long long* st = a.stats + (size_t)b * kNumStats;
        st[0] = (unsigned long long)misc[fRows];
        st[1] = (unsigned long long)misc[fFin];
        st[2] = (unsigned long long)survivors;
        st[3] = 0;
        st[4] = 0;
        st[5] = 1;
    }
}

}  // namespace

size_t fused_lds_bytes(int fcap, int fw) {
    (void)fw;
    return 16 * sizeof(double) + 32 * sizeof(int) + 256 * sizeof(uint32_t) +
           (size_t)(kFusedMaxW + 2) * sizeof(int) + (size_t)fcap * sizeof(uint64_t);
}

hipError_t launch_fused(const StepArgs& a, int bf16, hipStream_t st) {
    const size_t lds = fused_lds_bytes(a.fcap, a.fw);
    const dim3 grid((unsigned)(a.B * a.fw));
    if (bf16) fused_kernel<uint16_t><<<grid, kFusedThreads, lds, st>>>(a);
    else fused_kernel<float><<<grid, kFusedThreads, lds, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, int bf16, hipStream_t st) {
    if (a.fw > 0) return launch_fused(a, bf16, st);
    hipError_t e = launch_rows(a, bf16, st);
    return e != hipSuccess ? e : launch_select(a, bf16, st);
}

}  // namespace gr
