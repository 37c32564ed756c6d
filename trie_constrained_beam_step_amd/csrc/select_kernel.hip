// select_kernel.hip -- the per-request part of one trie-constrained beam step.
//
// One workgroup per request.  Each live row left its best s candidate keys
// (its summary), its number of finite candidates and its normaliser lse:
//   1. the K-th best summary key is a lower bound tau on the request's K-th
//      best candidate (the summaries are K or more of its candidates);
//   2. a row whose worst summary key is below tau, whose summary holds all its
//      candidates, or whose summary is at least K long, has every candidate
//      that can still be selected in its summary; the candidates of the few
//      other rows are recomputed exactly from the logits, with the same fp32
//      c = S_j + (x_v - lse_j) as the row kernel;
//   3. the candidates at or above tau go to LDS, where an exact radix select
//      keeps the K best, which are ranked (keys are unique) and decoded into
//      the new state: backpointer, token, score, next trie node, finished
//      flag, and the parent's sequence extended by the token (beamgrad README,
//      "How it works": the K best survive, EOS beams are carried unchanged;
//      sequences are -1 after they end).
// Every read is a flat, batched loop over (row, index) pairs found by binary
// search in an LDS prefix array, so loads are independent.  If the
// candidates at or above tau do not fit in LDS the request selects straight
// from the summaries and recomputed rows (exact, slower; counted in the step
// statistics).
#include "device_common.h"

namespace gr {
namespace {

enum { kSelN = 4, kSurv = 5 };
constexpr int kBatch = 8;                  // independent loads in flight per thread
constexpr uint64_t kSummaryRow = ~0ull;    // rw[j] after step 2: read the summary

template <typename DT>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(StepArgs a) {
    constexpr int NT = kSelectThreads;
    extern __shared__ __align__(16) uint8_t lds[];
    const int L = a.L, K = a.K, s = a.s;
    long long* red = reinterpret_cast<long long*>(lds);                 // 16
    int* misc = reinterpret_cast<int*>(red + 16);                       // 32: 16 + wave sums
    uint32_t* hist = reinterpret_cast<uint32_t*>(misc + 32);            // 256
    uint64_t* rw = reinterpret_cast<uint64_t*>(hist + 256);             // L: worst summary key, then edge base
    uint64_t* buf = rw + L;                                             // sb
    uint64_t* sel = buf + a.sb;                                         // K
    int* rcnt = reinterpret_cast<int*>(sel + K);                        // L
    int* pre = rcnt + L;                                                // L + 1

    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int32_t* cnt = a.cnt + (size_t)b * L;
    const uint64_t* summ = a.pool + (size_t)b * L * s;
    const DT* logits = reinterpret_cast<const DT*>(a.logits);

    long long tot = 0, nsum = 0, rows = 0;
    for (int j = tid; j < L; j += NT) {
        const int c = cnt[j];
        rcnt[j] = c;
        tot += c;
        nsum += c < s ? c : s;
        rows += isnan(a.lse_o[(size_t)b * K + j]) ? 0 : 1;
        rw[j] = ~0ull;
    }
    tot = block_sum_ll<NT>(tot, red);
    nsum = block_sum_ll<NT>(nsum, red);
    rows = block_sum_ll<NT>(rows, red);

    auto prefix_of = [&](auto&& ext) {
        for (int j = tid; j < L; j += NT) pre[j] = ext(j);
        return block_exclusive_scan<NT>(pre, L, misc + 16);
    };
    auto row_of = [&](int g) {
        int lo = 0, hi = L;  // pre[lo] <= g < pre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= g) lo = mid; else hi = mid;
        }
        return lo;
    };
    // f(j, key) for the first pre[j+1]-pre[j] candidates of every row j: its
    // summary keys, or (rescan set, rw[j] = edge base) its recomputed keys
    auto visit = [&](int total, bool rescan, auto&& f) {
        for (int g0 = tid; g0 < total; g0 += NT * kBatch) {
            uint64_t k[kBatch];
            int jj[kBatch], ii[kBatch], vv[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int g = g0 + u * NT;
                jj[u] = -1;
                vv[u] = -1;
                k[u] = 0;
                if (g < total) {
                    const int j = row_of(g);
                    const int i = g - pre[j];
                    jj[u] = j;
                    ii[u] = i;
                    if (!rescan || rw[j] == kSummaryRow) k[u] = summ[(size_t)j * s + i];
                    else vv[u] = a.off ? a.tok[(int64_t)rw[j] + i] : i;
                }
            }
            if (rescan) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    if (vv[u] >= 0) {
                        const size_t ps = (size_t)b * K + jj[u];
                        const float x = load_elem<DT>(logits + ps * (size_t)a.stride, vv[u]);
                        const float c = __fadd_rn(a.score[ps], __fsub_rn(x, a.lse_o[ps]));
                        k[u] = c == -INFINITY
                                   ? 0ull
                                   : cand_key(ord_f32(c), (uint32_t)jj[u] * (uint32_t)a.F + (uint32_t)ii[u]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (k[u]) f(jj[u], k[u]);
        }
    };
    auto for_lds = [&](const uint64_t* p, int n) {
        return [=](auto&& f) {
            for (int i = tid; i < n; i += NT) f(p[i]);
        };
    };

    if (tid == 0) {
        misc[kSelN] = 0;
        misc[kSurv] = 0;
    }
    __syncthreads();

    // 1. tau: the K-th best summary key (0 when the summaries are fewer than
    //    K or do not fit in LDS); rw[j] = the row's worst summary key
    uint64_t tau = 0;
    if (nsum >= K && nsum <= a.sb) {
        const int n = prefix_of([&](int j) { return rcnt[j] < s ? rcnt[j] : s; });
        visit(n, false, [&](int j, uint64_t k) {
            buf[atomicAdd(&misc[kSelN], 1)] = k;
            atomicMin((unsigned long long*)&rw[j], (unsigned long long)k);
        });
        __syncthreads();
        tau = radix_threshold<NT>(for_lds(buf, n), (uint32_t)K, hist, misc);
    }
    // 2. rows to recompute: more candidates than their summary, a summary
    //    shorter than K, and all of it at or above tau
    int nres = 0;
    for (int j = tid; j < L; j += NT) {
        const int c = rcnt[j];
        uint64_t base = kSummaryRow;
        if (c > s && s < K && rw[j] >= tau) {
            const size_t ps = (size_t)b * K + j;
            base = a.off ? (uint64_t)a.off[a.node[ps]] : 0ull;
            ++nres;
        }
        rw[j] = base;
    }
    nres = (int)block_sum_ll<NT>(nres, red);
    const int n = prefix_of([&](int j) {
        if (rw[j] == kSummaryRow) return rcnt[j] < s ? rcnt[j] : s;
        if (!a.off) return a.V;
        const size_t ps = (size_t)b * K + j;
        const int32_t nd = a.node[ps];
        return (int)(a.off[nd + 1] - a.off[nd]);
    });
    // 3. everything at or above tau, then the exact K best
    if (tid == 0) misc[kSelN] = 0;
    __syncthreads();
    visit(n, nres > 0, [&](int, uint64_t k) {
        if (k >= tau) {
            const int p = atomicAdd(&misc[kSurv], 1);
            if (p < a.sb) buf[p] = k;
        }
    });
    __syncthreads();
    const long long nsurv = misc[kSurv];
    int slow = 0;
    if (nsurv <= a.sb) {
        uint64_t theta = 0;
        if (nsurv > K) theta = radix_threshold<NT>(for_lds(buf, (int)nsurv), (uint32_t)K, hist, misc);
        for (int i = tid; i < (int)nsurv; i += NT)
            if (buf[i] >= theta) sel[atomicAdd(&misc[kSelN], 1)] = buf[i];
    } else {
        slow = 1;
        auto all = [&](auto&& f) {
            visit(n, nres > 0, [&](int, uint64_t k) {
                if (k >= tau) f(k);
            });
        };
        const uint64_t theta = radix_threshold<NT>(all, (uint32_t)K, hist, misc);
        all([&](uint64_t k) {
            if (k >= theta) sel[atomicAdd(&misc[kSelN], 1)] = k;
        });
    }
    __syncthreads();
    const int nsel = misc[kSelN];

    // 4. rank (keys are unique), decode and write the new state
    const int T = a.T, t = a.t;
    for (int i = tid; i < nsel; i += NT) {
        const uint64_t key = sel[i];
        int r = 0;
        for (int m = 0; m < nsel; ++m) r += sel[m] > key ? 1 : 0;
        const uint32_t flat = ~(uint32_t)key;
        const int j = (int)(flat / (uint32_t)a.F);
        const int ci = (int)(flat - (uint32_t)j * (uint32_t)a.F);
        const size_t ps = (size_t)b * K + j;
        int tokn, nd;
        uint8_t f;
        if (a.fin[ps]) {
            tokn = -1; nd = -1; f = 1;
        } else if (a.off) {
            const int64_t e = a.off[a.node[ps]] + ci;
            tokn = a.tok[e]; nd = a.child[e]; f = 0;
        } else {
            tokn = ci; nd = -1; f = (uint8_t)(ci == a.eos);
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
        atomicAdd(&a.stats[1], (unsigned long long)tot);
        atomicAdd(&a.stats[2], (unsigned long long)nsurv);
        atomicAdd(&a.stats[3], (unsigned long long)slow);
        atomicAdd(&a.stats[4], (unsigned long long)nres);
    }
}

}  // namespace

size_t select_lds_bytes(int sb, int K, int L) {
    return 16 * sizeof(long long) + 32 * sizeof(int) + 256 * sizeof(uint32_t) +
           (size_t)L * sizeof(uint64_t) + (size_t)(sb + K) * sizeof(uint64_t) +
           (size_t)(2 * L + 1) * sizeof(int);
}

hipError_t launch_select(const StepArgs& a, int bf16, hipStream_t st) {
    const size_t lds = select_lds_bytes(a.sb, a.K, a.L);
    if (bf16) select_kernel<uint16_t><<<dim3((unsigned)a.B), kSelectThreads, lds, st>>>(a);
    else select_kernel<float><<<dim3((unsigned)a.B), kSelectThreads, lds, st>>>(a);
    return hipGetLastError();
}

hipError_t set_select_lds_limit(int bytes) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel<float>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    hipError_t e2 = hipFuncSetAttribute((const void*)select_kernel<uint16_t>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return e != hipSuccess ? e : e2;
}

}  // namespace gr
