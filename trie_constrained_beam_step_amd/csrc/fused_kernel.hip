// fused_kernel.hip -- trie-constrained beam steps over short rows (a few KB
// of logits per beam), with no per-row summary.
//
// The step computes what the row kernel and the request kernel compute
// together (log-softmax normaliser over each live row, the CSR children of
// the row's trie node as candidates, c = S_j + (x_v - lse_j) in fp32, the K
// best of each request under (higher c, lower j*V + v), and the new state;
// FlashRec README, "Decoding"; beamgrad README, "How it works"), organised
// for rows too short to keep a 256-thread workgroup busy:
//   1. fused_kernel: the L rows of request b are split over fw workgroups
//      (rpw rows each); each wave of a workgroup takes whole rows: it
//      streams the row, folds its log-sum-exp in registers, gathers the
//      children's logits (their token ids are fetched before the stream,
//      their logits as soon as the stream's first loads are in flight) and
//      appends every finite candidate's 64-bit key to the workgroup's LDS
//      buffer -- no per-row selection and no per-row summary.
//      With one workgroup per request (fw = 1) it then selects, ranks and
//      decodes the request's K best itself: the whole step is one launch.
//      Otherwise it keeps its K best (a radix select over the buffer),
//      raises the request's running bound (a 64-bit atomic maximum) with its
//      own K-th best key -- every workgroup's K-th best is at most the
//      request's -- and writes its keys at or above that bound;
//   2. merge_kernel (fw > 1): one 1,024-thread workgroup per request gathers
//      the workgroups' keys at or above the final bound (compacting back to
//      the K best whenever the next chunk might not fit), ranks the K best
//      and decodes them; it resets the bound for the next step.
// The keys are those of the row and request kernels (ordered fp32 score,
// then the complement of j*F + i, i the candidate's edge ordinal in its
// node), so the results are identical to theirs.  The host takes this path
// only for CSR trie levels, unperturbed ranking (no sampling, length penalty
// or masks), the full-row normaliser, K <= kFusedCap / 2, rows of at most
// kFusedMaxRow logits and rpw x (the level's largest fan-out) <= kFusedCap,
// so no buffer can overflow.
#include "row_stream.h"

namespace gr {
namespace {

// LDS ints: candidate count, kept count, rows, finite candidates, claims;
// [16..18] the radix select's scratch
enum { fCount = 0, fKept = 2, fRows = 3, fFin = 4, fClaim = 5, fMisc = 16 };
// LDS 64-bit words ahead of those: [8..11] broadcasts; bucket_cut uses
// [0 .. 2 * waves) in between (32 for 1,024 threads)
constexpr int kRed = 32;
constexpr int kMergeThreads = 1024;
constexpr int kMergeCap = 16384;         // the merge kernel's LDS key buffer

// The request's K best of the n <= NT * PER candidate keys in buf (after a
// barrier), ranked best first (keys are unique: a key's rank is the number
// of better keys, counted for small selections, else by a bitonic sort) and
// decoded into the new state: parent slot, token, score, next trie node and
// the parent's sequence extended by the token; slots past the candidates
// become empty, rows past the live bound get no normaliser; then the
// request's step counters.
template <int NT, int PER>
__device__ void finish_request(const StepArgs& a, int b, uint64_t* buf, int n, uint32_t* hist, int* misc,
                               double* red, long long rows, long long fin, long long survivors) {
    const int tid = threadIdx.x;
    const int K = a.K, L = a.L, T = a.T, t = a.t;
    constexpr int Q = (kFusedCap / 2 + NT - 1) / NT;  // keys per thread the ranking holds
    if (n > K) {
        // a bucket cut keeps the K best and a few more (ranked below, the
        // extra ones not emitted); an exact radix select when too many remain
        int kept;
        const uint64_t cut = bucket_cut<NT>(buf, n, K, hist, misc + fMisc, reinterpret_cast<uint64_t*>(red), &kept);
        const int m = compact_ge<NT, PER>(buf, n, cut, &misc[fKept]);
        if (m <= Q * NT) {
            n = m;
        } else {
            const uint64_t th = radix_threshold<NT>(
                [&](auto&& g) {
                    for (int i = tid; i < m; i += NT) g(buf[i]);
                },
                (uint32_t)K, hist, misc + fMisc);
            n = compact_ge<NT, PER>(buf, m, th, &misc[fKept]);
        }
    }
    const int nsel = n;       // the keys ranked (their best K are the winners)
    const int nwin = min(n, K);
    // a winner's parent j, token and next node (the parent row's first edge
    // was stored by the rows), read apart from its rank so that the loads can
    // be in flight while the rank is counted
    constexpr int SQ = 8;  // sequence entries read ahead as well
    struct Won {
        int j;
        int32_t tok, nd;
        int32_t sq[SQ];
    };
    auto fetch = [&](uint64_t key) {
        const uint32_t flat = ~(uint32_t)key;
        Won d;
        d.j = (int)(flat / (uint32_t)a.F);
        const int ci = (int)(flat - (uint32_t)d.j * (uint32_t)a.F);
        const int64_t base = a.rbase[(size_t)b * L + d.j];
        d.tok = a.tok[base + ci];
        d.nd = a.child[base + ci];
        const int32_t* sp = a.seq + ((size_t)b * K + d.j) * T;
#pragma unroll
        for (int q = 0; q < SQ; ++q) d.sq[q] = q < t ? sp[q] : -1;
        return d;
    };
    auto put = [&](uint64_t key, const Won& d, int r) {
        const int j = d.j;
        const int32_t tokn = d.tok, nd = d.nd;
        const size_t ps = (size_t)b * K + j;
        const size_t o = (size_t)b * K + r;
        a.score_o[o] = unord_f32((uint32_t)(key >> 32));
        a.node_o[o] = nd;
        a.fin_o[o] = 0;
        a.parent_o[o] = j;
        a.token_o[o] = tokn;
        const int32_t* sp = a.seq + ps * T;
        int32_t* so = a.seq_o + o * T;
#pragma unroll
        for (int q = 0; q < SQ; ++q)
            if (q < T) so[q] = q < t ? d.sq[q] : (q == t ? tokn : -1);
        for (int q = SQ; q < T; ++q) so[q] = q < t ? sp[q] : (q == t ? tokn : -1);
    };
    // ranks (keys are unique), by bucketing; each thread then holds keys of
    // the bucketed order and issues their decode loads before counting
    uint64_t mine[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int i = tid + q * NT;
        mine[q] = i < nsel ? buf[i] : 0ull;
    }
    constexpr int QP = NT >= 1024 ? Q : 1;  // keys whose decode loads go out early (registers permitting)
    Won dq[QP];
    int rk[Q];
    bucket_ranks<NT, Q>(buf, nsel, mine, rk, hist, reinterpret_cast<int*>(buf + kFusedCap / 2), buf + kFusedCap / 2 + 128,
                        [&](int q, uint64_t key) {
                            if (q < QP) dq[q < QP ? q : 0] = fetch(key);
                        });
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (rk[q] >= 0 && rk[q] < K) {
            if (q < QP) put(mine[q], dq[q < QP ? q : 0], rk[q]);
            else put(mine[q], fetch(mine[q]), rk[q]);
        }
    }
    for (int r = nwin + tid; r < K; r += NT) {
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
        unsigned long long* st = a.stats + (size_t)b * kNumStats;
        st[0] = (unsigned long long)rows;
        st[1] = (unsigned long long)fin;
        st[2] = (unsigned long long)survivors;
        st[3] = 0;
        st[4] = 0;
        st[5] = 1;
    }
}

// The exact normaliser of a one-wave row (the rare fallback), out of line:
// its fp64 routines' constants stay out of the row loop's registers.
template <typename DT>
__device__ __attribute__((noinline)) float row_exact_lse(const DT* row, int V, int lane, double* red) {
    return exact_lse<64>(
        [&](auto&& g) {
            for (int64_t q = lane; q < V; q += 64) g(load_elem<DT>(row, q));
        },
        1.0f, red);
}

constexpr int kMetaRows = 16;  // rows per wave whose score and child range are read at once

// The fused step's body: Split = false for one workgroup per request (it
// finishes the request), true for a request split over fw > 1 workgroups.
template <typename DT, bool Split>
__device__ __forceinline__ void fused_body(const StepArgs& a) {
    constexpr int NT = kFusedThreads, NW = NT / 64, E = kAdmitPerThread, MR = kMetaRows;
    extern __shared__ __align__(16) uint8_t lds[];
    double* red = reinterpret_cast<double*>(lds);                   // kRed
    int* misc = reinterpret_cast<int*>(red + kRed);                  // 32
    uint32_t* hist = reinterpret_cast<uint32_t*>(misc + 32);         // 256
    uint64_t* buf = reinterpret_cast<uint64_t*>(hist + 256);         // fcap keys (8-byte aligned)
    int64_t* mE0 = reinterpret_cast<int64_t*>(buf + a.fcap);         // MR rows per wave: first edge,
    float* mS = reinterpret_cast<float*>(mE0 + NW * MR);             // parent score (-inf: empty slot),
    int* mF = reinterpret_cast<int*>(mS + NW * MR);                  // fan-out

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fw = a.fw;
    const int b = blockIdx.x / fw, w = blockIdx.x - b * fw;
    const int K = a.K;
    const int j0 = w * a.rpw, j1 = min(a.L, j0 + a.rpw);
    const float kNaN = __uint_as_float(0x7FC00000u);
    const DT* logits = reinterpret_cast<const DT*>(a.logits);
    if (tid < 16) misc[tid] = 0;
    __syncthreads();

    // 1. the workgroup's rows, one per wave at a time.  A wave reads the
    // score and child range of MR of its rows at once (lane l: row l of the
    // block) into its LDS slots; a row's child token ids are read while the
    // previous row streams; so a row costs about one memory round trip
    // instead of a chain of four.
    const int nr = j1 - j0 > wave ? (j1 - j0 - wave + NW - 1) / NW : 0;  // the wave's rows
    mE0 += wave * MR;
    mS += wave * MR;
    mF += wave * MR;
    auto load_meta = [&](int i0) {  // the wave's rows i0 .. i0 + MR - 1
        const int i = i0 + lane;
        float S = -INFINITY;
        int64_t e0 = 0;
        int f = 0;
        if (lane < MR && i < nr) {
            const int slot = b * K + j0 + wave + NW * i;
            const float Sl = a.score[slot];
            const uint8_t fin = a.fin[slot];
            const int32_t n = a.node[slot];
            if (Sl != -INFINITY && !fin) {  // (a finished flag has no EOS to carry here)
                S = Sl;
                if (n >= 0 && n < a.nnodes) {
                    e0 = a.off[n];
                    f = (int)(a.off[n + 1] - e0);
                }
            }
        }
        if (lane < MR) {  // (read back by the same wave only: no barrier)
            mS[lane] = S;
            mE0[lane] = e0;
            mF[lane] = f;
        }
    };
    auto load_tok = [&](int i, int32_t* c) {  // the first E*64 child tokens of the wave's row i
        const int64_t e0 = mE0[i % MR];
        const int f = mF[i % MR];
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int ci = lane + 64 * k;
            c[k] = ci < f ? a.tok[e0 + ci] : -1;
        }
    };
    int rows = 0;
    long long nfin = 0;
    int32_t cv[E];
    load_meta(0);
    if (nr > 0) load_tok(0, cv);
    for (int i = 0; i < nr; ++i) {
        const int j = j0 + wave + NW * i, slot = b * K + j;
        const float S = mS[i % MR];
        const int64_t e0 = mE0[i % MR];
        const int f = mF[i % MR];
        const bool more = i + 1 < nr;
        if (i % MR == MR - 1 && more) load_meta(i + 1);  // the next block (this row's values are read)
        int32_t cn[E];
#pragma unroll
        for (int k = 0; k < E; ++k) cn[k] = -1;
        if (S == -INFINITY) {  // empty
            if (lane == 0) a.lse_o[slot] = kNaN;
            if (more) load_tok(i + 1, cv);
            continue;
        }
        const DT* row = logits + (size_t)slot * (size_t)a.stride;
        if (lane == 0) a.rbase[(size_t)b * a.L + j] = e0;  // (the winners' decode reads it)
        float xv[E];
        float Rr = kFarBelow, sp = 0.0f, tmax = -INFINITY;
        int ninf = 0;
        DrawCtx dc;
        stream_row<DT, 64, short_row_batch<DT>(), kPlain, true>(
            row, a.V, lane, kLog2e, Rr, sp,
            [&] {
#pragma unroll
                for (int k = 0; k < E; ++k) xv[k] = cv[k] >= 0 ? load_elem<DT>(row, cv[k]) : 0.0f;
                if (more) load_tok(i + 1, cn);
            },
            nullptr, ninf, tmax, dc);
        double Rtop;
        float lse = block_lse<64, true>(Rr, sp, red, Rtop);
        if (fabs(Rtop) >= 0x1p30)  // rare: logits beyond the fused reference's range
            lse = row_exact_lse<DT>(row, a.V, lane, red);
        if (lane == 0) a.lse_o[slot] = lse;
        ++rows;
        if (lse != -INFINITY) {  // (no finite logit: no finite candidate)
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
#pragma unroll
        for (int k = 0; k < E; ++k) cv[k] = cn[k];
    }
    // the workgroup's counts
    nfin = wave_sum_ll(nfin);
    if (lane == 0) {
        atomicAdd(&misc[fRows], rows);
        atomicAdd(&misc[fFin], (int)nfin);
    }
    __syncthreads();
    const int n = min(misc[fCount], a.fcap);
    if constexpr (!Split) {  // the workgroup holds the whole request: finish it here
        finish_request<NT, kFusedCap / NT>(a, b, buf, n, hist, misc, red, misc[fRows], misc[fFin], min(n, K));
        return;
    }

    // 2. its K best (and the K-th's bucket mates), at or above the
    // request's running bound, for the merge
    uint64_t th = 0;
    if (n > K) {
        int kept;
        th = bucket_cut<NT>(buf, n, K, hist, misc + fMisc, reinterpret_cast<uint64_t*>(red), &kept);
        if (kept > K * kPartPerK)  // too many bucket mates for the slots: the exact K-th
            th = radix_threshold<NT>(
                [&](auto&& g) {
                    for (int i = tid; i < n; i += NT) g(buf[i]);
                },
                (uint32_t)K, hist, misc + fMisc);
    }
    if (tid == 0) {
        const unsigned long long old = atomicMax(&a.req_theta[b], (unsigned long long)th);
        const uint64_t cut = old > th ? old : th;
        red[8] = __longlong_as_double((long long)cut);
        misc[fKept] = 0;
    }
    __syncthreads();
    const uint64_t cut = (uint64_t)__double_as_longlong(red[8]);
    uint64_t* dst = a.part + ((size_t)b * fw + w) * K * kPartPerK;
    for (int i = tid; i < n; i += NT) {
        const bool keep = buf[i] >= cut;
        const int p = wave_claim(&misc[fKept], keep);
        if (keep) dst[p] = buf[i];
    }
    __syncthreads();
    if (tid == 0) {
        const size_t pw = (size_t)b * fw + w;
        a.part_n[pw] = misc[fKept];
        a.part_stats[2 * pw] = misc[fRows];
        a.part_stats[2 * pw + 1] = misc[fFin];
    }
}

// One workgroup per request (fw = 1): the whole step in one launch.
template <typename DT>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(4))) void fused_step_kernel(
    StepArgs a) {
    fused_body<DT, false>(a);
}

// Several steps of a search in one launch, each a one-workgroup fused step
// (fw = 1): a request's workgroup runs them in order, each step reading the
// state the previous one wrote.  Between steps: every wave waits for its
// memory operations to complete (its stores have reached L2), a barrier,
// then an agent-scope acquire fence, so that no vector L1 line read by an
// earlier step serves the new state.  Three waves per
// SIMD: the per-thread values the compiler keeps across the steps take
// 133 registers in the fp32 kernel.
template <typename DT>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(3))) void fused_search_kernel(
    SearchArgs sa) {
    for (int i = 0; i < sa.n; ++i) {
        if (i > 0) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        fused_body<DT, false>(sa.step[i]);
    }
}

// fw > 1 workgroups per request: rows, then each workgroup's kept keys for
// the merge kernel.  Without the request's selection, ranking and decoding
// it needs fewer registers, and more of its waves fit on a CU.
template <typename DT>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(kFusedRowsWaves))) void fused_rows_kernel(
    StepArgs a) {
    fused_body<DT, true>(a);
}

// One workgroup per request of a split step: the workgroups' kept keys at or
// above the request's final bound, gathered in chunks of kMergeCap - K
// (compacting back to the K best whenever the next chunk might not fit),
// then the K best, ranked and decoded.  The bound goes back to 0.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(StepArgs a) {
    constexpr int NT = kMergeThreads;
    extern __shared__ __align__(16) uint8_t lds[];
    double* red = reinterpret_cast<double*>(lds);                   // kRed
    int* misc = reinterpret_cast<int*>(red + kRed);                  // 32
    uint32_t* hist = reinterpret_cast<uint32_t*>(misc + 32);         // 256
    int* pre = reinterpret_cast<int*>(hist + 256);                   // kFusedMaxW + 2
    uint64_t* buf = reinterpret_cast<uint64_t*>(pre + kFusedMaxW + 2);  // kMergeCap keys
    const int tid = threadIdx.x;
    const int b = blockIdx.x, fw = a.fw, K = a.K;
    if (tid < 64) {  // lane q: workgroup q's kept count and counters (fw <= 64)
        const unsigned long long th = tid == 0 ? atomicExch(&a.req_theta[b], 0ull) : 0ull;
        int nq = 0;
        long long rq = 0, fq = 0;
        if (tid < fw) {
            const size_t pw = (size_t)b * fw + tid;
            nq = a.part_n[pw];
            rq = a.part_stats[2 * pw];
            fq = a.part_stats[2 * pw + 1];
        }
        const int inc = (int)wave_inclusive_scan((uint32_t)nq);
        if (tid < fw) pre[tid] = inc - nq;
        if (tid == 63) pre[fw] = inc;
        const long long rsum = wave_sum_ll(rq), fsum = wave_sum_ll(fq);
        // the workgroups' K best (not what the running bound let through:
        // that depends on the order they finished)
        const long long ksum = wave_sum_ll(fq < K ? fq : (long long)K);
        if (tid == 0) {
            red[8] = __longlong_as_double((long long)th);
            red[9] = __longlong_as_double(rsum);
            red[10] = __longlong_as_double(fsum);
            red[11] = __longlong_as_double(ksum);
            misc[fCount] = 0;
        }
    }
    __syncthreads();
    uint64_t bound = (uint64_t)__double_as_longlong(red[8]);
    const int N = pre[fw];
    const int chunk = kMergeCap - K;
    int n = 0;
    for (int g0 = 0; g0 < N; g0 += chunk) {
        const int g1 = min(N, g0 + chunk);
        constexpr int GB = 4;  // keys whose loads a thread has in flight together
        for (int gb = g0 + tid; gb < g1; gb += GB * NT) {
            uint64_t kk[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const int g = gb + u * NT;
                kk[u] = 0ull;
                if (g < g1) {
                    int lo = 0, hi = fw;  // pre[lo] <= g < pre[hi]
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (pre[mid] <= g) lo = mid; else hi = mid;
                    }
                    kk[u] = a.part[((size_t)b * fw + lo) * K * kPartPerK + (g - pre[lo])];
                }
            }
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const bool keep = gb + u * NT < g1 && kk[u] >= bound;
                const int p = wave_claim(&misc[fCount], keep);
                if (keep && p < kMergeCap) buf[p] = kk[u];  // (the chunks keep p below the buffer)
            }
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
            n = compact_ge<NT, kMergeCap / NT>(buf, n, th, &misc[fKept]);
            if (tid == 0) misc[fCount] = n;
            __syncthreads();
        }
    }
    finish_request<NT, kMergeCap / NT>(a, b, buf, n, hist, misc, red, __double_as_longlong(red[9]),
                                       __double_as_longlong(red[10]), __double_as_longlong(red[11]));
}

}  // namespace

size_t fused_lds_bytes(int fcap, int fw) {
    (void)fw;
    return kRed * sizeof(double) + 32 * sizeof(int) + 256 * sizeof(uint32_t) + (size_t)fcap * sizeof(uint64_t) +
           (size_t)(kFusedThreads / 64) * kMetaRows * (sizeof(int64_t) + sizeof(float) + sizeof(int));
}

static size_t merge_lds_bytes() {
    return kRed * sizeof(double) + 32 * sizeof(int) + 256 * sizeof(uint32_t) + (size_t)(kFusedMaxW + 2) * sizeof(int) +
           (size_t)kMergeCap * sizeof(uint64_t);
}

hipError_t launch_fused(const StepArgs& a, int bf16, hipStream_t st) {
    const size_t lds = fused_lds_bytes(a.fcap, a.fw);
    const dim3 grid((unsigned)(a.B * a.fw));
    if (a.fw == 1) {
        if (bf16) fused_step_kernel<uint16_t><<<grid, kFusedThreads, lds, st>>>(a);
        else fused_step_kernel<float><<<grid, kFusedThreads, lds, st>>>(a);
    } else {
        if (bf16) fused_rows_kernel<uint16_t><<<grid, kFusedThreads, lds, st>>>(a);
        else fused_rows_kernel<float><<<grid, kFusedThreads, lds, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_fused_search(const SearchArgs& sa, int bf16, hipStream_t st) {
    size_t lds = 0;
    for (int i = 0; i < sa.n; ++i) lds = lds > fused_lds_bytes(sa.step[i].fcap, 1) ? lds : fused_lds_bytes(sa.step[i].fcap, 1);
    const dim3 grid((unsigned)sa.step[0].B);
    if (bf16) fused_search_kernel<uint16_t><<<grid, kFusedThreads, lds, st>>>(sa);
    else fused_search_kernel<float><<<grid, kFusedThreads, lds, st>>>(sa);
    return hipGetLastError();
}

hipError_t launch_merge(const StepArgs& a, hipStream_t st) {
    merge_kernel<<<dim3((unsigned)a.B), kMergeThreads, merge_lds_bytes(), st>>>(a);
    return hipGetLastError();
}

hipError_t set_fused_lds_limit(int bytes) {
    return allow_dynamic_lds((const void*)merge_kernel, bytes);
}

hipError_t launch_step(const StepArgs& a, int bf16, hipStream_t st) {
    if (a.fw > 0) {
        hipError_t e = launch_fused(a, bf16, st);
        if (e == hipSuccess && a.fw > 1) e = launch_merge(a, st);
        return e;
    }
    hipError_t e = launch_rows(a, bf16, st);
    return e != hipSuccess ? e : launch_select(a, bf16, st);
}

}  // namespace gr
