// select_kernel.hip -- the per-request part of one trie-constrained beam step.
//
// One workgroup per request.  Each live row j left its best s candidate keys
// (its summary) at slots j*s .. j*s+s-1, its number of finite candidates, its
// fan-out, its first edge and the worst key of its summary:
//   1. the score halves (high 32 bits) of the summary keys are loaded into
//      LDS as one grid of L*s slots; tau, their K-th largest with its low 8
//      bits cleared, is a lower bound on the score half of the request's
//      K-th best candidate (the summaries are K or more of its candidates);
//   2. a row keeps its summary when the summary holds all its candidates, is
//      at least K long, or ends below tau (its other candidates are below the
//      summary's worst); the few other rows are listed and recomputed from the
//      logits, with the same fp32 c = S_j + (x_v - lse_j) as the row kernel;
//   3. the candidates at or above tau -- full keys of the kept summary slots,
//      read back from the pool, and those of the recomputed rows -- are
//      compacted in LDS, where an exact radix select keeps the K best, which
//      are ranked (keys are unique) and decoded into the new state:
//      backpointer, token, score, next trie node, finished flag, and the
//      parent's sequence extended by the token (beamgrad README, "How it
//      works": the K best survive, EOS beams are carried unchanged; sequences
//      are -1 after they end).
// Recomputed rows are read as one flat, batched loop over (row, index) pairs
// found by binary search in an LDS prefix over the rescan list, so loads are
// independent.  If the candidates at or above tau do not fit in LDS the
// request selects straight from the pool and recomputed rows (exact, slower;
// counted in the step statistics).
#include "device_common.h"

namespace gr {
namespace {

enum { kSelN = 4, kSurv = 5, kNres = 6 };
constexpr int kCountRankMax = 256;  // larger selections are ranked by bucketing
constexpr int kBatch = 8;  // independent loads in flight per thread
constexpr int kGridPerThread = kSelectMaxGrid / kSelectThreads;

template <typename DT>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(StepArgs a) {
    constexpr int NT = kSelectThreads;
    extern __shared__ __align__(16) uint8_t lds[];
    const int L = a.L, K = a.K, s = a.s, sh = a.s_log2;
    long long* red = reinterpret_cast<long long*>(lds);                 // 3 per wave, then 3 totals
    int* misc = reinterpret_cast<int*>(red + 3 * NT / 64 + 4);          // 32: 16 + wave sums
    uint32_t* hist = reinterpret_cast<uint32_t*>(misc + 32);            // 256
    int* rcur = reinterpret_cast<int*>(hist + 256);                     // 256: the ranking's bucket ends
    uint64_t* rwmm = reinterpret_cast<uint64_t*>(rcur + 256);           // 2 per wave: key ranges
    uint64_t* rw = rwmm + 2 * NT / 64;                                  // L: worst key, then first edge
    uint64_t* sel = rw + L;                                             // K
    int* rcnt = reinterpret_cast<int*>(sel + K);                        // L: finite count, -1 = recomputed
    int* rl = rcnt + L;                                                 // L: rescan list
    int* pre = rl + L;                                                  // L + 1: its prefix
    uint32_t* grid = reinterpret_cast<uint32_t*>(pre + L + 1);          // gs >= L*s
    // survivors: sb keys, in whatever the step's grid leaves of the LDS
    uint64_t* buf = reinterpret_cast<uint64_t*>(lds + ((reinterpret_cast<uint8_t*>(grid + a.gs) - lds + 7) & ~(size_t)7));

    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const size_t r0 = (size_t)b * L;  // first row id of the request
    const uint64_t* summ = a.pool + r0 * s;
    const uint32_t* summ_hi = reinterpret_cast<const uint32_t*>(summ) + 1;  // little-endian high words
    const DT* logits = reinterpret_cast<const DT*>(a.logits);
    const int ns = L * s;

    if (tid == 0) {
        misc[kSelN] = 0;
        misc[kSurv] = 0;
        misc[kNres] = 0;
    }
    // the summary grid's score halves are requested before the per-row
    // fields, so that both are in flight together; empty slots are cleared
    // once the rows' counts are known
    uint32_t gv[kGridPerThread];
#pragma unroll
    for (int u = 0; u < kGridPerThread; ++u) {
        const int q = tid + u * NT;
        gv[u] = q < ns ? summ_hi[2 * (size_t)q] : 0u;
    }
    long long tot = 0, nsum = 0, rows = 0;
    for (int j = tid; j < L; j += NT) {
        const int c = a.cnt[r0 + j];
        rcnt[j] = c;
        rw[j] = a.rworst[r0 + j];
        tot += c;
        nsum += c < s ? c : s;
        rows += a.rbase[r0 + j] >= 0 ? 1 : 0;
    }
    long long* totals = red + 3 * NT / 64;  // candidates, summary keys, rows read
    block_sum3_ll<NT>(tot, nsum, rows, red, totals);
    nsum = totals[1];

    // 1. the grid of summary score halves (0 = empty slot), and tau: a lower
    //    bound on their K-th largest (that value with its low 8 bits cleared:
    //    three radix passes instead of four; every use of tau is
    //    conservative), or 0 when the summaries are fewer than K
#pragma unroll
    for (int u = 0; u < kGridPerThread; ++u) {
        const int q = tid + u * NT;
        if (q < ns) {
            const int c = rcnt[q >> sh];
            grid[q] = (q & (s - 1)) < (c < s ? c : s) ? gv[u] : 0u;
        }
    }
    __syncthreads();
    uint32_t tau32 = 0;
    if (nsum >= K) {
        tau32 = radix_threshold<NT, uint32_t>(
            [&](auto&& f) {
#pragma unroll 8
                for (int u = 0; u < kGridPerThread; ++u) {
                    const int q = tid + u * NT;
                    if (q < ns) {
                        const uint32_t o = grid[q];
                        if (o) f(o);
                    }
                }
            },
            (uint32_t)K, hist, misc, 8);
    }
    const uint64_t tau = (uint64_t)tau32 << 32;

    // 2. rows to recompute: more candidates than their summary, a summary
    //    shorter than K, and all of it at or above tau
    for (int j = tid; j < L; j += NT) {
        const int c = rcnt[j];
        const bool res = c > s && s < K && rw[j] >= tau;
        rw[j] = (uint64_t)a.rbase[r0 + j];
        if (res) rcnt[j] = -1;
        const int p = wave_claim(&misc[kNres], res);
        if (res) {
            rl[p] = j;
            pre[p] = a.ncand[r0 + j];
        }
    }
    __syncthreads();
    const int nres = misc[kNres];
    const int total = block_exclusive_scan<NT>(pre, nres, misc + 16);

    // ranking score of live candidate (j, token v): c, divided by the length
    // penalty, plus its Gumbel draw when sampling; tokens not emitted this step
    auto rank = [&](float c, int j, int v) {
        float k = a.penal ? __fdiv_rn(c, a.pen_live) : c;
        if (a.sampling) k = __fadd_rn(k, gumbel_noise(a.seed, b, a.t, (uint32_t)j * (uint32_t)a.V + (uint32_t)v));
        return k;
    };
    auto masked = [&](int v) {
        return (a.banned && ((a.banned[v >> 5] >> (v & 31)) & 1u)) || (v == a.eos && a.t + 1 < a.min_len) ||
               v < a.nlo || v >= a.nhi;
    };
    // Sampled rows: a recomputed candidate whose fast draw estimate (within
    // kDrawErr of its exact draw) leaves its rank clearly below tau is
    // dropped before the exact fp64 draw -- only keys at or above tau are
    // ever used.  |exact rank - estimate| <= kDrawErr + 2^-22 |estimate| (the
    // two fp32 roundings of the sum), plus one smallest normal for safety.
    const float tau_f = unord_f32(tau32);
    auto below_tau = [&](float c, int j, int v) {
        if (!a.sampling || tau32 == 0) return false;
        const float kf = a.penal ? __fdiv_rn(c, a.pen_live) : c;
        const float est = __fadd_rn(kf, gumbel_fast_one(a.seed, b, a.t, (uint32_t)j * (uint32_t)a.V + (uint32_t)v));
        return est + (kDrawErr + 0x1p-22f * fabsf(est) + 0x1p-126f) < tau_f;
    };
    // f(key) for every finite candidate of the recomputed rows (sampled rows:
    // those that can reach tau)
    auto rescan = [&](auto&& f) {
        for (int g0 = tid; g0 < total; g0 += NT * kBatch) {
            int jj[kBatch], ii[kBatch], vv[kBatch];
            float sc[kBatch], ls[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int g = g0 + u * NT;
                vv[u] = -1;
                sc[u] = 0.0f;
                ls[u] = 0.0f;
                if (g < total) {
                    int lo = 0, hi = nres;  // pre[lo] <= g < pre[hi]
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (pre[mid] <= g) lo = mid; else hi = mid;
                    }
                    const int j = rl[lo];
                    const int i = g - pre[lo];
                    // (a dense trie level: code i, if the node has that child)
                    vv[u] = !a.off ? a.nlo + i
                            : a.dspan ? (a.child[(int64_t)rw[j] + i] >= 0 ? a.dbase + i : -1)
                                      : a.tok[(int64_t)rw[j] + i];
                    jj[u] = j;
                    ii[u] = a.off ? i : vv[u];  // the candidate's ordinal in its row
                    sc[u] = a.score[(size_t)b * K + j];
                    ls[u] = a.lse_o[(size_t)b * K + j];
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (vv[u] >= 0 && !masked(vv[u])) {
                    const size_t ps = (size_t)b * K + jj[u];
                    const float x = load_elem<DT>(logits + ps * (size_t)a.stride, vv[u]);
                    const float c = __fadd_rn(sc[u], __fsub_rn(__fmul_rn(x, a.inv_t), ls[u]));
                    if (c != -INFINITY && !below_tau(c, jj[u], vv[u]))
                        f(cand_key(ord_f32(rank(c, jj[u], vv[u])), (uint32_t)jj[u] * (uint32_t)a.F + (uint32_t)ii[u]));
                }
            }
        }
    };
    // a kept summary slot whose key is at or above tau
    auto kept_slot = [&](int q) {
        const uint32_t o = grid[q];
        return o != 0 && o >= tau32 && rcnt[q >> sh] >= 0;
    };

    // 3. everything at or above tau: the kept summary slots (listed, then
    //    their full keys read back in one batch), then the recomputed rows
#pragma unroll 8
    for (int u = 0; u < kGridPerThread; ++u) {
        const int q = tid + u * NT;
        const bool keep = q < ns && kept_slot(q);
        const int p = wave_claim(&misc[kSurv], keep);
        if (keep && p < a.sb) buf[p] = (uint64_t)q;
    }
    __syncthreads();
    {
        const int n1 = misc[kSurv] < a.sb ? misc[kSurv] : a.sb;
        for (int i = tid; i < n1; i += NT) buf[i] = summ[buf[i]];
    }
    rescan([&](uint64_t k) {
        const bool keep = k >= tau;
        const int p = wave_claim(&misc[kSurv], keep);
        if (keep && p < a.sb) buf[p] = k;
    });
    __syncthreads();
    const long long nsurv = misc[kSurv];
    int slow = 0;
    // the keys to rank (their best K win): in buf (the survivors, cut to the
    // K best and a few more) or in sel (the slow path's K best)
    constexpr int Q = 4096 / NT;  // keys per thread the ranking holds (K <= 4,096)
    uint64_t* rk_keys = buf;
    int nrk = 0;
    if (nsurv <= a.sb) {
        nrk = (int)nsurv;
        if (nrk > K) {
            // a bucket cut keeps the K best and the K-th's bucket mates; an
            // exact radix select when those would not fit the ranking
            int kept;
            uint64_t th = bucket_cut<NT>(buf, nrk, K, hist, misc, rwmm, &kept);
            if (kept > Q * NT)
                th = radix_threshold<NT>(
                    [&](auto&& f) {
                        for (int i = tid; i < nrk; i += NT) f(buf[i]);
                    },
                    (uint32_t)K, hist, misc);
            nrk = compact_ge<NT, kSelectMaxSurvivors / NT>(buf, nrk, th, &misc[kSelN]);
        }
    } else {
        // the survivors overflow the buffer; nsurv counts every one of them,
        // so fewer than K (the buffer may be shorter than K at the largest
        // widths) are all kept, without a selection
        slow = 1;
        auto all = [&](auto&& f) {
            for (int q = tid; q < ns; q += NT)
                if (kept_slot(q)) f(summ[q]);
            rescan([&](uint64_t k) {
                if (k >= tau) f(k);
            });
        };
        const uint64_t theta = nsurv > K ? radix_threshold<NT>(all, (uint32_t)K, hist, misc) : 0ull;
        all([&](uint64_t k) {
            const bool keep = k >= theta;
            const int p = wave_claim(&misc[kSelN], keep);
            if (keep) sel[p] = k;
        });
        __syncthreads();
        rk_keys = sel;
        nrk = misc[kSelN];
    }
    const int nsel = nrk < K ? nrk : K;  // the winners

    // 4. rank (keys are unique: counted for a few keys, else bucket_ranks),
    //    decode the K best and write the new state.
    const int T = a.T, t = a.t;
    auto decode = [&](uint64_t key, int r) {
        const uint32_t flat = ~(uint32_t)key;
        const int j = (int)(flat / (uint32_t)a.F);
        const int ci = (int)(flat - (uint32_t)j * (uint32_t)a.F);
        const size_t ps = (size_t)b * K + j;
        const int64_t base = (int64_t)rw[j];
        int tokn, nd;
        uint8_t f;
        if (base < 0) {  // finished beam, carried
            tokn = -1; nd = -1; f = 1;
        } else if (a.off) {
            tokn = a.dspan ? a.dbase + ci : a.tok[base + ci]; nd = a.child[base + ci]; f = 0;
        } else {
            tokn = ci; nd = -1; f = (uint8_t)(ci == a.eos);
        }
        const size_t o = (size_t)b * K + r;
        float score = unord_f32((uint32_t)(key >> 32));
        if (!a.rank_is_c) {  // the key ranks by the penalised / perturbed score; keep c
            if (base < 0) {
                score = a.score[ps];
            } else {
                const int v = a.off ? tokn : ci;
                const float x = load_elem<DT>(logits + ps * (size_t)a.stride, v);
                score = __fadd_rn(a.score[ps], __fsub_rn(__fmul_rn(x, a.inv_t), a.lse_o[ps]));
            }
        }
        a.score_o[o] = score;
        a.node_o[o] = nd;
        a.fin_o[o] = f;
        a.parent_o[o] = j;
        a.token_o[o] = tokn;
        const int32_t* sp = a.seq + ps * T;
        int32_t* so = a.seq_o + o * T;
        for (int q = 0; q < T; ++q) so[q] = q < t ? sp[q] : (q == t ? tokn : -1);
    };
    if (nrk <= kCountRankMax) {
        // few keys: each key's rank counted directly, by G lanes of a wave
        // (no barrier; counting costs nrk^2 LDS reads)
        int G = 1;
        while (G < 64 && 2 * G * nrk <= NT) G *= 2;
        for (int i0 = 0; i0 < nrk; i0 += NT / G) {
            const int i = i0 + tid / G, part = tid % G;
            const uint64_t key = i < nrk ? rk_keys[i] : 0ull;
            int r = 0;
            if (i < nrk) {  // four independent LDS reads per round
                int m = part;
                for (; m + 3 * G < nrk; m += 4 * G)
                    r += (rk_keys[m] > key ? 1 : 0) + (rk_keys[m + G] > key ? 1 : 0) +
                         (rk_keys[m + 2 * G] > key ? 1 : 0) + (rk_keys[m + 3 * G] > key ? 1 : 0);
                for (; m < nrk; m += G) r += rk_keys[m] > key ? 1 : 0;
            }
            for (int o = 1; o < G; o <<= 1) r += __shfl_xor(r, o);
            if (i < nrk && part == 0 && r < K) decode(key, r);
        }
    } else {
        uint64_t mine[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int i = tid + q * NT;
            mine[q] = i < nrk ? rk_keys[i] : 0ull;
        }
        int rk[Q];
        bucket_ranks<NT, Q>(rk_keys, nrk, mine, rk, hist, rcur, rwmm, [](int, uint64_t) {});
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (rk[q] >= 0 && rk[q] < K) decode(mine[q], rk[q]);
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
    if (tid == 0) {  // this request's counters (the host sums the requests)
        unsigned long long* st = a.stats + (size_t)b * kNumStats;
        st[0] = (unsigned long long)totals[2];
        st[1] = (unsigned long long)totals[0];
        st[2] = (unsigned long long)nsurv;
        st[3] = (unsigned long long)slow;
        st[4] = (unsigned long long)nres;
        st[5] = 0;
    }
}

}  // namespace

// LDS of the request kernel: fixed parts, the grid (gs slots), then the
// survivor buffer (sb keys, 8-byte aligned).
static size_t select_lds_head(int gs, int K, int L) {
    const size_t b = (3 * (kSelectThreads / 64) + 4) * sizeof(long long) + 32 * sizeof(int) +
                     256 * sizeof(uint32_t) + 256 * sizeof(int) + 2 * (kSelectThreads / 64) * sizeof(uint64_t) +
                     (size_t)(L + K) * sizeof(uint64_t) +
                     (size_t)(3 * L + 1) * sizeof(int) + (size_t)gs * sizeof(uint32_t);
    return (b + 7) & ~(size_t)7;
}

size_t select_lds_bytes(int gs, int sb, int K, int L) {
    return select_lds_head(gs, K, L) + (size_t)sb * sizeof(uint64_t);
}

int select_buffer_fit(size_t lds_bytes, int gs, int K, int L) {
    const size_t head = select_lds_head(gs, K, L);
    return lds_bytes > head ? (int)((lds_bytes - head) / sizeof(uint64_t)) : 0;
}

hipError_t launch_select(const StepArgs& a, int bf16, hipStream_t st) {
    const size_t lds = select_lds_bytes(a.gs, a.sb, a.K, a.L);
    if (bf16) select_kernel<uint16_t><<<dim3((unsigned)a.B), kSelectThreads, lds, st>>>(a);
    else select_kernel<float><<<dim3((unsigned)a.B), kSelectThreads, lds, st>>>(a);
    return hipGetLastError();
}

hipError_t set_select_lds_limit(int bytes) {
    hipError_t e = allow_dynamic_lds((const void*)select_kernel<float>, bytes);
    hipError_t e2 = allow_dynamic_lds((const void*)select_kernel<uint16_t>, bytes);
    return e != hipSuccess ? e : e2;
}

}  // namespace gr
