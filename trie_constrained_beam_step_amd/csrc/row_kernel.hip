// row_kernel.hip -- the per-row part of one trie-constrained beam step.
//
// One workgroup per possibly-live beam row (b, j):
//   (1) streams the row of V logits once from HBM with 16-byte non-temporal
//       loads, keeping a per-thread running max and a sum of exp2 terms in
//       fp32, combined across the workgroup in fp64 into the row's
//       log-sum-exp -- the log-softmax normaliser over the full row;
//   (2) walks the candidates of the row -- the CSR children of the slot's trie
//       node (FlashRec README, "Decoding"), or every token when unconstrained
//       (beamgrad README, "How it works") -- gathering their logits (cache-hot)
//       and forming c = S_j + (x_v - lse) in fp32;
//   (3) writes the row's best s candidates (its summary) and its number of
//       finite candidates.  The request kernel bounds its selection with the
//       summaries and recomputes the full candidate list of the few rows whose
//       whole summary clears that bound; with s >= K (or s >= the row's
//       candidates) no recomputation is ever needed.
// Rows holding at most E*NT candidates keep them in registers and pick the
// summary by ballot-count radix search.  Unconstrained rows with every token a
// candidate record batch maxima while streaming (of the logits, or of draw
// estimates when sampled) and read back only the batches that can hold their
// best s.  Other long rows go through an LDS buffer with radix-select
// compaction.
//
// A candidate is ordered by a 64-bit key: the order-preserving bit pattern of
// its fp32 score in the high word and the complement of j*F + i in the low
// word, where i is the candidate's ordinal in its row (the token id when
// unconstrained, F = V; the edge ordinal within the node's sorted children
// with a CSR trie level, F = the level's largest fan-out; the code index with
// a dense level, F = its token span).  Within a row the ordinal
// order is the token order, so a larger key is a better candidate under this
// library's order: higher score first, then lower flat index j*V + v.  (The
// beamgrad README, "Features", asks for a strict total order on candidates
// without fixing one; this tie-break is the library's definition.)  The
// request kernel finds the chosen edge without a search.  Keys are unique, so
// every selection is exact.
#include <type_traits>

#include "row_stream.h"

namespace gr {
namespace {

// LDS layout of the row kernel (bytes): red (16 doubles), misc (16 ints),
// hist (256 u32), then the candidate buffer (cap keys, cap token ids) and
// the compaction staging area (stg keys, stg ids).
enum { kCount = 4, kStage = 5, kPoolW = 6, kSumW = 7 };

constexpr int kFastSummary = 32;  // largest summary the register path selects

// Slice: the launch normalises each trie row over its node's children only
// (its own instantiation, so that the streaming kernel's registers are not
// shared with the slice's gathers).
// Row kernel variants: a streamed trie row; a trie row normalised over its
// node's children only (not streamed); an unconstrained sampled row, whose
// stream also bounds its candidates' ranks with fast Gumbel estimates; a
// streamed row of a dense trie level; an unconstrained unsampled row (every
// token a candidate).  Each is its own instantiation, so that one's
// registers do not weigh on the others.  (Dense levels are read by the slice
// variant too.)
enum RowVar { kVarStream = 0, kVarSlice = 1, kVarDrawn = 2, kVarDense = 3, kVarFree = 4 };

// Waves per SIMD of the sampled kernel: its draws are arithmetic-bound, so
// it trades occupancy for the registers of its Philox blocks (fp32 rows: 4,
// at most 128 registers; bf16 rows, twice the logits per vector: 3)
template <typename DT>
constexpr int drawn_waves_per_eu() { return sizeof(DT) == 2 ? 3 : 4; }

template <typename DT, int NT, int Var>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(Var == kVarDrawn ? drawn_waves_per_eu<DT>() : kRowBlocksPerCU)))
void row_kernel(StepArgs a) {
    constexpr bool Slice = Var == kVarSlice, Drawn = Var == kVarDrawn;
    constexpr bool DenseLevels = Var == kVarSlice || Var == kVarDense;
    if constexpr (Var == kVarFree) a.off = nullptr;  // (no trie: its paths compile away)
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
    // Request 0's counters, cleared here and rewritten by the request kernel.
    // The store is redundant, but this kernel sits at its register limit and,
    // measured on this toolchain, the allocator spills in the stream loop of
    // the hot instantiations (bf16 256-thread, fp32 64- and 256-thread)
    // without it.
    if (rowid == 0 && tid < kNumStats) a.stats[tid] = 0ull;
    // temperature (1/T = 1 when not sampling: exact); the ranking score of a
    // candidate of length len_pen: c, divided by the length penalty, plus its
    // Gumbel draw when sampling; tokens that may not be emitted this step
    const float inv_t = a.inv_t, sc = inv_t * kLog2e;
    auto rank_len = [&](float c, uint32_t vtok, float pen) {
        float k = a.penal ? __fdiv_rn(c, pen) : c;
        if (a.sampling) k = __fadd_rn(k, gumbel_noise(a.seed, b, a.t, (uint32_t)j * (uint32_t)a.V + vtok));
        return k;
    };
    auto rank = [&](float c, uint32_t vtok) { return rank_len(c, vtok, a.pen_live); };
    auto masked_ban = [&](int32_t v) { return a.banned && ((a.banned[v >> 5] >> (v & 31)) & 1u); };
    auto masked = [&](int32_t v) {
        return masked_ban(v) || (v == a.eos && a.t + 1 < a.min_len) || v < a.nlo || v >= a.nhi;
    };

    // per-row results: finite candidates, all candidates, first edge (-1
    // carried, -2 nothing), worst summary key when the summary is partial
    auto put_row = [&](int32_t c, int32_t nc, int64_t base, uint64_t worst, float lse) {
        a.cnt[rowid] = c;
        a.ncand[rowid] = nc;
        a.rbase[rowid] = base;
        a.rworst[rowid] = worst;
        a.lse_o[slot] = lse;
    };
    const float kNaN = __uint_as_float(0x7FC00000u);
    const float S = a.score[slot];
    if (S == -INFINITY) {  // empty slot: no candidate, row not read
        if (tid == 0) put_row(0, 0, -2, 0, kNaN);
        return;
    }
    if (a.fin[slot]) {  // finished: carried forward unchanged, row not read
        if (a.eos < 0) {  // no EOS in this search: a stray flag makes the slot empty
            if (tid == 0) put_row(0, 0, -2, 0, kNaN);
            return;
        }
        if (tid == 0) {
            int len = 0;  // the carried hypothesis' own length
            if (a.penal)
                for (int q = 0; q < a.T; ++q) len += a.seq[(size_t)slot * a.T + q] != -1 ? 1 : 0;
            a.pool[(size_t)rowid * a.s] = cand_key(ord_f32(rank_len(S, (uint32_t)a.eos, a.penal ? a.pen[len] : 1.0f)),
                                                  (uint32_t)j * (uint32_t)a.F + (uint32_t)a.eos);
            put_row(1, 1, -1, 0, kNaN);
        }
        return;
    }

    const DT* row = reinterpret_cast<const DT*>(a.logits) + (size_t)(b * a.K + j) * (size_t)a.stride;

    // the candidates: CSR children of the node, or every token of [nlo, nhi)
    // (all of them unless the normaliser is restricted to that range); an
    // unconstrained candidate's ordinal in its row is its token id.  A dense
    // trie level enumerates the node's row of the level's table: ordinal i is
    // token dbase + i where that entry holds a child.
    int64_t e0 = 0, ncands = a.nhi - a.nlo;
    if (a.off) {
        const int32_t n = a.node[slot];
        if (n >= 0 && n < a.nnodes) {
            if (DenseLevels && a.dspan) {
                e0 = (int64_t)n * a.dspan;
                ncands = a.dspan;
            } else {
                e0 = a.off[n];
                ncands = a.off[n + 1] - e0;
            }
        } else {
            ncands = 0;  // not a node of this level: no valid continuation
        }
    }
    // the token of trie candidate ci (-1: a dense level's code without a child)
    auto trie_tok = [&](int64_t ci) -> int32_t {
        if constexpr (DenseLevels)
            if (a.dspan) return a.child[e0 + ci] >= 0 ? a.dbase + (int32_t)ci : -1;
        return a.tok[e0 + ci];
    };
    // Common case: every candidate fits in registers (E per thread), the row
    // keeps all of them (no more than R) and its summary is small.  Their
    // token ids are fetched before the stream and their logits as soon as the
    // stream's first batch is in flight, so the gathers' latency hides behind
    // the stream and no dependent load is left once the normaliser is known.
    constexpr int E = kAdmitPerThread;
    // (a one-wave workgroup selects any summary size in registers; wider
    // ones merge per-wave summaries of at most kFastSummary keys in LDS)
    const bool fast = ncands <= (int64_t)E * NT && (NT == 64 || a.s <= kFastSummary || ncands <= a.s);
    // the thread's candidates: cv[k] = the token, -1 = none, -2 - token = a
    // token that may not be emitted (it still counts in a slice's normaliser)
    int32_t cv[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int ci = tid + k * NT;
        cv[k] = -1;
        if (fast && ci < ncands) {
            const int32_t v = a.off ? trie_tok(ci) : a.nlo + ci;
            cv[k] = v < 0 ? -1 : (masked(v) ? -2 - v : v);
        }
    }
    if (tid == 0) {
        misc[kCount] = 0;
        misc[kPoolW] = 0;
        misc[kSumW] = 0;
    }

    // Dense rows (unconstrained, every token a candidate, too many for the
    // register path) record batch maxima during the stream so that their best
    // s keys come from re-reading only the batches that can hold them.
    // (fp32 rows only: the bf16 stream has no registers to spare for it)
    // Masked tokens (banned, EOS under the minimum length) are allowed for as
    // many more logits at or above the bound.
    const bool eos_masked = a.eos >= 0 && a.t + 1 < a.min_len;
    const int n_mask = a.n_banned + (eos_masked ? 1 : 0);  // an upper bound on the distinct masked tokens
    // (a sampled row's stream bounds the ranks through Gumbel estimates: its
    // own kernel, any logit type)
    const bool dense = (Drawn || Var == kVarFree) && !fast && !a.off && a.gmax_off > 0 && a.s + n_mask <= NT &&
                       (Drawn ? a.sampling : sizeof(DT) == 4 && !a.sampling);
    float* gmax = reinterpret_cast<float*>(lds + a.gmax_off);
    // the tokens the normaliser runs over: the row, the range [nlo, nhi), or
    // (a trie row's slice) its node's children, read one by one
    const DT* nrow = row + a.nlo;
    const int nlen = a.nhi - a.nlo;
    const bool slice = Slice && a.off;

    // (1) normaliser over the row (or range, or slice)
    float Rr = kFarBelow, sp = 0.0f, tmax = -INFINITY;  // (every path below sets Rr and sp)
    int ninf = 0;
    float xv[E];
    DrawCtx dc;
    dc.seed = a.seed;
    dc.b = b;
    dc.t = a.t;
    dc.flat0 = (uint32_t)j * (uint32_t)a.V + (uint32_t)a.nlo;
    dc.q = a.penal ? __fdiv_rn(inv_t, a.pen_live) : inv_t;
    dc.xlo = INFINITY;
    dc.xhi = -INFINITY;
    if constexpr (Slice) {
        float mx = -INFINITY;
        Rr = kFarBelow;
        sp = 0.0f;
        const bool none = a.norm_mode == 3;  // log-probabilities already: no normaliser
        if (fast) {  // the thread's candidates are all of its share of the slice
            float xs[E];
#pragma unroll
            for (int k = 0; k < E; ++k) {
                xs[k] = cv[k] != -1 ? load_elem<DT>(row, cv[k] >= 0 ? cv[k] : -2 - cv[k]) : -INFINITY;
                xv[k] = xs[k];
            }
            if (!none) fold<E>(xs, mx, Rr, sp, sc);
        } else if (!none) {
            for (int64_t ci = tid; ci < ncands; ci += NT) {
                const int32_t v = trie_tok(ci);
                if (v < 0) continue;
                const float x = load_elem<DT>(row, v);
                fold<1>(&x, mx, Rr, sp, sc);
            }
        }
        (void)slice;
    } else {
        if constexpr (Drawn) {
            if (dense)
                stream_row<DT, NT, kStreamBatch, kDrawn>(nrow, nlen, tid, sc, Rr, sp, [] {}, gmax, ninf, tmax, dc);
        } else if constexpr (sizeof(DT) == 4) {
            if (dense)
                stream_row<DT, NT, kStreamBatch, kBound>(nrow, nlen, tid, sc, Rr, sp, [] {}, gmax, ninf, tmax, dc);
        }
        if (!dense) {
            stream_row<DT, NT, NT == 64 ? short_row_batch<DT>() : kStreamBatch, kPlain>(
                nrow, nlen, tid, sc, Rr, sp,
                [&] {
#pragma unroll
                    for (int k = 0; k < E; ++k) xv[k] = cv[k] >= 0 ? load_elem<DT>(row, cv[k]) : 0.0f;
                },
                gmax, ninf, tmax, dc);
        }
    }
    float lse;
    if (Slice && a.norm_mode == 3) {  // NONE: lse = 0 (the barrier orders the LDS counters' set-up)
        __syncthreads();
        lse = 0.0f;
    } else {
        double Rtop;
        lse = block_lse<NT>(Rr, sp, red, Rtop);
        if (fabs(Rtop) >= 0x1p30 && a.norm_mode != 3) {  // rare: logits beyond the fused reference's range
            if constexpr (Slice) {
                lse = exact_lse<NT>(
                    [&](auto&& f) {
                        for (int64_t ci = tid; ci < ncands; ci += NT) {
                            const int32_t v = trie_tok(ci);
                            if (v >= 0) f(load_elem<DT>(row, v));
                        }
                    },
                    inv_t, red);
            } else {
                lse = exact_lse<NT>(
                    [&](auto&& f) {
                        for (int64_t i = tid; i < nlen; i += NT) f(load_elem<DT>(nrow, i));
                    },
                    inv_t, red);
            }
        }
        // NONE without a trie: the row is streamed for its candidates (all of
        // it) and batch maxima; its sum is not used
        if (!Slice && a.norm_mode == 3) lse = 0.0f;
    }

    if (fast) {
        uint64_t kk[E];
        int nv = 0;
        const uint32_t jF = (uint32_t)j * (uint32_t)a.F;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            kk[k] = 0;
            if (cv[k] >= 0 && lse != -INFINITY) {
                const float c = __fadd_rn(S, __fsub_rn(__fmul_rn(xv[k], inv_t), lse));
                if (c != -INFINITY)
                    kk[k] = cand_key(ord_f32(rank(c, (uint32_t)cv[k])),
                                     jF + (uint32_t)(tid + k * NT) + (a.off ? 0u : (uint32_t)a.nlo));
            }
            nv += __popcll(__ballot(kk[k] != 0));
        }
        // the row's best s keys: thS, the s-th best, when it has more
        uint64_t thS = 0;
        int nkeep = nv;
        uint64_t* pseg = a.pool + (size_t)rowid * a.s;
        if constexpr (NT == 64) {
            if (nv > a.s) thS = wave_kth_key<E>(kk, a.s);
            int put = 0;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const bool keep = kk[k] && kk[k] >= thS;
                const uint64_t m = __ballot(keep);
                if (keep) pseg[put + lanes_below(m)] = kk[k];
                put += __popcll(m);
            }
        } else {
            // every wave's best s (all of its keys when it has no more) in
            // its segment of wtop, zero-padded to s; wave 0 selects the s-th
            // best of those (only when s <= kFastSummary: else the row has
            // no more than s candidates)
            uint64_t* wtop = reinterpret_cast<uint64_t*>(hist);  // NT/64 * kFastSummary keys
            if ((tid & 63) == 0 && nv) atomicAdd(&misc[kCount], nv);
            if (a.s <= kFastSummary) {
                uint64_t* seg = wtop + (tid >> 6) * kFastSummary;
                const uint64_t tw = nv > a.s ? wave_kth_key<E>(kk, a.s) : 0ull;
                int put = 0;
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const bool keep = kk[k] && kk[k] >= tw;
                    const uint64_t m = __ballot(keep);
                    if (keep) seg[put + lanes_below(m)] = kk[k];
                    put += __popcll(m);
                }
                for (int i = put + (tid & 63); i < a.s; i += 64) seg[i] = 0;
            }
            __syncthreads();
            nkeep = misc[kCount];
            if (nkeep > a.s) {
                constexpr int Q = (NT / 64 * kFastSummary + 63) / 64;
                if (tid < 64) {
                    uint64_t c2[Q];
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        const int i = tid + q * 64;  // wave i / kFastSummary, entry i % kFastSummary
                        c2[q] = (i < NT / 64 * kFastSummary && i % kFastSummary < a.s) ? wtop[i] : 0ull;
                    }
                    const uint64_t th = wave_kth_key<Q>(c2, a.s);
                    if (tid == 0) red[8] = __longlong_as_double((long long)th);
                }
                __syncthreads();
                thS = (uint64_t)__double_as_longlong(red[8]);
            }
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const bool keep = kk[k] && kk[k] >= thS;
                const int p = wave_claim(&misc[kSumW], keep);
                if (keep) pseg[p] = kk[k];
            }
        }
        if (tid == 0) put_row(nkeep, (int32_t)ncands, e0, nkeep > a.s ? thS : 0ull, lse);
        return;
    }

    if (lse == -INFINITY) ncands = 0;  // no finite logit: no finite candidate
    __syncthreads();

    const uint32_t R = (uint32_t)a.s;  // the row keeps its best s
    auto for_buf = [&](int n) {
        return [=](auto&& f) {
            for (int i = tid; i < n; i += NT) f(((uint64_t)bk[i] << 32) | (uint32_t)~bi[i]);
        };
    };
    auto cand = [&](float x) { return __fadd_rn(S, __fsub_rn(__fmul_rn(x, inv_t), lse)); };
    // the dense path ranks by c / pen_live (monotone in x), plus the draw when sampled
    auto dkey = [&](float x) { return a.penal ? __fdiv_rn(cand(x), a.pen_live) : cand(x); };
    int n = -1;        // keys in the buffer, once a path has filled it
    long long nf = 0;  // finite candidates of the row

    // (2a) dense rows: the rank is monotone in x, and at least R unmasked
    //      logits are >= T, the (R + n_mask)-th largest thread maximum, so
    //      the row's best R keys all rank at or above T and lie in batches
    //      whose maximum does.  Those batches are read again and their
    //      unmasked keys ranking >= rank(T) buffered.  Every finite logit has
    //      a finite c when c(-FLT_MAX) is finite; the finite candidates are
    //      then the logits that are neither -inf nor masked.
    //      Sampled rows bound with the estimates y = x q + g~ in place of x:
    //      for every finite candidate |rank - (D + y)| <= E(y) = 2^-20 (|y| +
    //      32 + M) + kDrawErr, with D = (S - lse) / pen and M = (|S| + |lse|) /
    //      pen (the fp32 roundings of the rank and of y, and |g| < 23).  The
    //      R-th best rank is then at least D + T - E(T), T the (R + n_mask)-th
    //      largest thread maximum of y, and no element with y + E(y) < T - E(T)
    //      reaches it.  The others are buffered as (x, v) and ranked exactly
    //      (fp64 draws) once the reread is done.
    bool dense_ok = false;
    if (dense && ncands > 0) {
        if constexpr (Drawn) {
            // every finite logit of the row must give a finite score, rank and
            // estimate: each is monotone in x, so the ends of the range decide
            auto fin = [](float v) { return v - v == 0.0f; };
            auto end_ok = [&](float x) {
                const float c = cand(x);
                const float cp = a.penal ? __fdiv_rn(c, a.pen_live) : c;
                return fin(c) && fabsf(cp) < 1.0e38f && fabsf(__fmul_rn(x, dc.q)) < 1.0e38f;
            };
            const bool bad = dc.xlo <= dc.xhi && !(end_ok(dc.xlo) && end_ok(dc.xhi));
            dense_ok = fin(lse) && !__syncthreads_or(bad);
        } else {
            dense_ok = cand(-3.40282347e38f) != -INFINITY;
        }
    }
    if (dense_ok) {
        long long gone = ninf;  // -inf logits, then masked finite ones of the range
        auto in_range = [&](int32_t v) { return v >= a.nlo && v < a.nhi; };
        for (int i = tid; i < a.n_banned; i += NT) {
            const int32_t v = a.banned_list[i];
            gone += in_range(v) && load_elem<DT>(row, v) != -INFINITY ? 1 : 0;
        }
        if (tid == 0 && eos_masked && in_range(a.eos) && !masked_ban(a.eos) && load_elem<DT>(row, a.eos) != -INFINITY)
            ++gone;
        nf = (long long)nlen - block_sum_ll<NT>(gone, reinterpret_cast<long long*>(red));
        float T = -INFINITY;
        if (nf > (long long)R) {  // T by wave 0 over the NT thread maxima
            hist[tid] = ord_f32(tmax);
            __syncthreads();
            if (tid < 64) {
                uint32_t m[NT / 64];
#pragma unroll
                for (int q = 0; q < NT / 64; ++q) m[q] = hist[tid + 64 * q];
                const uint32_t P = wave_kth_u32<NT / 64>(m, (int)R + n_mask);
                if (tid == 0) misc[0] = (int)P;
            }
            __syncthreads();
            const uint32_t P = (uint32_t)misc[0];
            T = P <= ord_f32(-INFINITY) ? -INFINITY : unord_f32(P);
        }
        // unsampled: the keys of rank >= cT; sampled: the estimates that can reach thr
        const float cT = T == -INFINITY ? -INFINITY : dkey(T);
        const double M = ((double)fabsf(S) + (double)fabsf(lse)) / (a.penal ? (double)a.pen_live : 1.0);
        auto ebound = [&](float y) { return 0x1p-20 * (fabs((double)y) + 32.0 + M) + (double)kDrawErr; };
        const double thr = T == -INFINITY ? -INFINITY : (double)T - ebound(T);
        auto reach = [&](float y) { return y != -INFINITY && (double)y + ebound(y) >= thr; };
        if (tid == 0) misc[kCount] = 0;
        __syncthreads();
        constexpr int VEC = 16 / (int)sizeof(DT);
        constexpr int64_t per = (int64_t)kStreamBatch * NT;
        const int head = row_head(nrow, nlen);
        const int64_t nvec = (int64_t)(nlen - head) / VEC;
        const int64_t nb = (nvec + per - 1) / per;
        const u32x4* vp = reinterpret_cast<const u32x4*>(nrow + head);
        // element x of token v (estimate draw gq when sampled)
        auto offer = [&](float x, int32_t v, float gq) {
            bool keep;
            if constexpr (Drawn) {
                keep = x != -INFINITY && !masked(v) && reach(__fadd_rn(__fmul_rn(x, dc.q), gq));
            } else {
                keep = cand(x) != -INFINITY && dkey(x) >= cT && !masked(v);
            }
            const int p = wave_claim(&misc[kCount], keep);
            if (keep && p < a.cap) {
                bk[p] = Drawn ? __float_as_uint(x) : ord_f32(dkey(x));
                bi[p] = (uint32_t)v;
            }
        };
        // The batches that can hold such keys (nb <= 32: at most one bit
        // each), listed over the whole workgroup as k*NT + thread in place
        // of the batch maxima, then read back by every thread at once (one
        // round of independent loads instead of one per batch).
        uint32_t qmask = 0;
        for (int k = 0; k < (int)nb; ++k) {
            const float g = gmax[k * NT + tid];
            const bool in = Drawn ? reach(g) : g != -INFINITY && dkey(g) >= cT;
            if (in) qmask |= 1u << k;
        }
        const int nq = __popc(qmask);
        const int incl = (int)wave_inclusive_scan((uint32_t)nq);
        int* wq = misc + 8;  // one per wave
        if ((tid & 63) == 63) wq[tid >> 6] = incl;
        __syncthreads();  // also: every batch maximum has been read
        int nlist = 0, o = incl - nq;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            o += w < (tid >> 6) ? wq[w] : 0;
            nlist += wq[w];
        }
        int* list = reinterpret_cast<int*>(gmax);
        for (uint32_t m = qmask; m; m &= m - 1) list[o++] = (__ffs(m) - 1) * NT + tid;
        __syncthreads();
        constexpr int kReread = 4;  // vectors in flight per thread
        const int nv = nlist * kStreamBatch;
        for (int i0 = tid; i0 < nv; i0 += kReread * NT) {
            u32x4 w[kReread];
            int64_t vi[kReread];
#pragma unroll
            for (int r = 0; r < kReread; ++r) {
                const int i = i0 + r * NT;
                vi[r] = -1;
                if (i < nv) {
                    const int e = list[i / kStreamBatch];
                    const int64_t v = (int64_t)(e / NT) * per + (int64_t)(i % kStreamBatch) * NT + (e % NT);
                    if (v < nvec) {
                        vi[r] = v;
                        w[r] = vp[v];
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < kReread; ++r) {
                float x[VEC], g[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q) g[q] = 0.0f;
                if (vi[r] >= 0) {
                    unpack<DT>(w[r], x);
                    if constexpr (Drawn)
                        gumbel_fast_run<VEC>(a.seed, b, a.t, dc.flat0 + (uint32_t)head + (uint32_t)(vi[r] * VEC), g);
                }
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    offer(vi[r] >= 0 ? x[q] : -INFINITY, (int32_t)(a.nlo + head + (vi[r] >= 0 ? vi[r] : 0) * VEC + q),
                          g[q]);
            }
        }
        auto fast_one = [&](int64_t i) {
            return Drawn ? gumbel_fast_one(a.seed, b, a.t, dc.flat0 + (uint32_t)i) : 0.0f;
        };
        if (tid < head) offer(load_elem<DT>(nrow, tid), a.nlo + tid, fast_one(tid));
        const int64_t tail0 = head + nvec * VEC;
        if (tail0 + tid < nlen) offer(load_elem<DT>(nrow, tail0 + tid), (int32_t)(a.nlo + tail0 + tid), fast_one(tail0 + tid));
        __syncthreads();
        n = misc[kCount];
        if (n > a.cap) {  // too many ties with the bound: the general path below
            n = -1;
            __syncthreads();
            if (tid == 0) misc[kCount] = 0;
            __syncthreads();
        } else if constexpr (Drawn) {  // the buffered elements' exact ranks
            for (int i = tid; i < n; i += NT) bk[i] = ord_f32(rank(cand(__uint_as_float(bk[i])), bi[i]));
            __syncthreads();
        }
    }

    // (2b) general case: admission into the LDS buffer with compaction
    uint64_t theta = 0;  // admission bound: keys below it cannot make the row's best s
    long long nfin = 0;
    if (n < 0)
    for (int64_t base = 0; base < ncands; base += (int64_t)E * NT) {
        // each thread takes E consecutive candidates: the Gumbel draws of an
        // unconstrained sampled row's run share Philox blocks (gumbel_run4)
        static_assert(E == 4, "gumbel_run4 draws four consecutive candidates");
        const int64_t c0 = base + (int64_t)tid * E;
        const bool run = Drawn && a.sampling && !a.off;
        f32x4 gq = {0.0f, 0.0f, 0.0f, 0.0f};
        if (run) gq = gumbel_run4(a.seed, b, a.t, (uint32_t)j * (uint32_t)a.V + (uint32_t)(a.nlo + c0));
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int64_t ci = c0 + k;
            bool adm = false;
            uint32_t o = 0;
            uint32_t ordn = 0;
            if (ci < ncands) {
                const int32_t v = a.off ? trie_tok(ci) : (int32_t)(a.nlo + ci);
                ordn = a.off ? (uint32_t)ci : (uint32_t)v;
                const float x = v < 0 || masked(v) ? -INFINITY : load_elem<DT>(row, v);
                const float c = __fadd_rn(S, __fsub_rn(__fmul_rn(x, inv_t), lse));
                if (c != -INFINITY) {
                    ++nfin;
                    o = ord_f32(run ? __fadd_rn(a.penal ? __fdiv_rn(c, a.pen_live) : c, gq[k])
                                    : rank(c, (uint32_t)v));
                    adm = (((uint64_t)o << 32) | (uint32_t)~ordn) >= theta;
                }
            }
            const int p = wave_claim(&misc[kCount], adm);
            if (adm) {
                bk[p] = o;
                bi[p] = ordn;
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
                const bool keep = (((uint64_t)bk[i] << 32) | (uint32_t)~bi[i]) >= theta;
                const int p = wave_claim(&misc[kStage], keep);
                if (keep) {
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

    if (n < 0) {
        __syncthreads();
        n = misc[kCount];
        nf = block_sum_ll<NT>(nfin, reinterpret_cast<long long*>(red));
    }

    // (3) the row's best s keys, the worst of them, and its number of
    //     finite candidates (the buffer holds all of them when they are at
    //     most R: no compaction has happened)
    uint64_t thS = 0;
    if (nf > (long long)R) {
        // wave 0 selects in registers (fp32 rows: the bf16 kernel has no
        // registers to spare for it)
        if (sizeof(DT) == 4 && n <= 256) {
            __syncthreads();
            if (tid < 64) {
                uint64_t kq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = tid + 64 * q;
                    kq[q] = i < n ? (((uint64_t)bk[i] << 32) | (uint32_t)~bi[i]) : 0ull;
                }
                const uint64_t th = wave_kth_key<4>(kq, (int)R);
                if (tid == 0) red[8] = __longlong_as_double((long long)th);
            }
            __syncthreads();
            thS = (uint64_t)__double_as_longlong(red[8]);
        } else {
            thS = radix_threshold<NT>(for_buf(n), R, hist, misc);
        }
    }
    unsigned long long* wmin = reinterpret_cast<unsigned long long*>(red + 12);
    if (tid == 0) {
        misc[kSumW] = 0;
        *wmin = ~0ull;
    }
    __syncthreads();
    uint64_t* pseg = a.pool + (size_t)rowid * a.s;
    const uint32_t jF = (uint32_t)j * (uint32_t)a.F;
    uint64_t lmin = ~0ull;
    for (int i = tid; i < n; i += NT) {
        const bool keep = (((uint64_t)bk[i] << 32) | (uint32_t)~bi[i]) >= thS;
        const int p = wave_claim(&misc[kSumW], keep);
        if (keep) {
            const uint64_t key = cand_key(bk[i], jF + bi[i]);
            pseg[p] = key;
            lmin = key < lmin ? key : lmin;
        }
    }
    lmin = wave_min_u64(lmin);
    if ((tid & 63) == 0 && lmin != ~0ull) atomicMin(wmin, (unsigned long long)lmin);
    __syncthreads();
    if (tid == 0) put_row((int32_t)nf, (int32_t)ncands, e0, nf > (long long)R ? (uint64_t)*wmin : 0ull, lse);
}

}  // namespace

size_t row_lds_bytes(int cap, int stg) {
    return 16 * sizeof(double) + 16 * sizeof(int) + 256 * sizeof(uint32_t) +
           (size_t)(2 * cap + 2 * stg) * sizeof(uint32_t);
}

// Dynamic LDS of a launch: what the buffers need, and for the long-row
// (256-thread) kernel at least a sixth of the CU's LDS less 256 bytes.  LDS
// is allocated in 1 KB granules, so five such workgroups share a CU (the
// registers would admit six); a floor 1 KB lower that lets six in measured
// the same on the 151,936- and 50,257-token rows.
size_t row_lds_launch_bytes(int cap, int stg, int V, int max_lds) {
    size_t b = row_lds_bytes(cap, stg);
    if (row_threads(V) == 256) {
        const size_t floor6 = (size_t)max_lds / kRowBlocksPerCU - 256;
        if (b < floor6) b = floor6;
    }
    return b;
}

hipError_t launch_rows(const StepArgs& args, int bf16, hipStream_t st) {
    const int NT = row_threads(args.V);
    const size_t lds = row_lds_launch_bytes(args.cap, args.stg, args.V, args.max_lds);
    // batch maxima of dense rows after the candidate buffer, when they fit
    StepArgs a = args;
    a.gmax_off = 0;
    if (!a.off) {
        const size_t off = row_lds_bytes(a.cap, a.stg);
        const int64_t vec = bf16 ? 8 : 4;
        const int64_t nb = a.V / vec / ((int64_t)kStreamBatch * NT) + 1;
        if (nb <= 32 && off + (size_t)nb * NT * sizeof(float) <= lds) a.gmax_off = (int32_t)off;
    }
    const dim3 grid((unsigned)(a.B * a.L));
    // rows that are not streamed: a trie row's slice, or its candidates alone
    // when there is no normaliser (unconstrained NONE rows are streamed:
    // every token is a candidate)
    const bool slice = (a.norm_mode == 2 || a.norm_mode == 3) && a.off;
    const int var = slice                     ? kVarSlice
                    : a.sampling && !a.off    ? kVarDrawn
                    : !a.off                  ? kVarFree
                    : a.dspan                 ? kVarDense
                                              : kVarStream;
    auto go = [&](auto dt, auto v) {
        using DT = decltype(dt);
        constexpr int V = decltype(v)::value;
        if (NT == 64) row_kernel<DT, 64, V><<<grid, 64, lds, st>>>(a);
        else row_kernel<DT, 256, V><<<grid, 256, lds, st>>>(a);
    };
    using VS = std::integral_constant<int, kVarStream>;
    using VL = std::integral_constant<int, kVarSlice>;
    using VD = std::integral_constant<int, kVarDrawn>;
    using VT = std::integral_constant<int, kVarDense>;
    using VF = std::integral_constant<int, kVarFree>;
    if (bf16) {
        if (var == kVarSlice) go(uint16_t{}, VL{});
        else if (var == kVarDrawn) go(uint16_t{}, VD{});
        else if (var == kVarDense) go(uint16_t{}, VT{});
        else if (var == kVarFree) go(uint16_t{}, VF{});
        else go(uint16_t{}, VS{});
    } else {
        if (var == kVarSlice) go(float{}, VL{});
        else if (var == kVarDrawn) go(float{}, VD{});
        else if (var == kVarDense) go(float{}, VT{});
        else if (var == kVarFree) go(float{}, VF{});
        else go(float{}, VS{});
    }
    return hipGetLastError();
}

hipError_t set_row_lds_limit(int bytes) {
    hipError_t e = hipSuccess, r;
    const void* fs[20] = {
        (const void*)row_kernel<float, 64, kVarStream>,    (const void*)row_kernel<float, 256, kVarStream>,
        (const void*)row_kernel<uint16_t, 64, kVarStream>, (const void*)row_kernel<uint16_t, 256, kVarStream>,
        (const void*)row_kernel<float, 64, kVarSlice>,     (const void*)row_kernel<float, 256, kVarSlice>,
        (const void*)row_kernel<uint16_t, 64, kVarSlice>,  (const void*)row_kernel<uint16_t, 256, kVarSlice>,
        (const void*)row_kernel<float, 64, kVarDrawn>,     (const void*)row_kernel<float, 256, kVarDrawn>,
        (const void*)row_kernel<uint16_t, 64, kVarDrawn>,  (const void*)row_kernel<uint16_t, 256, kVarDrawn>,
        (const void*)row_kernel<float, 64, kVarDense>,     (const void*)row_kernel<float, 256, kVarDense>,
        (const void*)row_kernel<uint16_t, 64, kVarDense>,  (const void*)row_kernel<uint16_t, 256, kVarDense>,
        (const void*)row_kernel<float, 64, kVarFree>,      (const void*)row_kernel<float, 256, kVarFree>,
        (const void*)row_kernel<uint16_t, 64, kVarFree>,   (const void*)row_kernel<uint16_t, 256, kVarFree>};
    for (const void* f : fs) {
        r = allow_dynamic_lds(f, bytes);
        if (r != hipSuccess) e = r;
    }
    return e;
}

}  // namespace gr
