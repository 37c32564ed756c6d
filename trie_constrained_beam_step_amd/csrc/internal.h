// internal.h -- shared between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gr {

constexpr int kMaxBeam = 4096;

// Everything one beam step needs, passed by value to both kernels.
struct StepArgs {
    int32_t B, K, V, T;     // batch, beam width, vocabulary, max steps
    int32_t t;              // 0-based index of this step
    int32_t L;              // live bound: only slots j < L can be live
    int32_t s;              // per-row summary size: each live row writes its best s keys
    int32_t F;              // flat-index stride: V, or the level's largest fan-out with a trie
    int32_t eos;            // -1 = none
    int32_t cap, stg;       // row-kernel LDS candidate buffer / staging entries
    int32_t sb;             // request-kernel LDS survivor buffer entries
    int32_t gs;             // request-kernel LDS summary grid slots (>= L*s)
    int32_t s_log2;         // s = 2^s_log2
    int32_t max_lds;        // device LDS bytes per workgroup
    int32_t gmax_off;       // row kernel: LDS byte offset of the dense rows' batch maxima (0 = none)
    // sampling (Gumbel top-K at temperature T > 0); inv_t = fl32(1/T), 1 when off
    float inv_t;
    int32_t sampling;
    uint64_t seed;
    // length penalty (live candidates have length t+1: pen_live = pen[t+1];
    // a carried beam uses pen[its length]), minimum length, banned tokens
    int32_t penal;               // alpha != 0
    float pen_live;
    const float* pen;            // [T + 1]
    int32_t min_len;
    const uint32_t* banned;      // [ceil(V/32)] bitmap, nullptr when none
    const int32_t* banned_list;  // [n_banned] the same ids, distinct
    int32_t n_banned;
    int32_t rank_is_c;           // no sampling and no penalty: a key's score half is c
    // normalisation: 0 = full row, 1 = tokens [nlo, nhi) only (others never
    // candidates), 2 = a trie row's children only (full row without a trie),
    // 3 = none (the values are log-probabilities: lse = 0, rows not streamed)
    int32_t norm_mode;
    int32_t nlo, nhi;
    int64_t stride;         // logits row stride in elements
    // trie level t; off == nullptr selects unconstrained search.  A dense
    // level (dspan > 0) is read through child = its [nnodes x dspan] table:
    // code i of node n is token dbase + i, with child node child[n*dspan + i]
    // (-1: no such child); tok is then unused.
    const int64_t* off;
    const int32_t* tok;
    const int32_t* child;
    int64_t nnodes;         // nodes at level t
    int32_t dspan, dbase;
    const void* logits;
    // state before the step ([B*K], [B*K*T])
    const float* score;
    const int32_t* node;
    const uint8_t* fin;
    const int32_t* seq;
    // state after the step
    float* score_o;
    int32_t* node_o;
    uint8_t* fin_o;
    int32_t* seq_o;
    int32_t* parent_o;      // history row t: [B*K]
    int32_t* token_o;
    float* lse_o;           // [B*K], indexed by the slot whose row was read
    // workspace
    uint64_t* pool;         // [B*L*s] each row's best s candidate keys (its summary)
    int32_t* cnt;           // [B*L] finite candidates per row
    int32_t* ncand;         // [B*L] candidates per row, finite or not (the row's fan-out)
    int64_t* rbase;         // [B*L] first edge of the row's node (0 unconstrained);
                            //       -1 finished (carried), -2 no candidate and not read
    uint64_t* rworst;       // [B*L] the worst key of the row's summary when cnt > s
    unsigned long long* stats;  // [B*6] per request: rows read, candidates, survivors,
                                //      slow-path requests, rows recomputed by the request kernel,
                                //      1 when the step ran fused
    // fused short-row step (fw > 0; 0: the row and request kernels).  The L
    // rows of a request are split over fw workgroups of rpw rows, each
    // keeping its candidates in an LDS buffer of fcap keys.  fw = 1: that
    // workgroup finishes the request (one launch).  fw > 1: each writes its
    // best K at or above the request's running bound, and the merge kernel
    // selects among them.
    int32_t fw, rpw, fcap;
    uint64_t* part;             // [B*fw*K] each workgroup's kept keys
    int32_t* part_n;            // [B*fw]   how many
    long long* part_stats;      // [B*fw*2] rows read, finite candidates
    unsigned long long* req_theta;  // [B] running lower bound on the K-th best key (0 between steps)
};

// Up to kSearchSteps one-workgroup fused steps (every step fw = 1, the same
// batch) as one launch; the arguments travel in the kernel's argument block.
constexpr int kSearchSteps = 8;
struct SearchArgs {
    StepArgs step[kSearchSteps];
    int32_t n;
};
static_assert(sizeof(SearchArgs) <= 4096, "a kernel argument block holds at most 4 KiB");
hipError_t launch_fused_search(const SearchArgs& sa, int dtype_bf16, hipStream_t st);

hipError_t launch_rows(const StepArgs& a, int dtype_bf16, hipStream_t st);
hipError_t launch_select(const StepArgs& a, int dtype_bf16, hipStream_t st);
hipError_t launch_fused(const StepArgs& a, int dtype_bf16, hipStream_t st);
hipError_t launch_merge(const StepArgs& a, hipStream_t st);
// the step's launches: the fused kernel when a.fw > 0, else rows then request
hipError_t launch_step(const StepArgs& a, int dtype_bf16, hipStream_t st);
hipError_t launch_reset(float* score, int32_t* node, uint8_t* fin, int32_t* seq,
                        int32_t* parents, int32_t* tokens, float* lse, int B, int K, int T,
                        int trie_root, hipStream_t st);
hipError_t launch_live_bound(const float* score, int B, int K, int* out, hipStream_t st);
hipError_t launch_probe_read(const void* src, size_t n16, uint32_t* sink, hipStream_t st);
hipError_t launch_probe_copy(void* dst, const void* src, size_t n16, hipStream_t st);
hipError_t launch_trie_densify(const int64_t* off, const int32_t* tok, const int32_t* child, int64_t nnodes,
                               int32_t tbase, int32_t span, int32_t* dense, hipStream_t st);
hipError_t launch_probe_draw_error(uint32_t r0, uint64_t count, double* out, hipStream_t st);
float draw_error_bound();

// Row-kernel workgroup size for a vocabulary (one wave for short rows).
inline int row_threads(int V) { return V <= 4096 ? 64 : 256; }
// Candidates each thread handles between two admission checks.
constexpr int kAdmitPerThread = 4;
// 16-byte vectors each thread keeps in flight per stream batch.
constexpr int kStreamBatch = 4;
constexpr int kSelectThreads = 1024;
constexpr int kSelectMaxGrid = 32768;  // request-kernel summary grid slots, at most
constexpr int kSelectMaxSurvivors = 16384;  // request-kernel survivor buffer keys, at most

constexpr int kRowBlocksPerCU = 6;  // the long-row kernel's register budget (waves per SIMD) and LDS floor divisor
// fused short-row step: workgroup size, LDS candidate buffer, workgroups
// per request at most, and the longest row (logits) it takes: fewer than two
// stream batches of a wave (4 KB bf16, 8 KB fp32), so that each lane loads
// its share of a row at once
constexpr int kFusedThreads = 256;
constexpr int kFusedCap = 4096;
constexpr int kFusedMaxW = 64;
constexpr int kFusedMaxRow = 2047;
constexpr int kFusedRowsWaves = 5;  // waves per SIMD of the split step's row kernel
// kept-key slots of a split step's workgroup, in units of K (its K best and
// the K-th's bucket mates)
constexpr int kPartPerK = 2;
constexpr int kFusedMaxRows = 16;  // live rows per request the automatic choice fuses
size_t fused_lds_bytes(int fcap, int fw);
constexpr int kNumStats = 6;
size_t row_lds_bytes(int cap, int stg);
size_t row_lds_launch_bytes(int cap, int stg, int V, int max_lds);
size_t select_lds_bytes(int gs, int sb, int K, int L);
// survivor-buffer entries that fit in lds_bytes with a grid of gs slots
int select_buffer_fit(size_t lds_bytes, int gs, int K, int L);
// Let launches of kernel f use as much dynamic LDS as the device's `bytes`
// leave beside f's static LDS (the runtime refuses a larger limit).
inline hipError_t allow_dynamic_lds(const void* f, int bytes) {
    hipFuncAttributes at;
    hipError_t e = hipFuncGetAttributes(&at, f);
    if (e != hipSuccess) return e;
    const int v = bytes - (int)at.sharedSizeBytes;
    return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, v > 0 ? v : 0);
}
// Every row / request kernel: allow_dynamic_lds with the device's LDS.
hipError_t set_row_lds_limit(int bytes);
hipError_t set_select_lds_limit(int bytes);
hipError_t set_fused_lds_limit(int bytes);

}  // namespace gr
