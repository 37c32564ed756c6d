// api.hip -- the C ABI declared in include/gr.h.
//
// Host-side validation, device memory ownership and the per-step launch
// sequence.  Everything a search needs on the device is allocated by
// gr_trie_build and gr_beam_init; gr_beam_step only computes sizes and
// enqueues the two step kernels on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "gr.h"

#include <cmath>
#include "internal.h"
#include "backward.h"

using gr::StepArgs;

namespace {

thread_local std::string g_err;

gr_status fail(gr_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

gr_status hip_fail(hipError_t e, const char* what) {
    return fail(GR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                       \
    do {                                          \
        hipError_t e_ = (expr);                   \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

template <typename T>
hipError_t dalloc(T** p, size_t count) {
    *p = nullptr;
    if (count == 0) count = 1;
    return hipMalloc((void**)p, count * sizeof(T));
}

int device_lds_limit() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 65536;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
        return 65536;
    return v;
}

constexpr int kTimingRing = 256;

}  // namespace

struct gr_trie {
    int32_t depth = 0, vocab = 0;
    std::vector<int64_t> num_nodes;  // [depth+1]
    std::vector<int32_t> max_fan;    // [depth]
    std::vector<int32_t> tmin, tmax; // [depth] the level's smallest and largest child token
    std::vector<int64_t*> off;
    std::vector<int32_t*> tok, child;
    std::vector<int32_t*> dense;     // [depth] the level's dense child table, or nullptr
};

struct gr_beam {
    gr_beam_config cfg{};
    const gr_trie* trie = nullptr;
    int32_t t = 0;       // next step index
    int64_t live = 1;    // bound on live slots per request
    int64_t live_prev = 1;     // the bound before the last step (for rewind)
    bool can_rewind = false;   // the last call was a step: its input state is intact
    int cur = 0;
    float* score[2] = {nullptr, nullptr};
    int32_t* node[2] = {nullptr, nullptr};
    uint8_t* fin[2] = {nullptr, nullptr};
    int32_t* seq[2] = {nullptr, nullptr};
    int32_t* parents = nullptr;
    int32_t* tokens = nullptr;
    float* lse = nullptr;
    uint64_t* pool = nullptr;
    int32_t* cnt = nullptr;
    int32_t* ncand = nullptr;
    int64_t* rbase = nullptr;
    uint64_t* rworst = nullptr;
    unsigned long long* stats = nullptr;  // [B*5] per request
    int* live_dev = nullptr;  // set_state's live bound
    // the fused short-row step's workspace (part_keys == 0: never fused)
    uint64_t* part = nullptr;
    int32_t* part_n = nullptr;
    long long* part_stats = nullptr;
    unsigned long long* req_theta = nullptr;
    size_t part_keys = 0, part_slots = 0;
    bool fused = true;  // take the fused step where it applies
    bool fused_split = false;  // also split a request's rows over workgroups
    size_t select_lds = 0;    // the request kernel's LDS per launch
    // whole-search graphs: the captured step launches of gr_beam_search,
    // keyed by their complete argument blocks (least recently used evicted)
    struct Graph {
        std::vector<gr::StepArgs> args;
        hipGraphExec_t exec = nullptr;
        uint64_t used = 0;
    };
    std::vector<Graph> graphs;
    uint64_t graph_clock = 0;
    hipStream_t cap_stream = nullptr;  // private capture stream (default priority)
    size_t pool_cap = 0;
    float temperature = 0.0f;  // > 0: Gumbel top-K sampling
    uint64_t seed = 0;
    // length penalty, minimum length, banned tokens
    float alpha = 0.0f;
    int32_t min_len = 0;
    bool has_banned = false;
    uint32_t* banned = nullptr;      // device bitmap [ceil(V/32)]
    int32_t* banned_list = nullptr;  // device [vocab]: the first n_banned hold the distinct ids
    int32_t n_banned = 0;
    float* pen = nullptr;            // device [T + 1]
    std::vector<float> pen_host;     // the same table on the host
    // normalisation variant: 0 full row, 1 token range [nlo, nhi), 2 slice
    int32_t norm_mode = 0, nlo = 0, nhi = 0;
    int sb = 0;   // request-kernel survivor buffer entries
    int gs = 0;   // request-kernel summary grid slots
    int max_lds = 65536;
    hipStream_t last_stream = nullptr;
    // timing
    bool timing = false;
    hipEvent_t ev[kTimingRing][3];
    bool ev_one[kTimingRing] = {};  // the slot timed a step of one kernel
    bool ev_made = false;
    int ev_head = 0, ev_pending = 0;
    double row_ms = 0.0, sel_ms = 0.0;
    int64_t timed_steps = 0;
};

// --------------------------------------------------------------- helpers

// What a step's launches need besides its buffers: the configuration, the
// trie, the request kernel's LDS plan and the search options.  A handle
// keeps one; the no-allocation step builds one per call.
struct StepPlan {
    gr_beam_config cfg{};
    const gr_trie* trie = nullptr;
    int gs = 0;              // request-kernel summary grid slots, at most
    size_t select_lds = 0;   // the request kernel's LDS per launch
    int max_lds = 65536;
    float temperature = 0.0f;
    uint64_t seed = 0;
    float alpha = 0.0f;
    const float* pen_host = nullptr;  // [T + 1] length penalties (alpha != 0)
    int32_t min_len = 0;
    bool has_banned = false;
    int32_t norm_mode = 0, nlo = 0, nhi = 0;
    bool fused = true;  // the fused short-row step where it applies
    bool fused_split = false;  // also for requests split over several workgroups
};

// The buffers a step reads and writes (device addresses).
struct StepBuffers {
    const float* score = nullptr;
    const int32_t* node = nullptr;
    const uint8_t* fin = nullptr;
    const int32_t* seq = nullptr;
    float* score_o = nullptr;
    int32_t* node_o = nullptr;
    uint8_t* fin_o = nullptr;
    int32_t* seq_o = nullptr;
    int32_t* parent_o = nullptr;  // this step's history row [B*K]
    int32_t* token_o = nullptr;
    float* lse = nullptr;
    uint64_t* pool = nullptr;
    int32_t* cnt = nullptr;
    int32_t* ncand = nullptr;
    int64_t* rbase = nullptr;
    uint64_t* rworst = nullptr;
    unsigned long long* stats = nullptr;
    const float* pen = nullptr;            // [T + 1], read when alpha != 0
    const uint32_t* banned = nullptr;      // bitmap, or nullptr
    const int32_t* banned_list = nullptr;
    int32_t n_banned = 0;
    // the fused step's: kept keys (part_keys of them), counts, bounds
    uint64_t* part = nullptr;
    int32_t* part_n = nullptr;          // part_slots of them
    long long* part_stats = nullptr;    // 2 * part_slots
    unsigned long long* req_theta = nullptr;
    size_t part_keys = 0, part_slots = 0;
};

static int64_t max_candidates(const StepPlan& p, int t) {
    return p.trie ? (int64_t)p.trie->max_fan[t] : (int64_t)p.cfg.vocab;
}

struct StepShape {
    int s, s_log2, cap, stg;
};

static int floor_log2(int64_t v) {
    int l = 0;
    while ((int64_t)2 << l <= v) ++l;
    return l;
}

// Per-row summary size s, a power of two: unconstrained rows keep about
// min(K, V) keys, so the request kernel rarely recomputes a row; with a trie
// about 16K/L keys per row (the whole row when L is small), so the summaries
// hold many times K candidates and only a few rows per request are
// recomputed.  L*s must fit the request kernel's LDS grid.
static StepShape step_shape(const StepPlan& p, int t, int64_t L) {
    const int K = p.cfg.beam_width;
    const int64_t mc = std::max<int64_t>(1, max_candidates(p, t));
    StepShape sh;
    int64_t s = std::min<int64_t>(K, mc);
    if (p.trie) s = std::min<int64_t>(s, std::max<int64_t>(1, (16 * (int64_t)K + L - 1) / L));
    s = std::min<int64_t>(s, std::max<int64_t>(1, p.gs / L));
    sh.s_log2 = floor_log2(std::max<int64_t>(1, s));
    sh.s = 1 << sh.s_log2;
    // LDS candidate buffer of the row kernel's general path: all candidates
    // when they fit with two admission chunks to spare, else s plus two
    // chunks (compaction back to s whenever the next chunk might not fit)
    // (one chunk suffices: the buffer is compacted back to s before a chunk
    // could overflow it; unconstrained rows take one so that their dense
    // path's batch maxima fit beside the buffer)
    const int ent = (p.trie ? 2 : 1) * gr::kAdmitPerThread * gr::row_threads(p.cfg.vocab);
    // a dense level's row enumerates the level's whole token span (codes
    // without a child are skipped as they come), more than its children:
    // the buffer without compaction must hold what is enumerated, or the
    // admission would compact with no staging room
    const int64_t nc = p.trie && p.trie->dense[t] ? std::max<int64_t>(mc, p.trie->tmax[t] - p.trie->tmin[t] + 1) : mc;
    if (nc <= (int64_t)sh.s + ent) {
        sh.cap = (int)nc;
        sh.stg = 0;
    } else {
        sh.cap = sh.s + ent;
        sh.stg = sh.s;
    }
    return sh;
}

// The request kernel's LDS for beam width K: a survivor buffer of 4K keys
// and the rest for the summary grid; at the largest widths the buffer
// shrinks so that the grid keeps one slot per row (requests whose survivors
// overflow the buffer take the exact slow path).  False if K leaves no room.
static bool select_plan(int K, int max_lds, int* sb_out, int* gs_out, size_t* lds_out) {
    const int64_t avail = (int64_t)max_lds - (int64_t)gr::select_lds_bytes(0, 0, K, K);
    int64_t sb = std::max<int64_t>(4 * (int64_t)K, 256);
    int64_t gs = (avail - 8 * sb) / 4;
    if (gs < (int64_t)K) {
        sb = (avail - 4 * (int64_t)K) / 8;
        gs = (avail - 8 * sb) / 4;
    }
    gs = std::min<int64_t>(gs, gr::kSelectMaxGrid);
    sb = std::min<int64_t>(sb, gr::kSelectMaxSurvivors);
    if (sb < 1 || gs < (int64_t)K) return false;
    *sb_out = (int)sb;
    *gs_out = (int)gs;
    *lds_out = gr::select_lds_bytes((int)gs, (int)sb, K, K);
    return true;
}

// The row kernel's largest LDS need over every step and live bound of a
// search with this plan.
static size_t row_lds_need(const StepPlan& p) {
    size_t m = 0;
    const int steps = p.trie ? std::min<int>(p.cfg.max_steps, p.trie->depth) : p.cfg.max_steps;
    for (int t = 0; t < steps; ++t) {
        for (int64_t L : {(int64_t)1, (int64_t)p.cfg.beam_width}) {
            const StepShape sh = step_shape(p, t, L);
            m = std::max(m, gr::row_lds_launch_bytes(sh.cap, sh.stg, p.cfg.vocab, p.max_lds));
        }
    }
    return m;
}

// The fused short-row step's split of step t with live bound L into fw
// workgroups of rpw rows per request, or false where the step takes the row
// and request kernels.  It needs a CSR trie level (not dense), unperturbed
// ranking and the full-row normaliser, K <= kFusedCap / 2, rows of at most
// kFusedMaxRow logits, and each workgroup's candidates (rpw x the level's
// largest fan-out) within its LDS buffer.  A request of at most
// kFusedMaxRows live rows whose candidates fit one buffer takes one
// workgroup (the whole step one launch); a larger one is split over about
// 256 x kFusedRowsWaves workgroups in all (as many as the CUs hold at the
// rows kernel's occupancy), at least four rows each (one per
// wave), and the merge kernel selects among their kept keys.  Measured on
// the benchmark's short-row steps, both beat the row and request kernels
// (deep trie 100 -> 85 us, SID-only 56 -> 50 us, K = 2,000 65 -> 49 us per
// step).  fused_split forces the split even for the smallest requests.
static bool fused_shape(const StepPlan& p, int t, int64_t L, int* fw_out, int* rpw_out) {
    if (!p.fused || !p.trie || p.trie->dense[t]) return false;
    if (p.temperature > 0.0f || p.alpha != 0.0f || p.has_banned || p.norm_mode != 0) return false;
    const int64_t K = p.cfg.beam_width, B = p.cfg.batch;
    if (K > gr::kFusedCap / 2) return false;
    if (p.cfg.vocab > gr::kFusedMaxRow) return false;
    const int64_t rmax = gr::kFusedCap / std::max<int64_t>(1, p.trie->max_fan[t]);
    if (rmax < 1) return false;
    if (!p.fused_split && L <= gr::kFusedMaxRows && L <= rmax) {
        *fw_out = 1;
        *rpw_out = (int)L;
        return true;
    }
    const int64_t target = 256 * gr::kFusedRowsWaves;  // workgroups: one per SIMD slot of the row kernel
    int64_t w = std::max<int64_t>(1, (target + B - 1) / B);
    w = std::min<int64_t>(w, std::max<int64_t>(1, (L + 3) / 4));
    w = std::min<int64_t>(w, gr::kFusedMaxW);
    const int64_t r = std::min<int64_t>((L + w - 1) / w, rmax);
    w = (L + r - 1) / r;
    if (w > gr::kFusedMaxW) return false;
    *fw_out = (int)w;
    *rpw_out = (int)r;
    return true;
}

// The fused step's largest workspace over every step and live bound of a
// search with this plan: kept keys (B x fw x K) and per-workgroup slots.
static void fused_need(const StepPlan& p, size_t* keys, size_t* slots) {
    *keys = 0;
    *slots = 0;
    const int steps = p.trie ? std::min<int>(p.cfg.max_steps, p.trie->depth) : 0;
    for (int t = 0; t < steps; ++t) {
        for (int64_t L = 1; L <= p.cfg.beam_width; ++L) {
            int fw = 0, rpw = 0;
            if (!fused_shape(p, t, L, &fw, &rpw) || fw < 2) continue;
            const size_t sl = (size_t)p.cfg.batch * fw;
            *slots = std::max(*slots, sl);
            *keys = std::max(*keys, sl * (size_t)p.cfg.beam_width * gr::kPartPerK);
        }
    }
}

static StepPlan plan_of(const gr_beam* h) {
    StepPlan p;
    p.cfg = h->cfg;
    p.trie = h->trie;
    p.gs = h->gs;
    p.select_lds = h->select_lds;
    p.max_lds = h->max_lds;
    p.temperature = h->temperature;
    p.seed = h->seed;
    p.alpha = h->alpha;
    p.pen_host = h->pen_host.empty() ? nullptr : h->pen_host.data();
    p.min_len = h->min_len;
    p.has_banned = h->has_banned;
    p.norm_mode = h->norm_mode;
    p.nlo = h->nlo;
    p.nhi = h->nhi;
    p.fused = h->fused;
    p.fused_split = h->fused_split;
    return p;
}

// The buffers of step t of handle h reading state half `in`.
static StepBuffers buffers_of(const gr_beam* h, int t, int in) {
    const size_t n = (size_t)h->cfg.batch * h->cfg.beam_width;
    const int on = 1 - in;
    StepBuffers u;
    u.score = h->score[in];
    u.node = h->node[in];
    u.fin = h->fin[in];
    u.seq = h->seq[in];
    u.score_o = h->score[on];
    u.node_o = h->node[on];
    u.fin_o = h->fin[on];
    u.seq_o = h->seq[on];
    u.parent_o = h->parents + (size_t)t * n;
    u.token_o = h->tokens + (size_t)t * n;
    u.lse = h->lse;
    u.pool = h->pool;
    u.cnt = h->cnt;
    u.ncand = h->ncand;
    u.rbase = h->rbase;
    u.rworst = h->rworst;
    u.stats = h->stats;
    u.pen = h->pen;
    u.banned = h->has_banned ? h->banned : nullptr;
    u.banned_list = h->banned_list;
    u.n_banned = h->has_banned ? h->n_banned : 0;
    u.part = h->part;
    u.part_n = h->part_n;
    u.part_stats = h->part_stats;
    u.req_theta = h->req_theta;
    u.part_keys = h->part_keys;
    u.part_slots = h->part_slots;
    return u;
}

static void harvest_timing(gr_beam* h, bool wait_all) {
    while (h->ev_pending > 0) {
        const int idx = (h->ev_head - h->ev_pending + kTimingRing) % kTimingRing;
        if (!wait_all && hipEventQuery(h->ev[idx][2]) != hipSuccess) {
            if (h->ev_pending < kTimingRing) return;
        }
        (void)hipEventSynchronize(h->ev[idx][2]);
        float a = 0.f, b = 0.f;
        if (h->ev_one[idx]) {
            (void)hipEventElapsedTime(&a, h->ev[idx][0], h->ev[idx][2]);
        } else {
            (void)hipEventElapsedTime(&a, h->ev[idx][0], h->ev[idx][1]);
            (void)hipEventElapsedTime(&b, h->ev[idx][1], h->ev[idx][2]);
        }
        h->row_ms += a;
        h->sel_ms += b;
        h->timed_steps += 1;
        h->ev_pending -= 1;
    }
}

// ------------------------------------------------------------------ trie

extern "C" gr_status gr_trie_validate(int32_t depth, int32_t vocab, const int64_t* num_nodes,
                                      const int64_t* const* node_offsets,
                                      const int32_t* const* child_tokens,
                                      const int32_t* const* child_nodes) {
    if (depth < 1) return fail(GR_ERR_INVALID_ARG, "depth %d < 1", depth);
    if (vocab < 1) return fail(GR_ERR_INVALID_ARG, "vocab %d < 1", vocab);
    if (!num_nodes || !node_offsets || !child_tokens || !child_nodes)
        return fail(GR_ERR_INVALID_ARG, "NULL trie array");
    if (num_nodes[0] != 1) return fail(GR_ERR_BAD_TRIE, "num_nodes[0] = %lld, the root level must have 1 node",
                                       (long long)num_nodes[0]);
    for (int L = 0; L <= depth; ++L)
        if (num_nodes[L] < 0 || num_nodes[L] > INT32_MAX)
            return fail(GR_ERR_BAD_TRIE, "num_nodes[%d] = %lld out of range", L, (long long)num_nodes[L]);
    for (int L = 0; L < depth; ++L) {
        const int64_t* off = node_offsets[L];
        const int32_t* tok = child_tokens[L];
        const int32_t* ch = child_nodes[L];
        const int64_t n = num_nodes[L];
        if (!off) return fail(GR_ERR_INVALID_ARG, "node_offsets[%d] is NULL", L);
        if (off[0] != 0) return fail(GR_ERR_BAD_TRIE, "level %d: offsets[0] = %lld, must be 0", L, (long long)off[0]);
        for (int64_t i = 0; i < n; ++i)
            if (off[i + 1] < off[i])
                return fail(GR_ERR_BAD_TRIE, "level %d: offsets decrease at node %lld", L, (long long)i);
        const int64_t E = off[n];
        if (E > INT32_MAX) return fail(GR_ERR_BAD_TRIE, "level %d: %lld edges exceed 2^31-1", L, (long long)E);
        if (E > 0 && (!tok || !ch)) return fail(GR_ERR_INVALID_ARG, "level %d: NULL token or child array", L);
        for (int64_t i = 0; i < n; ++i) {
            for (int64_t e = off[i]; e < off[i + 1]; ++e) {
                if (tok[e] < 0 || tok[e] >= vocab)
                    return fail(GR_ERR_BAD_TRIE, "level %d edge %lld: token %d outside [0, %d)", L,
                                (long long)e, tok[e], vocab);
                if (e > off[i] && tok[e] <= tok[e - 1])
                    return fail(GR_ERR_BAD_TRIE,
                                "level %d node %lld: child tokens not strictly increasing at edge %lld", L,
                                (long long)i, (long long)e);
                if (ch[e] < 0 || (int64_t)ch[e] >= num_nodes[L + 1])
                    return fail(GR_ERR_BAD_TRIE, "level %d edge %lld: child node %d outside [0, %lld)", L,
                                (long long)e, ch[e], (long long)num_nodes[L + 1]);
            }
        }
    }
    return GR_OK;
}

extern "C" gr_status gr_trie_build(int32_t depth, int32_t vocab, const int64_t* num_nodes,
                                   const int64_t* const* node_offsets,
                                   const int32_t* const* child_tokens,
                                   const int32_t* const* child_nodes, gr_stream stream,
                                   gr_trie** out) {
    if (!out) return fail(GR_ERR_INVALID_ARG, "out is NULL");
    gr_status st = gr_trie_validate(depth, vocab, num_nodes, node_offsets, child_tokens, child_nodes);
    if (st != GR_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    gr_trie* t = new (std::nothrow) gr_trie();
    if (!t) return fail(GR_ERR_OUT_OF_MEMORY, "host allocation failed");
    t->depth = depth;
    t->vocab = vocab;
    t->num_nodes.assign(num_nodes, num_nodes + depth + 1);
    t->off.assign(depth, nullptr);
    t->tok.assign(depth, nullptr);
    t->child.assign(depth, nullptr);
    t->max_fan.assign(depth, 0);
    t->tmin.assign(depth, 0);
    t->tmax.assign(depth, -1);
    t->dense.assign(depth, nullptr);
    for (int L = 0; L < depth; ++L) {
        const int64_t n = num_nodes[L];
        const int64_t E = node_offsets[L][n];
        int64_t mf = 0;
        for (int64_t i = 0; i < n; ++i) mf = std::max(mf, node_offsets[L][i + 1] - node_offsets[L][i]);
        t->max_fan[L] = (int32_t)mf;
        if (E > 0) {
            const auto mm = std::minmax_element(child_tokens[L], child_tokens[L] + E);
            t->tmin[L] = *mm.first;
            t->tmax[L] = *mm.second;
        }
        hipError_t e = dalloc(&t->off[L], (size_t)n + 1);
        if (e == hipSuccess) e = dalloc(&t->tok[L], (size_t)E);
        if (e == hipSuccess) e = dalloc(&t->child[L], (size_t)E);
        if (e == hipSuccess)
            e = hipMemcpyAsync(t->off[L], node_offsets[L], sizeof(int64_t) * (n + 1), hipMemcpyHostToDevice, s);
        if (e == hipSuccess && E > 0)
            e = hipMemcpyAsync(t->tok[L], child_tokens[L], sizeof(int32_t) * E, hipMemcpyHostToDevice, s);
        if (e == hipSuccess && E > 0)
            e = hipMemcpyAsync(t->child[L], child_nodes[L], sizeof(int32_t) * E, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) {
            gr_trie_free(t);
            return e == hipErrorOutOfMemory ? fail(GR_ERR_OUT_OF_MEMORY, "trie level %d: %s", L, hipGetErrorString(e))
                                            : hip_fail(e, "trie upload");
        }
    }
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        gr_trie_free(t);
        return hip_fail(e, "trie upload sync");
    }
    *out = t;
    return GR_OK;
}

extern "C" gr_status gr_trie_info(const gr_trie* trie, int32_t* depth, int32_t* vocab, int64_t* num_nodes,
                                  int32_t* max_fanout) {
    if (!trie) return fail(GR_ERR_INVALID_ARG, "trie is NULL");
    if (depth) *depth = trie->depth;
    if (vocab) *vocab = trie->vocab;
    if (num_nodes) std::copy(trie->num_nodes.begin(), trie->num_nodes.end(), num_nodes);
    if (max_fanout) std::copy(trie->max_fan.begin(), trie->max_fan.end(), max_fanout);
    return GR_OK;
}

extern "C" void gr_trie_free(gr_trie* trie) {
    if (!trie) return;
    for (size_t L = 0; L < trie->off.size(); ++L) {
        (void)hipFree(trie->off[L]);
        (void)hipFree(trie->tok[L]);
        (void)hipFree(trie->child[L]);
        if (L < trie->dense.size()) (void)hipFree(trie->dense[L]);
    }
    delete trie;
}

extern "C" gr_status gr_trie_densify(gr_trie* trie, int32_t level, int64_t max_bytes, gr_stream stream,
                                     int64_t* table_bytes) {
    if (!trie) return fail(GR_ERR_INVALID_ARG, "trie is NULL");
    if (level < 0 || level >= trie->depth) return fail(GR_ERR_INVALID_ARG, "level %d not in [0, %d)", level, trie->depth);
    const int64_t span = (int64_t)trie->tmax[level] - trie->tmin[level] + 1;
    const int64_t n = trie->num_nodes[level];
    const int64_t bytes = span > 0 ? n * span * (int64_t)sizeof(int32_t) : 0;
    if (table_bytes) *table_bytes = bytes;
    if (trie->dense[level] || bytes == 0) return GR_OK;  // already dense, or no edges
    if (max_bytes >= 0 && bytes > max_bytes)
        return fail(GR_ERR_UNSUPPORTED, "level %d: dense table of %lld bytes exceeds %lld", level, (long long)bytes,
                    (long long)max_bytes);
    hipStream_t s = (hipStream_t)stream;
    int32_t* d = nullptr;
    hipError_t e = dalloc(&d, (size_t)(n * span));
    if (e != hipSuccess)
        return e == hipErrorOutOfMemory ? fail(GR_ERR_OUT_OF_MEMORY, "dense level %d: %s", level, hipGetErrorString(e))
                                        : hip_fail(e, "dense table allocation");
    e = gr::launch_trie_densify(trie->off[level], trie->tok[level], trie->child[level], n, trie->tmin[level],
                                (int32_t)span, d, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e, "dense table build");
    }
    trie->dense[level] = d;
    return GR_OK;
}

// ------------------------------------------------------------------ beam

// Configuration rules shared by gr_beam_init and the no-allocation step; a
// zero row stride becomes V.
static gr_status check_config(gr_beam_config* c, const gr_trie* trie) {
    gr_beam_config& cfg = *c;
    if (cfg.batch < 1) return fail(GR_ERR_INVALID_ARG, "batch %d < 1", cfg.batch);
    if (cfg.beam_width < 1 || cfg.beam_width > gr::kMaxBeam)
        return fail(GR_ERR_INVALID_ARG, "beam_width %d outside [1, %d]", cfg.beam_width, gr::kMaxBeam);
    if (cfg.vocab < 1 || cfg.vocab > (1 << 30)) return fail(GR_ERR_INVALID_ARG, "vocab %d outside [1, 2^30]", cfg.vocab);
    if ((uint64_t)cfg.beam_width * (uint64_t)cfg.vocab >= (1ull << 32))
        return fail(GR_ERR_INVALID_ARG, "K*V = %llu must be < 2^32",
                    (unsigned long long)cfg.beam_width * (unsigned long long)cfg.vocab);
    if ((int64_t)cfg.batch * cfg.beam_width > INT32_MAX)
        return fail(GR_ERR_INVALID_ARG, "B*K too large");
    if (cfg.max_steps < 1) return fail(GR_ERR_INVALID_ARG, "max_steps %d < 1", cfg.max_steps);
    if (cfg.eos_token < -1 || cfg.eos_token >= cfg.vocab)
        return fail(GR_ERR_INVALID_ARG, "eos_token %d outside [-1, V)", cfg.eos_token);
    if (cfg.logits_dtype != GR_F32 && cfg.logits_dtype != GR_BF16)
        return fail(GR_ERR_INVALID_ARG, "logits_dtype %d is neither GR_F32 nor GR_BF16", cfg.logits_dtype);
    if (cfg.logits_row_stride == 0) cfg.logits_row_stride = cfg.vocab;
    if (cfg.logits_row_stride < cfg.vocab)
        return fail(GR_ERR_INVALID_ARG, "row stride %lld < vocab", (long long)cfg.logits_row_stride);
    if (trie) {
        if (trie->vocab != cfg.vocab)
            return fail(GR_ERR_INVALID_ARG, "trie vocab %d != config vocab %d", trie->vocab, cfg.vocab);
        if (cfg.max_steps > trie->depth)
            return fail(GR_ERR_INVALID_ARG, "max_steps %d > trie depth %d", cfg.max_steps, trie->depth);
        if (cfg.eos_token != -1) return fail(GR_ERR_INVALID_ARG, "eos_token must be -1 with a trie");
    }
    return GR_OK;
}

static void beam_release(gr_beam* h) {
    for (int i = 0; i < 2; ++i) {
        (void)hipFree(h->score[i]);
        (void)hipFree(h->node[i]);
        (void)hipFree(h->fin[i]);
        (void)hipFree(h->seq[i]);
    }
    (void)hipFree(h->parents);
    (void)hipFree(h->tokens);
    (void)hipFree(h->lse);
    (void)hipFree(h->pool);
    (void)hipFree(h->cnt);
    (void)hipFree(h->ncand);
    (void)hipFree(h->rbase);
    (void)hipFree(h->rworst);
    (void)hipFree(h->banned);
    (void)hipFree(h->banned_list);
    (void)hipFree(h->pen);
    (void)hipFree(h->stats);
    (void)hipFree(h->live_dev);
    (void)hipFree(h->part);
    (void)hipFree(h->part_n);
    (void)hipFree(h->part_stats);
    (void)hipFree(h->req_theta);
    for (auto& g : h->graphs)
        if (g.exec) (void)hipGraphExecDestroy(g.exec);
    h->graphs.clear();
    if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
    if (h->ev_made)
        for (int i = 0; i < kTimingRing; ++i)
            for (int k = 0; k < 3; ++k) (void)hipEventDestroy(h->ev[i][k]);
}

extern "C" gr_status gr_beam_init(const gr_beam_config* cfg_in, const gr_trie* trie, gr_stream stream,
                                  gr_beam** out) {
    if (!cfg_in || !out) return fail(GR_ERR_INVALID_ARG, "NULL config or out");
    gr_beam_config cfg = *cfg_in;
    if (gr_status e = check_config(&cfg, trie)) return e;

    gr_beam* h = new (std::nothrow) gr_beam();
    if (!h) return fail(GR_ERR_OUT_OF_MEMORY, "host allocation failed");
    h->cfg = cfg;
    h->trie = trie;
    const size_t B = cfg.batch, K = cfg.beam_width, T = cfg.max_steps;
    const size_t n = B * K;

    const int max_lds = device_lds_limit();
    h->max_lds = max_lds;
    if (!select_plan((int)K, max_lds, &h->sb, &h->gs, &h->select_lds)) {
        delete h;
        return fail(GR_ERR_UNSUPPORTED, "beam width %d leaves no LDS for selection", (int)K);
    }
    const size_t row_lds_max = row_lds_need(plan_of(h));
    if (row_lds_max > (size_t)max_lds) {
        delete h;
        return fail(GR_ERR_UNSUPPORTED, "row kernel needs %zu B of LDS > device limit %d", row_lds_max, max_lds);
    }
    h->pool_cap = B * (size_t)h->gs;  // L*s <= gs rows x slots per request

    hipError_t e = hipSuccess;
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
        e = dalloc(&h->score[i], n);
        if (e == hipSuccess) e = dalloc(&h->node[i], n);
        if (e == hipSuccess) e = dalloc(&h->fin[i], n);
        if (e == hipSuccess) e = dalloc(&h->seq[i], n * T);
    }
    if (e == hipSuccess) e = dalloc(&h->parents, n * T);
    if (e == hipSuccess) e = dalloc(&h->tokens, n * T);
    if (e == hipSuccess) e = dalloc(&h->lse, n);
    if (e == hipSuccess) e = dalloc(&h->pool, h->pool_cap);
    if (e == hipSuccess) e = dalloc(&h->cnt, n);
    if (e == hipSuccess) e = dalloc(&h->ncand, n);
    if (e == hipSuccess) e = dalloc(&h->rbase, n);
    if (e == hipSuccess) e = dalloc(&h->rworst, n);
    if (e == hipSuccess) e = dalloc(&h->banned, ((size_t)cfg.vocab + 31) / 32);
    if (e == hipSuccess) e = dalloc(&h->banned_list, (size_t)cfg.vocab);
    if (e == hipSuccess) e = dalloc(&h->pen, T + 1);
    h->pen_host.assign(T + 1, 1.0f);
    if (e == hipSuccess)
        e = hipMemcpy(h->pen, h->pen_host.data(), (T + 1) * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = dalloc(&h->stats, B * gr::kNumStats);
    if (e == hipSuccess) e = dalloc(&h->live_dev, 1);
    {  // the fused step's workspace, for the split steps too (they can be
       // switched on later); its counters and bounds start at zero
        size_t keys = 0, slots = 0;
        StepPlan pl = plan_of(h);
        pl.fused_split = true;
        fused_need(pl, &keys, &slots);
        h->part_keys = keys;
        h->part_slots = slots;
        if (e == hipSuccess && keys) e = dalloc(&h->part, keys);
        if (e == hipSuccess && slots) e = dalloc(&h->part_n, slots);
        if (e == hipSuccess && slots) e = dalloc(&h->part_stats, 2 * slots);
        if (e == hipSuccess) e = dalloc(&h->req_theta, B);
        if (e == hipSuccess) e = hipMemset(h->req_theta, 0, B * sizeof(unsigned long long));
    }
    if (e != hipSuccess) {
        beam_release(h);
        delete h;
        return e == hipErrorOutOfMemory ? fail(GR_ERR_OUT_OF_MEMORY, "beam state: %s", hipGetErrorString(e))
                                        : hip_fail(e, "beam state allocation");
    }
    // Each kernel's dynamic-LDS limit is a property of the function, shared by
    // every handle: it is set to the device's limit (the same value on every
    // call), never to this handle's needs, which could lower it under another
    // live handle that needs more.  Launches still request only what they use.
    e = gr::set_row_lds_limit(max_lds);
    if (e == hipSuccess) e = gr::set_select_lds_limit(max_lds);
    if (e == hipSuccess) e = gr::set_fused_lds_limit(max_lds);
    if (e != hipSuccess) {
        beam_release(h);
        delete h;
        return hip_fail(e, "setting the kernels' LDS limit");
    }
    gr_status st = gr_beam_reset(h, stream);
    if (st == GR_OK) {
        e = hipStreamSynchronize((hipStream_t)stream);
        if (e != hipSuccess) st = hip_fail(e, "beam init sync");
    }
    if (st != GR_OK) {
        beam_release(h);
        delete h;
        return st;
    }
    *out = h;
    return GR_OK;
}

extern "C" gr_status gr_beam_set_sampling(gr_beam* h, float temperature, uint64_t seed) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    if (!(temperature >= 0.0f) || std::isinf(temperature))
        return fail(GR_ERR_INVALID_ARG, "temperature %g must be finite and >= 0", (double)temperature);
    h->temperature = temperature;
    h->seed = seed;
    return GR_OK;
}

extern "C" gr_status gr_beam_set_penalties(gr_beam* h, float alpha, int32_t min_length,
                                           const int32_t* banned, int32_t n_banned, gr_stream stream) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    if (!std::isfinite(alpha)) return fail(GR_ERR_INVALID_ARG, "alpha %g is not finite", (double)alpha);
    if (min_length < 0) return fail(GR_ERR_INVALID_ARG, "min_length %d < 0", min_length);
    if (n_banned < 0 || (n_banned > 0 && !banned))
        return fail(GR_ERR_INVALID_ARG, "banned list: NULL pointer or negative count %d", n_banned);
    const int V = h->cfg.vocab, T = h->cfg.max_steps;
    std::vector<uint32_t> bits(((size_t)V + 31) / 32, 0u);
    std::vector<int32_t> list;
    for (int32_t i = 0; i < n_banned; ++i) {
        const int32_t v = banned[i];
        if (v < 0 || v >= V) return fail(GR_ERR_INVALID_ARG, "banned token %d outside [0, %d)", v, V);
        if (!(bits[(size_t)v >> 5] & (1u << (v & 31)))) list.push_back(v);
        bits[(size_t)v >> 5] |= 1u << (v & 31);
    }

    // pen(len) = ((5 + len) / 6) ** alpha in double, rounded to float
    std::vector<float> pen(T + 1);
    for (int len = 0; len <= T; ++len) pen[len] = (float)std::pow((5.0 + len) / 6.0, (double)alpha);
    hipStream_t st = (hipStream_t)stream;
    HIP_TRY(hipMemcpyAsync(h->banned, bits.data(), bits.size() * sizeof(uint32_t), hipMemcpyHostToDevice, st),
            "banned tokens copy");
    HIP_TRY(hipMemcpyAsync(h->pen, pen.data(), pen.size() * sizeof(float), hipMemcpyHostToDevice, st),
            "penalty table copy");
    if (!list.empty())
        HIP_TRY(hipMemcpyAsync(h->banned_list, list.data(), list.size() * sizeof(int32_t),
                               hipMemcpyHostToDevice, st),
                "banned list copy");
    HIP_TRY(hipStreamSynchronize(st), "penalties sync");  // the host vectors go out of scope
    h->n_banned = (int32_t)list.size();
    h->alpha = alpha;
    h->min_len = min_length;
    h->has_banned = n_banned > 0;
    h->pen_host = pen;
    return GR_OK;
}

extern "C" gr_status gr_beam_set_fused(gr_beam* h, int32_t mode) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    if (mode < 0 || mode > 2) return fail(GR_ERR_INVALID_ARG, "fused mode %d not in 0..2", mode);
    h->fused = mode != 0;
    h->fused_split = mode == 2;
    return GR_OK;
}

extern "C" gr_status gr_beam_set_normalization(gr_beam* h, int32_t mode, int32_t lo, int32_t hi) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    if (mode < GR_NORM_FULL || mode > GR_NORM_NONE) return fail(GR_ERR_INVALID_ARG, "unknown normalisation mode %d", mode);
    if (mode == GR_NORM_RANGE && !(0 <= lo && lo < hi && hi <= h->cfg.vocab))
        return fail(GR_ERR_INVALID_ARG, "range [%d, %d) not inside [0, %d)", lo, hi, h->cfg.vocab);
    h->norm_mode = mode;
    h->nlo = lo;
    h->nhi = hi;
    return GR_OK;
}

extern "C" gr_status gr_beam_reset(gr_beam* h, gr_stream stream) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    const gr_beam_config& c = h->cfg;
    h->cur = 0;
    HIP_TRY(gr::launch_reset(h->score[0], h->node[0], h->fin[0], h->seq[0], h->parents, h->tokens, h->lse,
                             c.batch, c.beam_width, c.max_steps, h->trie ? 0 : -1, (hipStream_t)stream),
            "reset kernel");
    h->t = 0;
    h->live = 1;
    h->can_rewind = false;
    h->last_stream = (hipStream_t)stream;
    return GR_OK;
}

extern "C" gr_status gr_beam_rewind(gr_beam* h) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    if (!h->can_rewind) return fail(GR_ERR_STATE, "no step to rewind (only the last step, once)");
    h->cur = 1 - h->cur;
    h->t -= 1;
    h->live = h->live_prev;
    h->can_rewind = false;
    return GR_OK;
}

// The arguments of step t with live bound L on the buffers u and the logits
// at d_logits.  pool_keys: the summary keys the pool holds.
static gr_status make_step_args(const StepPlan& p, int t, int64_t L, const StepBuffers& u, const void* d_logits,
                                size_t pool_keys, StepArgs* out) {
    const gr_beam_config& c = p.cfg;
    const StepShape sh = step_shape(p, t, L);
    StepArgs a;
    memset(&a, 0, sizeof(a));  // padding too: cached graphs compare whole argument blocks
    a.B = c.batch;
    a.K = c.beam_width;
    a.V = c.vocab;
    a.T = c.max_steps;
    a.t = t;
    a.L = (int32_t)L;
    a.s = sh.s;
    a.max_lds = p.max_lds;
    a.F = p.trie ? std::max<int32_t>(1, p.trie->max_fan[t]) : c.vocab;
    a.eos = c.eos_token;
    a.cap = sh.cap;
    a.stg = sh.stg;
    // the step's grid holds L*s slots (even: the survivor buffer after it is
    // 8-byte aligned); the survivor buffer takes the rest of the request
    // kernel's LDS (at least sb keys, many more when L*s is well below gs)
    a.gs = (int32_t)((L * sh.s + 1) & ~(int64_t)1);
    a.sb = gr::select_buffer_fit(p.select_lds, a.gs, c.beam_width, (int)L);
    a.sampling = p.temperature > 0.0f;
    a.inv_t = a.sampling ? 1.0f / p.temperature : 1.0f;
    a.seed = p.seed;
    a.penal = p.alpha != 0.0f;
    a.pen_live = a.penal && p.pen_host ? p.pen_host[t + 1] : 1.0f;
    a.pen = u.pen;
    a.min_len = p.min_len;
    a.banned = u.banned;
    a.banned_list = u.banned_list;
    a.n_banned = u.n_banned;
    a.rank_is_c = !(a.sampling || a.penal);
    a.norm_mode = p.norm_mode;
    a.nlo = p.norm_mode == 1 ? p.nlo : 0;
    a.nhi = p.norm_mode == 1 ? p.nhi : c.vocab;
    a.s_log2 = sh.s_log2;
    a.stride = c.logits_row_stride;
    if (p.trie) {
        a.off = p.trie->off[t];
        a.tok = p.trie->tok[t];
        a.child = p.trie->child[t];
        a.nnodes = p.trie->num_nodes[t];
        if (p.trie->dense[t]) {
            a.child = p.trie->dense[t];
            a.dspan = p.trie->tmax[t] - p.trie->tmin[t] + 1;
            a.dbase = p.trie->tmin[t];
            a.F = a.dspan;
        }
    }
    a.logits = d_logits;
    a.score = u.score;
    a.node = u.node;
    a.fin = u.fin;
    a.seq = u.seq;
    a.score_o = u.score_o;
    a.node_o = u.node_o;
    a.fin_o = u.fin_o;
    a.seq_o = u.seq_o;
    a.parent_o = u.parent_o;
    a.token_o = u.token_o;
    a.lse_o = u.lse;
    a.pool = u.pool;
    a.cnt = u.cnt;
    a.ncand = u.ncand;
    a.rbase = u.rbase;
    a.rworst = u.rworst;
    a.stats = u.stats;
    int fw = 0, rpw = 0;
    if (fused_shape(p, t, L, &fw, &rpw) &&
        (fw == 1 || ((size_t)c.batch * fw * c.beam_width * gr::kPartPerK <= u.part_keys &&
                     (size_t)c.batch * fw <= u.part_slots &&
                     u.req_theta))) {
        a.fw = fw;
        a.rpw = rpw;
        // the key buffer: every candidate of the workgroup's rows (a split
        // workgroup's LDS, so more of them fit on a CU); a whole request's
        // also holds its winners padded to a power of two for the sort
        a.fcap = fw == 1 ? gr::kFusedCap
                         : (int)std::min<int64_t>(gr::kFusedCap,
                                                  (int64_t)rpw * std::max<int32_t>(1, p.trie->max_fan[t]));
        a.part = u.part;
        a.part_n = u.part_n;
        a.part_stats = u.part_stats;
        a.req_theta = u.req_theta;
    }
    if ((size_t)c.batch * L * sh.s > pool_keys || L * sh.s > p.gs)
        return fail(GR_ERR_STATE, "workspace too small for step %d (internal error)", t);
    *out = a;
    return GR_OK;
}

static gr_status make_step_args(const gr_beam* h, int t, int64_t L, int in, const void* d_logits, StepArgs* out) {
    return make_step_args(plan_of(h), t, L, buffers_of(h, t, in), d_logits, h->pool_cap, out);
}

// Step t may run: within max_steps and the trie depth.
static gr_status check_step(const gr_beam_config& c, const gr_trie* trie, int t) {
    if (t >= c.max_steps) return fail(GR_ERR_STATE, "step %d: max_steps %d reached", t, c.max_steps);
    if (trie && t >= trie->depth)
        return fail(GR_ERR_STATE, "step %d: trie depth %d reached", t, trie->depth);
    return GR_OK;
}
static gr_status check_step(const gr_beam* h, int t) { return check_step(h->cfg, h->trie, t); }

// Live bound after step t with live bound L.
static int64_t next_live(const gr_beam* h, int t, int64_t L) {
    const int64_t mc = std::max<int64_t>(1, max_candidates(plan_of(h), t));
    return std::min<int64_t>((int64_t)h->cfg.beam_width, L * mc);
}

extern "C" gr_status gr_beam_step(gr_beam* h, const void* d_logits, gr_stream stream) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    if (!d_logits) return fail(GR_ERR_INVALID_ARG, "logits pointer is NULL");
    const gr_beam_config& c = h->cfg;
    if (gr_status e = check_step(h, h->t)) return e;
    hipStream_t st = (hipStream_t)stream;
    const int t = h->t;
    const int64_t L = std::min<int64_t>(h->live, c.beam_width);
    StepArgs a;
    if (gr_status e = make_step_args(h, t, L, h->cur, d_logits, &a)) return e;
    const int on = 1 - h->cur;

    int slot = 0;
    if (h->timing) {
        if (!h->ev_made) {
            for (int i = 0; i < kTimingRing; ++i)
                // timing-only events: no system-scope fence (cache writeback and
                // invalidation) at each record, which would perturb the step
                for (int k = 0; k < 3; ++k)
                    HIP_TRY(hipEventCreateWithFlags(&h->ev[i][k], hipEventDisableSystemFence), "event create");
            h->ev_made = true;
        }
        if (h->ev_pending == kTimingRing) harvest_timing(h, false);
        slot = h->ev_head;
        HIP_TRY(hipEventRecord(h->ev[slot][0], st), "event record");
    }
    // a fused step's row work counts as the row kernel's time and its merge,
    // when the requests were split, as the request kernel's
    if (h->timing) h->ev_one[slot] = a.fw == 1;
    if (a.fw > 0) {
        HIP_TRY(gr::launch_fused(a, c.logits_dtype == GR_BF16, st), "fused step launch");
        if (a.fw > 1) {
            if (h->timing) HIP_TRY(hipEventRecord(h->ev[slot][1], st), "event record");
            HIP_TRY(gr::launch_merge(a, st), "merge launch");
        }
    } else {
        HIP_TRY(gr::launch_rows(a, c.logits_dtype == GR_BF16, st), "row kernel launch");
        if (h->timing) HIP_TRY(hipEventRecord(h->ev[slot][1], st), "event record");
        HIP_TRY(gr::launch_select(a, c.logits_dtype == GR_BF16, st), "select kernel launch");
    }
    if (h->timing) {
        HIP_TRY(hipEventRecord(h->ev[slot][2], st), "event record");
        h->ev_head = (h->ev_head + 1) % kTimingRing;
        h->ev_pending += 1;
    }
    h->cur = on;
    h->t = t + 1;
    h->live_prev = h->live;
    h->live = next_live(h, t, L);
    h->can_rewind = true;
    h->last_stream = st;
    return GR_OK;
}

static constexpr size_t kGraphCache = 8;

static bool same_args(const std::vector<StepArgs>& x, const std::vector<StepArgs>& y) {
    return x.size() == y.size() && memcmp(x.data(), y.data(), x.size() * sizeof(StepArgs)) == 0;
}

extern "C" gr_status gr_beam_search(gr_beam* h, const void* const* d_logits, int32_t nsteps, gr_stream stream) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    if (!d_logits) return fail(GR_ERR_INVALID_ARG, "logits pointer list is NULL");
    if (nsteps < 1) return fail(GR_ERR_INVALID_ARG, "nsteps %d < 1", nsteps);
    const gr_beam_config& c = h->cfg;
    for (int i = 0; i < nsteps; ++i) {
        if (!d_logits[i]) return fail(GR_ERR_INVALID_ARG, "logits pointer of step %d is NULL", i);
        if (gr_status e = check_step(h, h->t + i)) return e;
    }
    // the launches of every step, from the host state alone
    std::vector<StepArgs> args((size_t)nsteps);
    int64_t L = std::min<int64_t>(h->live, c.beam_width), L_last = L;
    int cur = h->cur;
    for (int i = 0; i < nsteps; ++i) {
        if (gr_status e = make_step_args(h, h->t + i, L, cur, d_logits[i], &args[(size_t)i])) return e;
        L_last = L;
        L = next_live(h, h->t + i, L);
        cur = 1 - cur;
    }
    const bool bf16 = c.logits_dtype == GR_BF16;
    // every step a one-workgroup fused step: the steps run in one launch
    // (kSearchSteps at a time), each request's workgroup stepping through them
    bool one_wg = true;
    for (const StepArgs& a : args) one_wg = one_wg && a.fw == 1;
    if (one_wg) {
        for (int i0 = 0; i0 < nsteps; i0 += gr::kSearchSteps) {
            gr::SearchArgs sa;
            memset(&sa, 0, sizeof(sa));
            sa.n = std::min(nsteps - i0, gr::kSearchSteps);
            for (int k = 0; k < sa.n; ++k) sa.step[k] = args[(size_t)(i0 + k)];
            const hipError_t le = gr::launch_fused_search(sa, bf16, (hipStream_t)stream);
            if (le != hipSuccess) {
                if (i0 > 0) {  // the first i0 steps are enqueued: the handle follows them
                    h->t += i0;
                    h->cur = (h->cur + i0) & 1;
                    h->live_prev = args[(size_t)(i0 - 1)].L;
                    h->live = args[(size_t)i0].L;
                    h->can_rewind = true;
                    h->last_stream = (hipStream_t)stream;
                }
                return hip_fail(le, i0 > 0 ? "search launch (its first steps are enqueued)" : "search launch");
            }
        }
    }
    gr_beam::Graph* g = nullptr;
    if (!one_wg)
        for (auto& e : h->graphs)
            if (same_args(e.args, args)) g = &e;
    if (!one_wg && !g) {
        if (!h->cap_stream)
            HIP_TRY(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking), "capture stream");
        HIP_TRY(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal), "begin capture");
        hipError_t le = hipSuccess;
        for (int i = 0; i < nsteps && le == hipSuccess; ++i) {
            le = gr::launch_step(args[(size_t)i], bf16, h->cap_stream);
        }
        hipGraph_t graph = nullptr;
        const hipError_t ce = hipStreamEndCapture(h->cap_stream, &graph);
        if (le != hipSuccess || ce != hipSuccess) {
            if (graph) (void)hipGraphDestroy(graph);
            return hip_fail(le != hipSuccess ? le : ce, "capturing the search");
        }
        hipGraphExec_t exec = nullptr;
        const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (ie != hipSuccess) return hip_fail(ie, "instantiating the search graph");
        if (h->graphs.size() >= kGraphCache) {
            auto lru = std::min_element(h->graphs.begin(), h->graphs.end(),
                                        [](const gr_beam::Graph& x, const gr_beam::Graph& y) { return x.used < y.used; });
            (void)hipGraphExecDestroy(lru->exec);
            h->graphs.erase(lru);
        }
        h->graphs.push_back(gr_beam::Graph{std::move(args), exec, 0});
        g = &h->graphs.back();
    }
    if (g) {
        g->used = ++h->graph_clock;
        HIP_TRY(hipGraphLaunch(g->exec, (hipStream_t)stream), "search graph launch");
    }
    h->t += nsteps;
    h->cur = cur;
    h->live_prev = L_last;
    h->live = L;
    h->can_rewind = true;
    h->last_stream = (hipStream_t)stream;
    return GR_OK;
}

// ----------------------------------------------------- no-allocation step

// The workspace of gr_beam_step_static: one per GPU, for the life of the
// process.  Host code never uses this name as an address (on the host it
// is only a stand-in): each device's copy is found once with
// hipGetSymbolAddress and that address is what the kernels receive.
static __device__ __align__(256) uint8_t scratch[GR_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
constexpr size_t kStaticMaxRequests = 8192;  // requests the fused step's counters cover
struct StaticDevice {
    std::once_flag once;
    void* ptr = nullptr;   // this device's scratch
    hipError_t err = hipSuccess;
    int max_lds = 0;
};
StaticDevice g_static[kMaxDevices];

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}
}  // namespace

extern "C" gr_status gr_beam_step_static(const gr_step_io* io, gr_stream stream) {
    if (!io) return fail(GR_ERR_INVALID_ARG, "io is NULL");
    gr_beam_config cfg = io->config;
    if (gr_status e = check_config(&cfg, io->trie)) return e;
    if (!io->logits || !io->scores || !io->nodes || !io->finished || !io->sequences || !io->scores_out ||
        !io->nodes_out || !io->finished_out || !io->sequences_out || !io->parents_out || !io->tokens_out ||
        !io->lse_out)
        return fail(GR_ERR_INVALID_ARG, "NULL buffer in io");
    if (io->step < 0) return fail(GR_ERR_INVALID_ARG, "step %d < 0", io->step);
    if (gr_status e = check_step(cfg, io->trie, io->step)) return e;
    if (io->live_bound < 0) return fail(GR_ERR_INVALID_ARG, "live_bound %d < 0", io->live_bound);
    if (!(io->temperature >= 0.0f) || std::isinf(io->temperature))
        return fail(GR_ERR_INVALID_ARG, "temperature %g must be finite and >= 0", (double)io->temperature);
    const size_t n = (size_t)cfg.batch * cfg.beam_width, T = cfg.max_steps;
    {  // outputs may not overlap inputs
        const void* in[4] = {io->scores, io->nodes, io->finished, io->sequences};
        const size_t nin[4] = {n * 4, n * 4, n, n * T * 4};
        const void* ou[7] = {io->scores_out, io->nodes_out, io->finished_out, io->sequences_out,
                             io->parents_out, io->tokens_out, io->lse_out};
        const size_t nou[7] = {n * 4, n * 4, n, n * T * 4, n * 4, n * 4, n * 4};
        for (int i = 0; i < 4; ++i)
            for (int k = 0; k < 7; ++k)
                if (overlaps(in[i], nin[i], ou[k], nou[k]))
                    return fail(GR_ERR_INVALID_ARG, "output buffer %d overlaps input buffer %d", k, i);
    }
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "current device");
    if (dev < 0 || dev >= kMaxDevices) return fail(GR_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    StaticDevice& sd = g_static[dev];
    // once per device, with that device current: its copy of the buffer and
    // the kernels' LDS limit
    std::call_once(sd.once, [&] {
        sd.err = hipGetSymbolAddress(&sd.ptr, HIP_SYMBOL(scratch));
        if (sd.err != hipSuccess) return;
        sd.max_lds = device_lds_limit();
        sd.err = gr::set_row_lds_limit(sd.max_lds);
        if (sd.err == hipSuccess) sd.err = gr::set_select_lds_limit(sd.max_lds);
        if (sd.err == hipSuccess) sd.err = gr::set_fused_lds_limit(sd.max_lds);
    });
    if (sd.err != hipSuccess) return hip_fail(sd.err, "static scratch set-up");

    StepPlan p;
    p.cfg = cfg;
    p.trie = io->trie;
    p.max_lds = sd.max_lds;
    p.temperature = io->temperature;
    p.seed = io->seed;
    int sb = 0;
    if (!select_plan(cfg.beam_width, p.max_lds, &sb, &p.gs, &p.select_lds))
        return fail(GR_ERR_UNSUPPORTED, "beam width %d leaves no LDS for selection", cfg.beam_width);
    const int t = io->step;
    const int64_t K = cfg.beam_width;
    const int64_t L = io->live_bound > 0 ? std::min<int64_t>(io->live_bound, K) : K;
    const StepShape sh = step_shape(p, t, L);
    if (gr::row_lds_launch_bytes(sh.cap, sh.stg, cfg.vocab, p.max_lds) > (size_t)p.max_lds)
        return fail(GR_ERR_UNSUPPORTED, "row kernel needs more LDS than the device has");

    // the workspace, carved from this device's buffer (256-byte aligned
    // parts).  The fused step's per-request bounds sit at a fixed place at
    // the front: zero when the library loads, and every fused step leaves
    // them zero.
    const size_t B = (size_t)cfg.batch;
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t o_theta = 0, o_front = up(kStaticMaxRequests * 8);
    const size_t rows = B * (size_t)L;
    const size_t keys = rows * (size_t)sh.s;
    const size_t o_pool = o_front, o_cnt = up(o_pool + keys * 8), o_ncand = up(o_cnt + rows * 4);
    const size_t o_rbase = up(o_ncand + rows * 4), o_rworst = up(o_rbase + rows * 8);
    const size_t o_stats = up(o_rworst + rows * 8), o_part = up(o_stats + B * gr::kNumStats * 8);
    p.fused = B <= kStaticMaxRequests;
    int fw = 0, rpw = 0;
    size_t slots = 0;
    if (fused_shape(p, t, L, &fw, &rpw) && fw > 1) slots = B * fw;
    const size_t o_part_n = up(o_part + slots * cfg.beam_width * gr::kPartPerK * 8);
    const size_t o_part_stats = up(o_part_n + slots * 4);
    size_t need = o_part_stats + slots * 16;
    if (need > GR_STATIC_SCRATCH_BYTES && slots) {  // without the fused step's buffers
        p.fused = false;
        slots = 0;
        need = o_part;
    }
    if (need > GR_STATIC_SCRATCH_BYTES)
        return fail(GR_ERR_UNSUPPORTED,
                    "step needs %zu bytes of static workspace (batch %d x live bound %lld rows, %d summary keys "
                    "each) > GR_STATIC_SCRATCH_BYTES = %zu",
                    need, cfg.batch, (long long)L, sh.s, (size_t)GR_STATIC_SCRATCH_BYTES);
    uint8_t* w = static_cast<uint8_t*>(sd.ptr);
    StepBuffers u;
    u.score = io->scores;
    u.node = io->nodes;
    u.fin = io->finished;
    u.seq = io->sequences;
    u.score_o = io->scores_out;
    u.node_o = io->nodes_out;
    u.fin_o = io->finished_out;
    u.seq_o = io->sequences_out;
    u.parent_o = io->parents_out;
    u.token_o = io->tokens_out;
    u.lse = io->lse_out;
    u.pool = reinterpret_cast<uint64_t*>(w + o_pool);
    u.cnt = reinterpret_cast<int32_t*>(w + o_cnt);
    u.ncand = reinterpret_cast<int32_t*>(w + o_ncand);
    u.rbase = reinterpret_cast<int64_t*>(w + o_rbase);
    u.rworst = reinterpret_cast<uint64_t*>(w + o_rworst);
    u.stats = reinterpret_cast<unsigned long long*>(w + o_stats);  // written by the step's last kernel
    u.req_theta = reinterpret_cast<unsigned long long*>(w + o_theta);
    u.part = reinterpret_cast<uint64_t*>(w + o_part);
    u.part_n = reinterpret_cast<int32_t*>(w + o_part_n);
    u.part_stats = reinterpret_cast<long long*>(w + o_part_stats);
    u.part_keys = slots * cfg.beam_width * gr::kPartPerK;
    u.part_slots = slots;
    StepArgs a;
    if (gr_status e = make_step_args(p, t, L, u, io->logits, keys, &a)) return e;
    HIP_TRY(gr::launch_step(a, cfg.logits_dtype == GR_BF16, (hipStream_t)stream), "step launch");
    return GR_OK;
}

extern "C" gr_status gr_beam_backward(gr_beam* h, const float* d_grad_final, int32_t* d_path_slot,
                                      int32_t* d_path_token, float* d_weight, gr_stream stream) {
    if (!h || !d_grad_final || !d_path_slot || !d_path_token || !d_weight)
        return fail(GR_ERR_INVALID_ARG, "NULL argument");
    if (h->t < 1) return fail(GR_ERR_STATE, "no step has been taken");
    const gr_beam_config& c = h->cfg;
    gr::BackwardArgs a;
    a.B = c.batch;
    a.K = c.beam_width;
    a.T = c.max_steps;
    a.steps = h->t;
    a.parents = h->parents;
    a.tokens = h->tokens;
    a.score = h->score[h->cur];
    a.seq = h->seq[h->cur];
    a.grad = d_grad_final;
    a.pen = h->pen;
    a.path_slot = d_path_slot;
    a.path_token = d_path_token;
    a.weight = d_weight;
    HIP_TRY(gr::launch_backward_paths(a, (hipStream_t)stream), "backward paths launch");
    h->last_stream = (hipStream_t)stream;
    return GR_OK;
}

extern "C" gr_status gr_beam_backward_scatter(gr_beam* h, int32_t step, const int32_t* d_path_slot,
                                              const int32_t* d_path_token, const float* d_weight, float* d_grad,
                                              int64_t grad_row_stride, gr_stream stream) {
    if (!h || !d_path_slot || !d_path_token || !d_weight || !d_grad)
        return fail(GR_ERR_INVALID_ARG, "NULL argument");
    const gr_beam_config& c = h->cfg;
    if (step < 0 || step >= h->t) return fail(GR_ERR_INVALID_ARG, "step %d outside [0, %d)", step, h->t);
    const int64_t stride = grad_row_stride == 0 ? c.vocab : grad_row_stride;
    if (stride < c.vocab) return fail(GR_ERR_INVALID_ARG, "row stride %lld < vocab %d", (long long)stride, c.vocab);
    gr::ScatterArgs a;
    a.B = c.batch;
    a.K = c.beam_width;
    a.V = c.vocab;
    a.t = step;
    a.stride = stride;
    a.path_slot = d_path_slot;
    a.path_token = d_path_token;
    a.weight = d_weight;
    a.grad = d_grad;
    HIP_TRY(gr::launch_backward_scatter(a, (hipStream_t)stream), "backward scatter launch");
    h->last_stream = (hipStream_t)stream;
    return GR_OK;
}

extern "C" gr_status gr_beam_view_get(const gr_beam* h, gr_beam_view* out) {
    if (!h || !out) return fail(GR_ERR_INVALID_ARG, "NULL beam or out");
    out->step = h->t;
    out->batch = h->cfg.batch;
    out->beam_width = h->cfg.beam_width;
    out->vocab = h->cfg.vocab;
    out->max_steps = h->cfg.max_steps;
    out->scores = h->score[h->cur];
    out->nodes = h->node[h->cur];
    out->finished = h->fin[h->cur];
    out->sequences = h->seq[h->cur];
    out->parents = h->parents;
    out->tokens = h->tokens;
    out->lse = h->lse;
    return GR_OK;
}

extern "C" gr_status gr_beam_set_state(gr_beam* h, int32_t step, const float* d_scores, const int32_t* d_nodes,
                                       const uint8_t* d_finished, const int32_t* d_sequences,
                                       gr_stream stream) {
    if (!h || !d_scores || !d_nodes || !d_finished || !d_sequences)
        return fail(GR_ERR_INVALID_ARG, "NULL argument");
    const gr_beam_config& c = h->cfg;
    if (step < 0 || step >= c.max_steps)
        return fail(GR_ERR_INVALID_ARG, "step %d outside [0, %d)", step, c.max_steps);
    hipStream_t st = (hipStream_t)stream;
    const size_t n = (size_t)c.batch * c.beam_width;
    const int k = h->cur;
    HIP_TRY(hipMemcpyAsync(h->score[k], d_scores, n * sizeof(float), hipMemcpyDeviceToDevice, st), "copy scores");
    HIP_TRY(hipMemcpyAsync(h->node[k], d_nodes, n * sizeof(int32_t), hipMemcpyDeviceToDevice, st), "copy nodes");
    HIP_TRY(hipMemcpyAsync(h->fin[k], d_finished, n, hipMemcpyDeviceToDevice, st), "copy finished");
    HIP_TRY(hipMemcpyAsync(h->seq[k], d_sequences, n * c.max_steps * sizeof(int32_t), hipMemcpyDeviceToDevice, st),
            "copy sequences");
    // live bound of the next step: 1 + the last slot holding a beam (a score
    // that is not -inf) in any request
    int live = 0;
    HIP_TRY(gr::launch_live_bound(h->score[k], c.batch, c.beam_width, h->live_dev, st), "live bound");
    HIP_TRY(hipMemcpyAsync(&live, h->live_dev, sizeof(int), hipMemcpyDeviceToHost, st), "read live bound");
    HIP_TRY(hipStreamSynchronize(st), "set_state");
    h->t = step;
    h->live = std::max(1, live);
    h->can_rewind = false;
    h->last_stream = st;
    return GR_OK;
}

extern "C" void gr_beam_free(gr_beam* h) {
    if (!h) return;
    (void)hipDeviceSynchronize();
    beam_release(h);
    delete h;
}

// --------------------------------------------------------- observability

extern "C" gr_status gr_beam_timing_enable(gr_beam* h, int32_t enable) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    h->timing = enable != 0;
    return GR_OK;
}

extern "C" gr_status gr_beam_timing_get(gr_beam* h, double* row_ms, double* select_ms, int64_t* steps) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    harvest_timing(h, true);
    if (row_ms) *row_ms = h->row_ms;
    if (select_ms) *select_ms = h->sel_ms;
    if (steps) *steps = h->timed_steps;
    return GR_OK;
}

extern "C" gr_status gr_beam_timing_reset(gr_beam* h) {
    if (!h) return fail(GR_ERR_INVALID_ARG, "beam is NULL");
    harvest_timing(h, true);
    h->row_ms = h->sel_ms = 0.0;
    h->timed_steps = 0;
    return GR_OK;
}

extern "C" gr_status gr_beam_last_stats(gr_beam* h, gr_step_stats* out) {
    if (!h || !out) return fail(GR_ERR_INVALID_ARG, "NULL beam or out");
    // per request, written by the step's last kernel: summed here
    const size_t B = (size_t)h->cfg.batch;
    std::vector<unsigned long long> per(B * gr::kNumStats);
    HIP_TRY(hipMemcpyAsync(per.data(), h->stats, per.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost,
                           h->last_stream),
            "stats copy");
    HIP_TRY(hipStreamSynchronize(h->last_stream), "stats sync");
    unsigned long long s[gr::kNumStats] = {0, 0, 0, 0, 0, 0};
    for (size_t b = 0; b < B; ++b)
        for (int k = 0; k < gr::kNumStats; ++k) s[k] += per[b * gr::kNumStats + k];
    out->rows_read = (int64_t)s[0];
    out->candidates = (int64_t)s[1];
    out->survivors = (int64_t)s[2];
    out->slow_path_requests = (int64_t)s[3];
    out->rescanned_rows = (int64_t)s[4];
    out->fused_requests = (int64_t)s[5];
    return GR_OK;
}

// ----------------------------------------------------------------- probes

extern "C" gr_status gr_probe_read(const void* d_src, size_t bytes, uint32_t* d_sink, gr_stream stream) {
    if (!d_src || !d_sink || bytes % 16) return fail(GR_ERR_INVALID_ARG, "probe_read: bad arguments");
    HIP_TRY(gr::launch_probe_read(d_src, bytes / 16, d_sink, (hipStream_t)stream), "probe_read launch");
    return GR_OK;
}

extern "C" gr_status gr_probe_copy(void* d_dst, const void* d_src, size_t bytes, gr_stream stream) {
    if (!d_src || !d_dst || bytes % 16) return fail(GR_ERR_INVALID_ARG, "probe_copy: bad arguments");
    HIP_TRY(gr::launch_probe_copy(d_dst, d_src, bytes / 16, (hipStream_t)stream), "probe_copy launch");
    return GR_OK;
}

extern "C" gr_status gr_probe_draw_error(uint32_t r0, uint64_t count, double* d_out, gr_stream stream) {
    if (!d_out || count > (1ull << 32)) return fail(GR_ERR_INVALID_ARG, "probe_draw_error: bad arguments");
    HIP_TRY(gr::launch_probe_draw_error(r0, count, d_out, (hipStream_t)stream), "probe_draw_error launch");
    return GR_OK;
}

extern "C" double gr_draw_error_bound(void) { return (double)gr::draw_error_bound(); }

// ------------------------------------------------------------------- misc

extern "C" gr_status gr_memcpy(void* dst, const void* src, size_t bytes, gr_stream stream) {
    if (bytes == 0) return GR_OK;
    if (!dst || !src) return fail(GR_ERR_INVALID_ARG, "memcpy: NULL pointer");
    HIP_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, (hipStream_t)stream), "memcpy");
    return GR_OK;
}

extern "C" const char* gr_status_string(gr_status s) {
    switch (s) {
        case GR_OK: return "GR_OK";
        case GR_ERR_INVALID_ARG: return "GR_ERR_INVALID_ARG";
        case GR_ERR_BAD_TRIE: return "GR_ERR_BAD_TRIE";
        case GR_ERR_STATE: return "GR_ERR_STATE";
        case GR_ERR_OUT_OF_MEMORY: return "GR_ERR_OUT_OF_MEMORY";
        case GR_ERR_HIP: return "GR_ERR_HIP";
        case GR_ERR_UNSUPPORTED: return "GR_ERR_UNSUPPORTED";
        case GR_STATUS_MAX_ENUM: break;
    }
    return "GR_ERR_UNKNOWN";
}

extern "C" const char* gr_last_error(void) { return g_err.c_str(); }

extern "C" const char* gr_version(void) { return "gr 0.1.0 (gfx950)"; }
