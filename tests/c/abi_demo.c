/*
 * abi_demo.c -- the library's C ABI used from plain C, with no Python and no
 * torch: a small SID trie is built, a three-step constrained search runs on
 * device logits that the HIP runtime allocates, and every step's new state is
 * read back and checked against the CPU oracle of the same step.
 *
 * Exit status: 0 = every check passed; 77 = no GPU (the host-only part --
 * status strings, version, trie validation -- was checked); anything else =
 * a failure (printed).
 *
 * The catalog: 3 levels, codebook 4, level L uses tokens 4L .. 4L+3 (V = 12);
 * the SIDs are the codes (a, b, c) with (a + 2b + 3c) mod 5 != 0, so nodes
 * have different fan-outs.  Logits come from a fixed linear congruential
 * generator.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gr.h"
#include "oracle.h"

enum { D = 3, CB = 4, V = 12, B = 2, K = 6, T = 3 };

#define CHECK(cond, ...)                              \
    do {                                              \
        if (!(cond)) {                                \
            fprintf(stderr, "FAIL: " __VA_ARGS__);    \
            fprintf(stderr, "\n");                    \
            exit(1);                                  \
        }                                             \
    } while (0)

#define GR(call)                                                                        \
    do {                                                                                \
        gr_status st_ = (call);                                                         \
        CHECK(st_ == GR_OK, "%s -> %s (%s)", #call, gr_status_string(st_), gr_last_error()); \
    } while (0)

#define HIP(call)                                                             \
    do {                                                                      \
        hipError_t e_ = (call);                                               \
        CHECK(e_ == hipSuccess, "%s -> %s", #call, hipGetErrorString(e_));    \
    } while (0)

/* The per-level CSR of the catalog.  Node ids at every level below the root
 * run backwards through the sorted prefixes: node n of level L >= 1 is the
 * (num_nodes[L] - 1 - n)-th distinct L-code prefix in sorted order, so no
 * child id equals its edge's ordinal by construction and the search must
 * follow the child ids it is given. */
static int64_t num_nodes[D + 1];
static int64_t off_store[D][CB * CB * CB + 1];
static int32_t tok_store[D][CB * CB * CB];
static int32_t child_store[D][CB * CB * CB];

static int in_catalog(int a, int b, int c) { return (a + 2 * b + 3 * c) % 5 != 0; }

/* index of a prefix among the level's prefixes (each level enumerates its
 * prefixes in sorted order); -1 if no SID extends it */
static int prefix_index(int len, const int* code) {
    int idx = 0;
    for (int p = 0; p < CB * CB * CB; ++p) {
        const int pc[3] = {p / (CB * CB), (p / CB) % CB, p % CB};
        if (!in_catalog(pc[0], pc[1], pc[2])) continue;
        /* is p the first SID of its len-prefix? then that prefix counts once */
        int first = 1;
        for (int q = 0; q < p && first; ++q) {
            const int qc[3] = {q / (CB * CB), (q / CB) % CB, q % CB};
            if (!in_catalog(qc[0], qc[1], qc[2])) continue;
            int same = 1;
            for (int i = 0; i < len; ++i) same &= qc[i] == pc[i];
            if (same) first = 0;
        }
        if (!first) continue;
        int same = 1;
        for (int i = 0; i < len; ++i) same &= pc[i] == code[i];
        if (same) return idx;
        ++idx;
    }
    return -1;
}

/* the p-th code tuple of length L in lexicographic order */
static void tuple(int L, int p, int* code) {
    for (int i = L - 1; i >= 0; --i) {
        code[i] = p % CB;
        p /= CB;
    }
}

static int tuples(int L) {
    int n = 1;
    for (int i = 0; i < L; ++i) n *= CB;
    return n;
}

/* the id of a prefix's node (-1 if no SID extends it); needs num_nodes */
static int node_id(int len, const int* code) {
    const int i = prefix_index(len, code);
    return (i < 0 || len == 0) ? i : (int)num_nodes[len] - 1 - i;
}

static void build_catalog(void) {
    int code[3] = {0, 0, 0};
    for (int L = 0; L <= D; ++L) {
        num_nodes[L] = 0;
        for (int p = 0; p < tuples(L); ++p) {
            tuple(L, p, code);
            if (prefix_index(L, code) >= 0) ++num_nodes[L];
        }
    }
    for (int L = 0; L < D; ++L) {
        /* fan-out of each node id, then the offsets in id order */
        int64_t fan[CB * CB * CB];
        memset(fan, 0, sizeof fan);
        for (int p = 0; p < tuples(L); ++p) {
            tuple(L, p, code);
            const int n = node_id(L, code);
            if (n < 0) continue;
            for (int c = 0; c < CB; ++c) {
                code[L] = c;
                fan[n] += node_id(L + 1, code) >= 0 ? 1 : 0;
            }
        }
        off_store[L][0] = 0;
        for (int n = 0; n < num_nodes[L]; ++n) off_store[L][n + 1] = off_store[L][n] + fan[n];
        for (int p = 0; p < tuples(L); ++p) {
            tuple(L, p, code);
            const int n = node_id(L, code);
            if (n < 0) continue;
            int64_t e = off_store[L][n];
            for (int c = 0; c < CB; ++c) {  /* children in token order */
                code[L] = c;
                const int child = node_id(L + 1, code);
                if (child < 0) continue;
                tok_store[L][e] = CB * L + c;
                child_store[L][e] = child;
                ++e;
            }
        }
    }
}

static uint64_t lcg = 0x2545F4914F6CDD1DULL;
static float next_logit(void) {
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((double)(lcg >> 40) / (double)(1ULL << 24) * 6.0 - 3.0);
}

int main(void) {
    /* host-only part */
    CHECK(strcmp(gr_status_string(GR_OK), "GR_OK") == 0, "status string");
    CHECK(strstr(gr_version(), "gfx950") != NULL, "version names the target");
    build_catalog();
    const int64_t* offs[D];
    const int32_t* toks[D];
    const int32_t* chs[D];
    for (int L = 0; L < D; ++L) {
        offs[L] = off_store[L];
        toks[L] = tok_store[L];
        chs[L] = child_store[L];
    }
    GR(gr_trie_validate(D, V, num_nodes, offs, toks, chs));
    int renumbered = 0;  /* child ids that differ from their edge ordinal */
    for (int L = 0; L < D; ++L)
        for (int64_t e = 0; e < off_store[L][num_nodes[L]]; ++e) renumbered += child_store[L][e] != e;
    CHECK(renumbered > 0, "the node numbering must differ from the edge ordinals");
    printf("catalog: %lld SIDs, nodes per level %lld %lld %lld\n", (long long)num_nodes[D],
           (long long)num_nodes[0], (long long)num_nodes[1], (long long)num_nodes[2]);

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
        printf("no GPU: host-only checks passed\n");
        return 77;
    }

    /* the search on the GPU */
    gr_trie* trie = NULL;
    GR(gr_trie_build(D, V, num_nodes, offs, toks, chs, NULL, &trie));
    gr_beam_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.batch = B;
    cfg.beam_width = K;
    cfg.vocab = V;
    cfg.max_steps = T;
    cfg.eos_token = -1;
    cfg.logits_dtype = GR_F32;
    gr_beam* beam = NULL;
    GR(gr_beam_init(&cfg, trie, NULL, &beam));
    float* d_logits = NULL;
    HIP(hipMalloc((void**)&d_logits, sizeof(float) * B * K * V));

    /* the oracle's own state, per request */
    float score[B][K];
    int32_t node[B][K];
    uint8_t fin[B][K];
    int32_t seq[B][K * T];
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < K; ++j) {
            score[b][j] = j == 0 ? 0.0f : -INFINITY;
            node[b][j] = j == 0 ? 0 : -1;
            fin[b][j] = 0;
            for (int q = 0; q < T; ++q) seq[b][j * T + q] = -1;
        }

    static float logits[B][K][V];
    for (int t = 0; t < T; ++t) {
        for (int b = 0; b < B; ++b)
            for (int j = 0; j < K; ++j)
                for (int v = 0; v < V; ++v) logits[b][j][v] = next_logit();
        HIP(hipMemcpy(d_logits, logits, sizeof logits, hipMemcpyHostToDevice));
        GR(gr_beam_step(beam, d_logits, NULL));
        HIP(hipDeviceSynchronize());

        gr_beam_view view;
        GR(gr_beam_view_get(beam, &view));
        CHECK(view.step == t + 1, "step counter %d after step %d", view.step, t);
        float g_score[B][K];
        int32_t g_node[B][K], g_parent[B][K], g_token[B][K], g_seq[B][K * T];
        HIP(hipMemcpy(g_score, view.scores, sizeof g_score, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g_node, view.nodes, sizeof g_node, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g_parent, view.parents + (size_t)t * B * K, sizeof g_parent, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g_token, view.tokens + (size_t)t * B * K, sizeof g_token, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g_seq, view.sequences, sizeof g_seq, hipMemcpyDeviceToHost));

        for (int b = 0; b < B; ++b) {
            gro_step_args a;
            memset(&a, 0, sizeof a);
            a.beam = K;
            a.vocab = V;
            a.eos = -1;
            a.dtype = 0;
            a.row_stride = V;
            a.max_steps = T;
            a.step = t;
            a.offsets = off_store[t];
            a.num_nodes = num_nodes[t];
            a.tokens = tok_store[t];
            a.children = child_store[t];
            a.request = b;
            float s2[K], lse[K];
            int32_t n2[K], q2[K * T], p2[K], k2[K];
            uint8_t f2[K];
            int64_t ncand = 0;
            CHECK(gro_step(&a, logits[b], score[b], node[b], fin[b], seq[b], s2, n2, f2, q2, p2, k2, lse,
                           &ncand) == GRO_OK, "oracle step");
            for (int j = 0; j < K; ++j) {
                CHECK(p2[j] == g_parent[b][j] && k2[j] == g_token[b][j] && n2[j] == g_node[b][j],
                      "step %d request %d slot %d: GPU (parent %d, token %d, node %d), oracle (%d, %d, %d)", t, b,
                      j, g_parent[b][j], g_token[b][j], g_node[b][j], p2[j], k2[j], n2[j]);
                CHECK(isinf(s2[j]) ? s2[j] == g_score[b][j] : fabsf(s2[j] - g_score[b][j]) <= 1e-4f,
                      "step %d request %d slot %d: score %g vs oracle %g", t, b, j, g_score[b][j], s2[j]);
                for (int q = 0; q < T; ++q)
                    CHECK(q2[j * T + q] == g_seq[b][j * T + q], "step %d request %d slot %d: sequence", t, b, j);
            }
            memcpy(score[b], s2, sizeof s2);
            memcpy(node[b], n2, sizeof n2);
            memcpy(fin[b], f2, sizeof f2);
            memcpy(seq[b], q2, sizeof q2);
        }
        printf("step %d: %d requests x %d slots equal to the oracle\n", t, B, K);
    }
    HIP(hipFree(d_logits));
    gr_beam_free(beam);
    gr_trie_free(trie);
    printf("ok: C ABI search matches the oracle\n");
    return 0;
}
