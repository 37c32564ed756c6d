/*
 * oracle.c -- plain CPU oracle of one trie-constrained beam step.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Single thread, no SIMD
 * intrinsics, no blocking or fusion: each part follows the definition in
 * oracle.h in the order written there.  Build with -ffp-contract=off and
 * without -ffast-math so that every fp32 operation is one IEEE rounding.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    float k;         /* ranking score: c, or c + Gumbel noise when sampling */
    float c;         /* candidate score */
    int64_t flat;    /* parent slot * V + token id (tie-break key) */
    int32_t parent;
    int32_t token;   /* -1 for a finished beam carried forward */
    int32_t node;    /* child node at the next level, -1 if none */
    uint8_t fin;
} cand_t;

/* The strict total order: higher ranking score first, then lower flat
 * index.  Float comparison, so -0.0 and +0.0 compare equal. */
static int better(const cand_t* a, const cand_t* b) {
    if (a->k > b->k) return 1;
    if (a->k < b->k) return 0;
    return a->flat < b->flat;
}

/* Philox4x32-10 as defined by Salmon et al. (SC 2011): ten rounds of two
 * 32x32->64-bit multiplications by 0xD2511F53 and 0xCD9E8D57 whose high
 * halves are mixed with the other two counter words and the key, the key
 * advanced by the Weyl constants 0x9E3779B9 and 0xBB67AE85 between rounds. */
void gro_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        const uint32_t y1 = (uint32_t)p1;
        const uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        const uint32_t y3 = (uint32_t)p0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

float gro_length_penalty(int32_t len, float alpha) {
    return (float)pow((5.0 + (double)len) / 6.0, (double)alpha);
}

float gro_gumbel(uint64_t seed, int32_t request, int32_t step, int64_t flat) {
    const uint32_t ctr[4] = {(uint32_t)(flat / 4), (uint32_t)request, (uint32_t)step, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    gro_philox4x32_10(ctr, key, r);
    const double u = ((double)r[flat % 4] + 0.5) * 0x1p-32;
    return (float)(-log(-log(u)));
}

static int cmp_best_first(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (better(a, b)) return -1;
    if (better(b, a)) return 1;
    return 0;
}

static float logit_at(const void* row, int32_t dtype, int64_t v) {
    if (dtype == 1) {
        uint32_t bits = (uint32_t)((const uint16_t*)row)[v] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return f;
    }
    return ((const float*)row)[v];
}

/* A tempered logit fl32(x * inv_t) (inv_t = 1 when not sampling: exact). */
static float tlogit_at(const void* row, int32_t dtype, int64_t v, float inv_t) {
    return logit_at(row, dtype, v) * inv_t;
}

/* log-sum-exp of one (tempered) row: max first, then the fp64 sum of
 * exp(x - max) in token order, then one rounding of max + log(sum) to fp32.
 * A row whose max is -inf has no finite candidate; its normaliser is -inf. */
static float row_lse_t(const void* row, int32_t vocab, int32_t dtype, float inv_t) {
    float m = -INFINITY;
    for (int64_t v = 0; v < vocab; ++v) {
        float x = tlogit_at(row, dtype, v, inv_t);
        if (x > m) m = x;
    }
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int64_t v = 0; v < vocab; ++v) {
        double x = (double)tlogit_at(row, dtype, v, inv_t);
        s += exp(x - (double)m);
    }
    return (float)((double)m + log(s));
}

float gro_row_lse(const void* row, int32_t vocab, int32_t dtype) {
    return row_lse_t(row, vocab, dtype, 1.0f);
}

/* The same over a list of tokens (a candidate slice), in list order. */
static float slice_lse_t(const void* row, int32_t dtype, const int32_t* toks, int64_t n, float inv_t) {
    float m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        float x = tlogit_at(row, dtype, toks[i], inv_t);
        if (x > m) m = x;
    }
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += exp((double)tlogit_at(row, dtype, toks[i], inv_t) - (double)m);
    return (float)((double)m + log(s));
}

/* Bounded selection of the K best: a binary heap whose root is the worst
 * kept candidate (textbook "keep the K largest" heap). */
typedef struct {
    cand_t* h;
    int64_t n, cap;
} heap_t;

static void sift_down(heap_t* q, int64_t i) {
    for (;;) {
        int64_t l = 2 * i + 1, r = l + 1, w = i;
        /* the worst of i, l, r goes to the top */
        if (l < q->n && better(&q->h[w], &q->h[l])) w = l;
        if (r < q->n && better(&q->h[w], &q->h[r])) w = r;
        if (w == i) return;
        cand_t t = q->h[i]; q->h[i] = q->h[w]; q->h[w] = t;
        i = w;
    }
}

static void sift_up(heap_t* q, int64_t i) {
    while (i > 0) {
        int64_t p = (i - 1) / 2;
        if (!better(&q->h[p], &q->h[i])) return;  /* parent already worse */
        cand_t t = q->h[i]; q->h[i] = q->h[p]; q->h[p] = t;
        i = p;
    }
}

static int is_banned(const gro_step_args* a, int32_t v) {
    for (int32_t i = 0; i < a->n_banned; ++i)
        if (a->banned[i] == v) return 1;
    return 0;
}

static void offer(heap_t* q, const cand_t* c) {
    if (q->n < q->cap) {
        q->h[q->n] = *c;
        sift_up(q, q->n);
        q->n++;
    } else if (better(c, &q->h[0])) {
        q->h[0] = *c;
        sift_down(q, 0);
    }
}

int gro_step(const gro_step_args* a, const void* logits,
             const float* score, const int32_t* node, const uint8_t* fin,
             const int32_t* seq,
             float* score_out, int32_t* node_out, uint8_t* fin_out, int32_t* seq_out,
             int32_t* parent_out, int32_t* token_out, float* lse_out,
             int64_t* n_candidates) {
    if (!a || a->beam < 1 || a->vocab < 1 || a->row_stride < a->vocab) return GRO_EINVAL;
    if (a->dtype != 0 && a->dtype != 1) return GRO_EINVAL;
    if (a->max_steps < 1 || a->step < 0) return GRO_EINVAL;
    if (a->step >= a->max_steps) return GRO_ESTATE;
    if (a->eos >= a->vocab) return GRO_EINVAL;
    const int constrained = a->offsets != NULL;
    if (constrained && (!a->tokens || !a->children || a->num_nodes < 1)) return GRO_EINVAL;
    if (!(a->temperature >= 0.0f) || isinf(a->temperature)) return GRO_EINVAL;
    if (!isfinite(a->alpha) || a->n_banned < 0 || (a->n_banned > 0 && !a->banned)) return GRO_EINVAL;
    if (a->norm_mode < 0 || a->norm_mode > 3) return GRO_EINVAL;
    if (a->norm_mode == 1 && !(0 <= a->norm_lo && a->norm_lo < a->norm_hi && a->norm_hi <= a->vocab))
        return GRO_EINVAL;
    const int32_t lo = a->norm_mode == 1 ? a->norm_lo : 0, hi = a->norm_mode == 1 ? a->norm_hi : a->vocab;
    const int sampling = a->temperature > 0.0f;
    const float inv_t = sampling ? 1.0f / a->temperature : 1.0f;
    /* ranking score of a candidate of a hypothesis of length len_:
     * fl32(c / pen(len)), plus its Gumbel draw when sampling */
    #define RANK(c_, flat_, len_)                                                       \
        (sampling ? ((c_) / gro_length_penalty((len_), a->alpha)) +                      \
                        gro_gumbel(a->seed, a->request, a->step, (flat_))                \
                  : (c_) / gro_length_penalty((len_), a->alpha))
    /* a token that may not be emitted at this step (or lies outside the range) */
    #define MASKED(v_)                                                                  \
        (is_banned(a, (v_)) || ((v_) == a->eos && t + 1 < a->min_length) ||            \
         (v_) < lo || (v_) >= hi)

    const int32_t K = a->beam, V = a->vocab, T = a->max_steps, t = a->step;
    const size_t esz = a->dtype == 1 ? 2 : 4;

    heap_t q;
    q.cap = K;
    q.n = 0;
    q.h = (cand_t*)malloc(sizeof(cand_t) * (size_t)K);
    if (!q.h) return GRO_ENOMEM;

    int64_t ncand = 0;
    for (int32_t j = 0; j < K; ++j) {
        lse_out[j] = NAN;
        const float S = score[j];
        if (S == -INFINITY) continue;                 /* empty slot */
        if (fin[j]) {                                 /* finished: carried forward */
            if (a->eos < 0) { free(q.h); return GRO_ESTATE; }
            const int64_t flat = (int64_t)j * V + a->eos;
            int32_t len = 0;  /* the carried hypothesis' own length */
            for (int32_t s = 0; s < T; ++s) len += seq[(size_t)j * T + s] != -1;
            cand_t c = {RANK(S, flat, len), S, flat, j, -1, -1, 1};
            offer(&q, &c);
            ++ncand;
            continue;
        }
        const void* row = (const char*)logits + (size_t)j * (size_t)a->row_stride * esz;
        float lse;
        if (a->norm_mode == 3) {            /* log-probabilities already */
            lse = 0.0f;
        } else if (a->norm_mode == 1) {     /* the token range only */
            lse = row_lse_t((const char*)row + (size_t)lo * esz, hi - lo, a->dtype, inv_t);
        } else if (a->norm_mode == 2 && constrained) {   /* the node's children only */
            const int32_t n = node[j];
            if (n < 0 || n >= a->num_nodes) { free(q.h); return GRO_ESTATE; }
            lse = slice_lse_t(row, a->dtype, a->tokens + a->offsets[n], a->offsets[n + 1] - a->offsets[n], inv_t);
        } else {
            lse = row_lse_t(row, V, a->dtype, inv_t);
        }
        lse_out[j] = lse;
        if (lse == -INFINITY) continue;               /* no finite logit */
        if (constrained) {
            const int32_t n = node[j];
            if (n < 0 || n >= a->num_nodes) { free(q.h); return GRO_ESTATE; }
            for (int64_t e = a->offsets[n]; e < a->offsets[n + 1]; ++e) {
                const int32_t v = a->tokens[e];
                if (MASKED(v)) continue;
                const float lp = tlogit_at(row, a->dtype, v, inv_t) - lse;
                const float c = S + lp;
                if (c == -INFINITY) continue;
                const int64_t flat = (int64_t)j * V + v;
                cand_t cd = {RANK(c, flat, t + 1), c, flat, j, v, a->children[e], 0};
                offer(&q, &cd);
                ++ncand;
            }
        } else {
            for (int32_t v = 0; v < V; ++v) {
                if (MASKED(v)) continue;
                const float lp = tlogit_at(row, a->dtype, v, inv_t) - lse;
                const float c = S + lp;
                if (c == -INFINITY) continue;
                const int64_t flat = (int64_t)j * V + v;
                cand_t cd = {RANK(c, flat, t + 1), c, flat, j, v, -1, (uint8_t)(v == a->eos)};
                offer(&q, &cd);
                ++ncand;
            }
        }
    }

    qsort(q.h, (size_t)q.n, sizeof(cand_t), cmp_best_first);

    for (int32_t i = 0; i < K; ++i) {
        int32_t* so = seq_out + (size_t)i * T;
        if (i < q.n) {
            const cand_t* c = &q.h[i];
            score_out[i] = c->c;
            node_out[i] = c->node;
            fin_out[i] = c->fin;
            parent_out[i] = c->parent;
            token_out[i] = c->token;
            const int32_t* sp = seq + (size_t)c->parent * T;
            for (int32_t s = 0; s < T; ++s) so[s] = s < t ? sp[s] : -1;
            so[t] = c->token;
        } else {
            score_out[i] = -INFINITY;
            node_out[i] = -1;
            fin_out[i] = 0;
            parent_out[i] = -1;
            token_out[i] = -1;
            for (int32_t s = 0; s < T; ++s) so[s] = -1;
        }
    }
    if (n_candidates) *n_candidates = ncand;
    free(q.h);
    return GRO_OK;
    #undef RANK
    #undef MASKED
}

/* ------------------------------------------------------------- backward */

int gro_backward(int32_t K, int32_t T, int32_t steps, const int32_t* parents, const int32_t* tokens,
                 const float* score_final, const int32_t* seq_final, const float* grad_final,
                 float alpha, int32_t* path_slot, int32_t* path_token, float* weight) {
    if (K < 1 || T < 1 || steps < 0 || steps > T || !isfinite(alpha)) return GRO_EINVAL;
    for (int32_t k = 0; k < K; ++k) {
        for (int32_t t = 0; t < steps; ++t) {
            path_slot[(size_t)t * K + k] = -1;
            path_token[(size_t)t * K + k] = -1;
        }
        weight[k] = 0.0f;
        if (score_final[k] == -INFINITY) continue;   /* empty final slot */
        int32_t i = k;
        for (int32_t t = steps - 1; t >= 0; --t) {
            if (i < 0) return GRO_ESTATE;
            const int32_t p = parents[(size_t)t * K + i];
            path_slot[(size_t)t * K + k] = p;
            path_token[(size_t)t * K + k] = tokens[(size_t)t * K + i];
            i = p;
        }
        int32_t len = 0;
        for (int32_t q = 0; q < T; ++q) len += seq_final[(size_t)k * T + q] != -1;
        weight[k] = grad_final[k] / gro_length_penalty(len, alpha);
    }
    return GRO_OK;
}

int gro_backward_scatter(int32_t K, int32_t V, const int32_t* path_slot_t, const int32_t* path_token_t,
                         const float* weight, float* grad) {
    if (K < 1 || V < 1) return GRO_EINVAL;
    for (int32_t k = 0; k < K; ++k) {
        const int32_t p = path_slot_t[k], v = path_token_t[k];
        if (v < 0) continue;
        if (p < 0 || p >= K || v >= V) return GRO_EINVAL;
        int first = 1;   /* only the first beam through (p, v) writes */
        for (int32_t q = 0; q < k; ++q)
            if (path_slot_t[q] == p && path_token_t[q] == v) { first = 0; break; }
        if (!first) continue;
        float acc = 0.0f;
        for (int32_t q = k; q < K; ++q)
            if (path_slot_t[q] == p && path_token_t[q] == v) acc += weight[q];
        grad[(size_t)p * V + v] += acc;
    }
    return GRO_OK;
}
