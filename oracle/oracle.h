/*
 * oracle.h -- plain CPU oracle of one trie-constrained beam step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously correct reference
 * that the GPU library is checked against.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load or call it; the GPU
 * library never includes, links or calls anything here, and nothing here
 * includes or calls the GPU library.
 *
 * What one step computes (FlashRec README, "Decoding" and "Features": every
 * continuation is restricted to valid SID edges of a CSR trie; beamgrad
 * README, "How it works" and "Features": every live beam proposes its tokens,
 * cumulative log-probabilities rank the candidates, the K best survive under a
 * strict total order, beams that emitted EOS are carried forward unchanged and
 * keep competing, sequences are -1 after they end):
 *
 *   for one request, for each slot j of the previous step:
 *     empty    (score == -inf):       no candidate, row not read;
 *     finished (fin[j], eos >= 0):    one candidate (score[j], flat j*V+eos,
 *                                     token -1, node -1, finished);
 *     live:    m    = max_v x[j][v]                       (fp32 values)
 *              s    = sum_v exp((double)x[j][v] - m)     (fp64, v order)
 *              lse  = (float)(m + log(s))                (one rounding)
 *              for each valid token v (trie children of node[j] at level
 *              `step`, or all of [0,V) when unconstrained):
 *                lp = x[j][v] - lse;   c = score[j] + lp (fp32, RNE, this order)
 *                candidate (c, flat j*V+v, parent j, token v,
 *                           node = child node or -1, finished = (v == eos))
 *   candidates with c == -inf are dropped; the rest are ordered by
 *     a before b  <=>  a.c > b.c  or  (a.c == b.c and a.flat < b.flat)
 *   and the first min(K, #candidates) fill slots 0.. best first; the rest of
 *   the slots become empty (score -inf, node/parent/token -1, sequence -1).
 *
 * Sampling, temperature T > 0 (FlashRec README, "Serving", the API item:
 * deterministic top-k at temperature 0, Gumbel top-k without replacement
 * above it):
 *   each live row is tempered, xt[v] = fl32(x[j][v] * fl32(1/T)), and m, s,
 *   lse and lp above are taken over xt;
 *   every candidate draws one standard Gumbel variate
 *     g = (float)(-log(-log(u))),  u = (r + 0.5) * 2^-32      (fp64)
 *   where r is output word (flat mod 4) of Philox4x32-10 (Salmon, Moraes,
 *   Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011)
 *   at counter (flat div 4, request, step, 0) and key (seed mod 2^32,
 *   seed div 2^32); a carried beam draws at its flat j*V+eos;
 *   candidates are ordered by the perturbed score k = fl32(c + g) (then lower
 *   flat), the first min(K, #candidates) fill the slots in that order, and
 *   each slot keeps its unperturbed score c.
 *   At T = 0 nothing is tempered or drawn: k = c.
 *
 * Length penalty, minimum length and banned tokens (beamgrad README,
 * "Features": GNMT length penalty, minimum length, banned tokens; "How it
 * works": the cumulative log-probability is ranked by
 * raw / ((5 + length) / 6) ** alpha):
 *   a banned token is never a candidate; EOS is not a candidate while the
 *   hypothesis would be shorter than min_length (step + 1 < min_length);
 *   length = number of tokens of the hypothesis including EOS: step + 1 for a
 *   live beam's candidate, the count of its non-(-1) tokens for a carried
 *   beam;  pen(len) = (float)pow((5 + len) / 6, alpha)  (fp64, one rounding);
 *   the ranking score becomes k = fl32(c / pen(len)) before any Gumbel draw,
 *   k = fl32(fl32(c / pen(len)) + g) when sampling; slots keep the raw c.
 *   alpha = 0, min_length <= 1 and no banned token change nothing.
 *
 * Normalisation variants (the default normalises over the full row):
 *   RANGE [lo, hi) (FlashRec README, "Decoding": lm_head is evaluated only
 *     over the SID token range): m, s and lse are taken over the tempered
 *     logits of tokens lo <= v < hi only, in token order; a token outside
 *     the range is never a candidate;
 *   SLICE (Qwen-2.5-1B-RLCD-Fast model card, "Sub-Vocabulary Logit
 *     Slicing": probabilities normalised over the candidate slice only):
 *     m, s and lse are taken over the row's own candidates -- its trie
 *     node's children in edge order, or every token when unconstrained --
 *     before any mask (banned tokens and the minimum length remove
 *     candidates from the ranking, not from the slice);
 *   NONE (beamgrad README, the C API example: the decoder takes log_probs
 *     [T, K, V]): the values are log-probabilities already, lse = 0, so
 *     lp = x (tempered when sampling) and c = score[j] + lp.
 *
 * Surrogate backward (beamgrad README, "How it works": backward holds the
 * selection fixed; the gradient of final beam k's score with respect to
 * log_probs[t, p, v] is 1 / penalty(length_k) on k's path and zero
 * elsewhere; "Features": each step gets only its own path gradient, never a
 * dense [B, T, K, V] array): see gro_backward and gro_backward_scatter.
 *
 * Readings where the pages leave a step open are listed in the design notes:
 * full-row normalisation, one live slot at start, flat = parent slot * V +
 * global token id, EOS carried with token -1 and no length penalty, and the
 * sampling rule above (per-step draws, unperturbed scores kept).
 */
#ifndef GR_ORACLE_H
#define GR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t beam;        /* K >= 1 */
    int32_t vocab;       /* V >= 1 */
    int32_t eos;         /* EOS token id, -1 = none */
    int32_t dtype;       /* 0 = fp32 logits, 1 = bf16 bit patterns (uint16) */
    int64_t row_stride;  /* elements between consecutive rows, >= vocab */
    int32_t max_steps;   /* T, length of each sequence row */
    int32_t step;        /* t, 0-based, < max_steps */
    /* trie level `step` (CSR); offsets == NULL selects unconstrained search */
    const int64_t* offsets;   /* [num_nodes + 1] */
    int64_t num_nodes;
    const int32_t* tokens;    /* [offsets[num_nodes]] */
    const int32_t* children;  /* [offsets[num_nodes]] */
    /* sampling: temperature 0 = deterministic top-K */
    float temperature;        /* T >= 0, finite */
    int32_t request;          /* request index b (part of the noise counter) */
    uint64_t seed;            /* Philox key */
    /* length penalty, minimum length, banned tokens */
    float alpha;              /* GNMT exponent, finite (0 = none) */
    int32_t min_length;       /* EOS allowed once the hypothesis has this many tokens */
    const int32_t* banned;    /* [n_banned] token ids, any order; NULL when n_banned = 0 */
    int32_t n_banned;
    /* normalisation: 0 = full row, 1 = RANGE [norm_lo, norm_hi), 2 = SLICE, 3 = NONE */
    int32_t norm_mode;
    int32_t norm_lo, norm_hi;
} gro_step_args;

/* Error codes (negative) */
#define GRO_OK 0
#define GRO_EINVAL (-1)
#define GRO_ENOMEM (-2)
#define GRO_ESTATE (-3)

/*
 * One step of one request.  All pointers are host memory.
 *   logits      K rows of V values, row j at logits + j*row_stride elements
 *   score,node,fin           [K]   state before the step
 *   seq                      [K*T] tokens of each slot, -1 padded
 *   score_out,node_out,fin_out,seq_out   same shapes, state after the step
 *   parent_out, token_out    [K]   backpointer and emitted token per slot
 *   lse_out                  [K]   the row normaliser of each live slot,
 *                                  NaN for slots whose row is not read
 *   n_candidates             number of candidates before selection
 * Returns GRO_OK or a negative error code.
 */
int gro_step(const gro_step_args* a, const void* logits,
             const float* score, const int32_t* node, const uint8_t* fin,
             const int32_t* seq,
             float* score_out, int32_t* node_out, uint8_t* fin_out, int32_t* seq_out,
             int32_t* parent_out, int32_t* token_out, float* lse_out,
             int64_t* n_candidates);

/* The row normaliser alone: (float)(max + log(sum exp(x - max))) in fp64. */
float gro_row_lse(const void* row, int32_t vocab, int32_t dtype);

/* Philox4x32-10 of one counter block under one key (out may alias ctr). */
void gro_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The Gumbel variate of candidate `flat` of `request` at `step` (see above). */
float gro_gumbel(uint64_t seed, int32_t request, int32_t step, int64_t flat);

/* The length penalty pen(len) = (float)pow((5 + len) / 6, alpha). */
float gro_length_penalty(int32_t len, float alpha);

/*
 * Paths of the final beams of one request after `steps` steps, and their
 * weights.  parents, tokens: [steps * K] history (row t = step t: the slot
 * each new slot came from, the token it emitted, -1 for a carried beam's
 * token and for empty slots); score_final [K], seq_final [K * T] the state
 * after the last step; grad_final [K] the upstream gradient of each final
 * beam's ranked score.  For every final slot k with a finite score, walking
 * back from i = k at t = steps-1 down to 0: p = parents[t][i], v =
 * tokens[t][i], path_slot[t*K + k] = p, path_token[t*K + k] = v (-1 where
 * the beam was carried: that step adds no log-probability), i = p.
 * weight[k] = fl32(grad_final[k] / pen(len_k)), len_k = the tokens of
 * seq_final[k] that are not -1.  Empty final slots get path -1, weight 0.
 * Returns GRO_OK, or GRO_ESTATE if a finite beam's walk reaches slot -1.
 */
int gro_backward(int32_t K, int32_t T, int32_t steps, const int32_t* parents, const int32_t* tokens,
                 const float* score_final, const int32_t* seq_final, const float* grad_final,
                 float alpha, int32_t* path_slot, int32_t* path_token, float* weight);

/*
 * The gradient with respect to log_probs of step t of sum_k grad_final[k] *
 * (ranked final score of k), added to grad [K * V] (row p = slot p of step
 * t): for each distinct (p, v) with v >= 0 on some final beam's path at
 * step t, acc = the fp32 sum, from 0 in ascending k, of weight[k] over the
 * beams k whose path passes (p, v); then grad[p*V + v] += acc (one add).
 * path_slot_t, path_token_t: row t of gro_backward's outputs [K].
 */
int gro_backward_scatter(int32_t K, int32_t V, const int32_t* path_slot_t, const int32_t* path_token_t,
                         const float* weight, float* grad);

#ifdef __cplusplus
}
#endif
#endif
