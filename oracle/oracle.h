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
 * Readings where the pages leave a step open are listed in the design notes:
 * full-row normalisation, one live slot at start, flat = parent slot * V +
 * global token id, EOS carried with token -1 and no length penalty.
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

#ifdef __cplusplus
}
#endif
#endif
