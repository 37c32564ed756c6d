/*
 * gr.h -- one step of wide, trie-constrained beam search on AMD gfx950.
 *
 * What a step computes (FlashRec README, "Decoding": a fused kernel over a
 * dense or CSR-sparse trie restricts decoding to the catalog of valid
 * semantic IDs, so an illegal SID is never a candidate; "API": deterministic
 * top-k at temperature 0; beamgrad README, "How it works" and "Features":
 * every live beam proposes its tokens, cumulative log-probabilities rank
 * them, the K best survive under a strict total order, beams that emitted EOS
 * are carried forward unchanged and keep competing, sequences are -1 after
 * they end):
 *
 *   for every request b and every slot j of the previous step
 *     empty slot (score -inf): nothing;
 *     finished slot: one candidate, its score unchanged, token -1;
 *     live slot: lse_j = log sum_v exp(x[b][j][v]) over the full row of V
 *       logits; for each valid token v (the children of the slot's trie node
 *       at the current level, or every v when there is no trie)
 *       c = score_j + (x[b][j][v] - lse_j)          (fp32, in this order)
 *   the min(K, #candidates) best candidates of each request, ordered by
 *   higher c first and then lower flat index j*V + v, become slots 0.. of the
 *   next step; their parent slot, token, score, next trie node and finished
 *   flag are written; remaining slots become empty.
 *
 * The first step starts from one live slot per request (score +0, the trie
 * root); all other slots are empty.
 *
 * Conventions
 *   - Every call returns gr_status; out-parameters are written only on
 *     GR_OK; gr_last_error() gives a message for the calling thread.
 *   - Argument and trie errors are detected on the host before anything is
 *     enqueued.  Errors of the HIP runtime map to GR_ERR_HIP.  Faults of an
 *     already-enqueued kernel surface at the caller's next synchronisation.
 *   - Streams are hipStream_t values passed as void* (NULL = the null
 *     stream).  Work is enqueued on the given stream; no call except the
 *     build/init/free calls synchronises.
 *   - Device pointers are plain addresses from hipMalloc (or any allocator
 *     on the same device, e.g. PyTorch's).
 *   - Ownership: a handle owns every device buffer it allocates (only at
 *     build or init time); the caller owns logits and streams.  A gr_trie is
 *     immutable after build and may be shared by several gr_beam handles
 *     (free it after them).  A gr_beam must not be used from two threads at
 *     once, nor stepped on two streams concurrently.
 *   - Limits: K * V < 2^32; 1 <= K <= 4096; V <= 2^30.
 */
#ifndef GR_H
#define GR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GR_OK = 0,
    GR_ERR_INVALID_ARG = 1,   /* a NULL pointer, a size out of range */
    GR_ERR_BAD_TRIE = 2,      /* the CSR arrays violate the rules of gr_trie_validate */
    GR_ERR_STATE = 3,         /* stepping past max_steps or past the trie depth */
    GR_ERR_OUT_OF_MEMORY = 4, /* a device or host allocation failed */
    GR_ERR_HIP = 5,           /* the HIP runtime reported an error */
    GR_ERR_UNSUPPORTED = 6,   /* a valid request this build does not handle */
    GR_STATUS_MAX_ENUM = 0x7FFFFFFF  /* not a status: makes every int32 value >= 0 a
                                        valid gr_status (gr_status_string of an unknown
                                        code is then defined behaviour) */
} gr_status;

typedef enum { GR_F32 = 0, GR_BF16 = 1 } gr_dtype;

typedef void* gr_stream;               /* a hipStream_t */
typedef struct gr_trie gr_trie;        /* opaque */
typedef struct gr_beam gr_beam;        /* opaque */

/* ------------------------------------------------------------------ trie */

/*
 * Check a per-level CSR trie on the host (no device is touched).
 * (FlashRec README, "Decoding": the CSR-sparse trie of valid SIDs.)
 *
 *   depth          D >= 1 levels (steps of a constrained search)
 *   vocab          V, every child token lies in [0, V)
 *   num_nodes      [D+1] nodes per level; num_nodes[0] == 1 (the root,
 *                  node 0); num_nodes[D] = number of leaves (catalog size)
 *   node_offsets   [D] host arrays; level L has num_nodes[L]+1 int64
 *                  entries, first 0, non-decreasing; the edges of node n are
 *                  node_offsets[L][n] .. node_offsets[L][n+1]-1
 *   child_tokens   [D] host arrays of node_offsets[L][num_nodes[L]] int32
 *                  token ids, strictly increasing within each node
 *   child_nodes    [D] host arrays, same length, int32 node ids at level
 *                  L+1 in [0, num_nodes[L+1]); at level D-1 these are leaf
 *                  ids (e.g. catalog rows)
 * Returns GR_OK, GR_ERR_INVALID_ARG (NULL pointers, D < 1, V < 1) or
 * GR_ERR_BAD_TRIE (with the first violation in gr_last_error()).
 */
gr_status gr_trie_validate(int32_t depth, int32_t vocab, const int64_t* num_nodes,
                           const int64_t* const* node_offsets,
                           const int32_t* const* child_tokens,
                           const int32_t* const* child_nodes);

/*
 * Validate (as above), then copy the trie to device memory owned by the new
 * handle.  The copies are enqueued on `stream` and complete before the call
 * returns, so the host arrays may be released afterwards.
 */
gr_status gr_trie_build(int32_t depth, int32_t vocab, const int64_t* num_nodes,
                        const int64_t* const* node_offsets,
                        const int32_t* const* child_tokens,
                        const int32_t* const* child_nodes,
                        gr_stream stream, gr_trie** out);

/* Shape of a built trie: depth, vocab, nodes per level ([depth+1], may be
 * NULL) and the largest fan-out of each level ([depth], may be NULL). */
gr_status gr_trie_info(const gr_trie* trie, int32_t* depth, int32_t* vocab,
                       int64_t* num_nodes, int32_t* max_fanout);

void gr_trie_free(gr_trie* trie);   /* NULL-safe */

/* Give trie level `level` a dense representation (FlashRec README,
 * "Decoding": the SID-constraint kernel reads a dense or a CSR-sparse trie).
 * The table has num_nodes[level] rows by span columns, where span = (largest
 * - smallest child token of the level) + 1.  Entry [n][i] holds the child of
 * node n through token smallest + i, or -1 where node n has no such child.
 * Steps at that level then enumerate a node's row of the table instead of
 * its CSR edge range: a child's token and child node come from one load,
 * independent of the edge offsets.  Results are identical either way; tie
 * order and the edge ordinal become the code index, which is also token
 * order.  The table is built on the device from the CSR arrays on `stream`,
 * and the call waits for it.  Call it before enqueueing steps that should
 * use the table; a step reads a level's representation when it is enqueued.
 * The table is owned by the trie and freed with it.
 * *table_bytes (may be NULL) receives the table's size even when the call
 * declines.  Returns GR_OK if the level is already dense or has no edges;
 * GR_ERR_UNSUPPORTED (nothing allocated) when the table would exceed
 * max_bytes (< 0: no limit); GR_ERR_INVALID_ARG on a NULL trie or a level
 * outside [0, depth); GR_ERR_OUT_OF_MEMORY if the allocation fails. */
gr_status gr_trie_densify(gr_trie* trie, int32_t level, int64_t max_bytes, gr_stream stream,
                          int64_t* table_bytes);

/* ------------------------------------------------------------------ beam */

typedef struct {
    int32_t batch;          /* B >= 1 independent requests */
    int32_t beam_width;     /* K, 1 <= K <= 4096 */
    int32_t vocab;          /* V, logits per row; must equal the trie's */
    int32_t max_steps;      /* T >= 1; with a trie, T <= depth */
    int32_t eos_token;      /* EOS id in [0, V), or -1 for none; must be -1 with a trie */
    int32_t logits_dtype;   /* GR_F32 or GR_BF16 */
    int64_t logits_row_stride; /* elements between consecutive rows; 0 = V */
} gr_beam_config;

/*
 * Allocate a beam state for `cfg` and set it to the start of a search
 * (slot 0 of every request live with score +0 at the trie root; the other
 * slots empty; histories -1).  trie == NULL selects unconstrained search.
 * (beamgrad README, "C and C++": an opaque handle made by an init call,
 * zero-default options, an explicit free; the shapes follow its Python
 * example: scores [B, K], sequences [B, K, T].  The single live slot at the
 * start is this library's reading: the pages do not say how a search begins.)
 * All device memory a search needs (state, history, workspace) is allocated
 * here; gr_beam_step allocates nothing.  Synchronises `stream`.
 */
gr_status gr_beam_init(const gr_beam_config* cfg, const gr_trie* trie, gr_stream stream,
                       gr_beam** out);

/* Reset to the start of a search (as after init), enqueued on `stream`. */
gr_status gr_beam_reset(gr_beam* beam, gr_stream stream);

/*
 * Enqueue one beam step on `stream`: the computation at the top of this
 * header (beamgrad README, "How it works": every live beam proposes its
 * tokens, cumulative log-probabilities rank them, the K best survive and
 * finished beams are carried; FlashRec README, "Features", "Decoding": only
 * the children of each beam's trie node are candidates).
 *   d_logits  device array of B*K rows; row (b, j) starts at element
 *             (b*K + j) * row_stride and holds V values of the configured
 *             dtype (fp32, or bf16 as raw 16-bit patterns).  Rows of empty
 *             and finished slots are not read.  Caller-owned; it must stay
 *             valid until the stream has passed this step.
 * The step index advances on the host at once.  Returns GR_ERR_STATE past
 * max_steps (or past the trie depth), GR_ERR_INVALID_ARG for a NULL logits
 * pointer, GR_ERR_HIP if a launch fails.  Never allocates, never syncs.
 */
gr_status gr_beam_step(gr_beam* beam, const void* d_logits, gr_stream stream);

/*
 * Whole-search launch (FlashRec README, "Decoding": a wide beam step runs as
 * one captured graph replay; here the whole multi-step loop does).  Enqueues
 * `nsteps` consecutive steps on `stream` as one HIP graph launch, or, when
 * every step is a fused step of one workgroup per request, as one kernel
 * launch per eight steps in which each request's workgroup runs its steps
 * in order (no graph is captured then): step i
 * (index step + i) reads the logits at d_logits[i] (host array of nsteps
 * device pointers, each laid out as for gr_beam_step).  The result equals
 * nsteps gr_beam_step calls with the same logits, bit for bit.  The first
 * call with a given starting state (step index, live bound, buffer half),
 * settings and logits pointers captures and instantiates a graph (driver
 * host work, a few hundred microseconds); later calls that match replay it
 * from a cache of 8 per beam, so a serving loop that reuses its logits
 * buffers pays only the replay.  Library timing events are not recorded
 * for graph launches.  gr_beam_rewind afterwards undoes the last of the
 * steps.  Errors: GR_ERR_INVALID_ARG for NULL pointers or nsteps < 1,
 * GR_ERR_STATE if a step would pass max_steps or the trie depth (nothing
 * is enqueued then), GR_ERR_HIP if capture, instantiation or launch fails
 * (in the single-launch form, steps that earlier launches of the same call
 * enqueued stay enqueued, and the beam's step index counts them).
 */
gr_status gr_beam_search(gr_beam* beam, const void* const* d_logits, int32_t nsteps, gr_stream stream);

/*
 * One beam step for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops that must not call hipMalloc, harnesses
 * that forbid it.  It computes exactly what gr_beam_step computes, with the
 * same kernels, but without a gr_beam handle: the caller passes the state
 * before the step and buffers for the state after it, and the step's
 * workspace (each row's candidate summary, counts and first edge, and the
 * step counters) lives in one static device buffer of the library,
 * GR_STATIC_SCRATCH_BYTES per GPU, held until the process ends.  Nothing is
 * allocated and nothing synchronises; the first call on a device also looks
 * up that device's buffer and sets the kernels' LDS limit (driver calls, no
 * allocation).
 *
 * Every call on one GPU uses that GPU's one buffer: calls whose work may
 * overlap on a GPU (other streams, other threads) race and give wrong
 * results.  Order them on one stream.  The buffer keeps the last call's
 * contents; each step writes all of the workspace it later reads.
 *
 *   config      as for gr_beam_init (logits_row_stride 0 = V)
 *   trie        NULL = unconstrained; else config.max_steps <= its depth
 *   step        0-based index t of this step (t < max_steps, t < depth):
 *               selects the trie level and the EOS rules
 *   live_bound  every slot j >= live_bound of every request is empty
 *               (0 = beam_width: all may be live); rows past it are not read
 *   temperature, seed  as gr_beam_set_sampling (0 = deterministic)
 *   logits      device rows as for gr_beam_step
 *   scores, nodes, finished, sequences  the state before the step, device
 *               arrays of the gr_beam_view shapes ([B, K], [B, K, T])
 *   *_out       the state after the step, same shapes; parents_out and
 *               tokens_out are this step's history rows [B, K]; lse_out
 *               [B, K] the normaliser of each row read (NaN otherwise).
 *               Outputs must not overlap the inputs.
 *
 * Errors: GR_ERR_INVALID_ARG for a NULL io or buffer, a bad configuration or
 * overlapping buffers; GR_ERR_STATE for a step index past max_steps or the
 * trie depth; GR_ERR_UNSUPPORTED when the step's workspace exceeds
 * GR_STATIC_SCRATCH_BYTES (the message names the bytes it needs; it grows
 * with batch x live_bound) or the configuration exceeds the kernels' LDS;
 * GR_ERR_HIP if a launch or the buffer lookup fails.  Length penalties,
 * banned tokens and normalisation variants need device tables and are not
 * offered here (use a gr_beam handle).
 */
#define GR_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

typedef struct {
    gr_beam_config config;
    const gr_trie* trie;
    int32_t step;
    int32_t live_bound;
    float temperature;
    uint64_t seed;
    const void* logits;
    const float* scores;
    const int32_t* nodes;
    const uint8_t* finished;
    const int32_t* sequences;
    float* scores_out;
    int32_t* nodes_out;
    uint8_t* finished_out;
    int32_t* sequences_out;
    int32_t* parents_out;
    int32_t* tokens_out;
    float* lse_out;
} gr_step_io;

gr_status gr_beam_step_static(const gr_step_io* io, gr_stream stream);

/*
 * Choose how a step runs (a tuning switch; results are identical either way;
 * FlashRec README, "Decoding": a wide beam step as one launch).
 *   mode 1 (the default): a step over a CSR trie level whose rows are short
 *     (V below 2,048 logits), ranked by the plain cumulative score with
 *     the full-row normaliser, K <= 2048, skips the per-row summaries: with
 *     at most 16 live rows per request one kernel does the whole step;
 *     otherwise the rows of each request are split over several workgroups
 *     that keep their K best, and a merge kernel selects among them.  Every
 *     other step runs the row kernel and then the request kernel.
 *   mode 0: every step runs the row kernel and then the request kernel.
 *   mode 2: as mode 1, with even the smallest requests split (for tests).
 * Errors: GR_ERR_INVALID_ARG for NULL or another mode.
 */
gr_status gr_beam_set_fused(gr_beam* beam, int32_t mode);

/*
 * Undo the last gr_beam_step: the state it read becomes current again and
 * the step index goes back by one (history rows it wrote are left as they
 * are; stepping again rewrites them).  A step reads one half of the
 * double-buffered state and writes the other, so nothing is copied and
 * nothing is enqueued: repeating a step on new logits costs only the step.
 * Allowed once after each step.  Work already enqueued is unaffected; the
 * next step must be ordered after the rewound one if both use the state
 * (same stream).  Errors: GR_ERR_INVALID_ARG for NULL, GR_ERR_STATE when
 * the last call on the beam was not a step (init, reset, set_state, or a
 * rewind).
 */
gr_status gr_beam_rewind(gr_beam* beam);

/* Device views of the state after the last step.  Valid until the next
 * step, reset or free; owned by the handle.  (beamgrad README, the Python
 * example: scores [B, K] best first, sequences [B, K, T] with -1 after a
 * beam ends, the parent chosen at each step.)  Errors: GR_ERR_INVALID_ARG
 * for a NULL beam or out. */
typedef struct {
    int32_t step;        /* steps done so far */
    int32_t batch, beam_width, vocab, max_steps;
    float* scores;       /* [B, K] cumulative scores, best first; -inf = empty */
    int32_t* nodes;      /* [B, K] trie node at the next level (leaf id after
                            the last level); -1 = empty or unconstrained */
    uint8_t* finished;   /* [B, K] 1 if the beam has emitted EOS */
    int32_t* sequences;  /* [B, K, T] tokens, -1 after the end / unused */
    int32_t* parents;    /* [T, B, K] parent slot chosen at each step, -1 = empty */
    int32_t* tokens;     /* [T, B, K] token emitted at each step, -1 = carried/empty */
    float* lse;          /* [B, K] row normaliser of each slot read by the last
                            step (indexed by the previous step's slot), NaN if
                            that row was not read */
} gr_beam_view;

gr_status gr_beam_view_get(const gr_beam* beam, gr_beam_view* out);

/*
 * Overwrite the state (for re-synchronising with another implementation,
 * resuming, or repeating a step).  All pointers are device arrays of the
 * shapes in gr_beam_view; they are copied on `stream`.  `step` becomes the
 * index of the next step (0 <= step < max_steps).  History rows before
 * `step` are left as they are.  The call then finds the last slot of any
 * request that holds a beam (a score that is not -inf), which bounds the
 * rows the next step reads, and returns once `stream` has done the copies.
 */
gr_status gr_beam_set_state(gr_beam* beam, int32_t step, const float* d_scores,
                            const int32_t* d_nodes, const uint8_t* d_finished,
                            const int32_t* d_sequences, gr_stream stream);

void gr_beam_free(gr_beam* beam);   /* NULL-safe; synchronises the device */

/*
 * Sampling (FlashRec README, "Serving", API item: deterministic top-k at
 * temperature 0, Gumbel top-k without replacement above it).  With
 * temperature T > 0, later steps temper every live row (xt = fl32(x *
 * fl32(1/T))), normalise it over the full row, and rank each candidate by
 * fl32(c + g), c = S_j + (xt_v - lse_j) its cumulative score and g a standard
 * Gumbel draw: g = -log(-log(u)) in fp64 rounded to fp32, u = (r + 1/2) 2^-32,
 * r = word (flat mod 4) of Philox4x32-10 (Salmon et al., SC 2011) at counter
 * (flat div 4, request index in the batch, step, 0) with key (seed low 32
 * bits, seed high 32 bits), flat = j*V + token (a finished beam draws at
 * j*V + eos).  The K best by that rank fill the slots in that order, and each
 * slot keeps its unperturbed score c.  T = 0 (the default) restores the
 * deterministic top-K.  Takes effect from the next gr_beam_step; does not
 * synchronise.  Errors: GR_ERR_INVALID_ARG for a NULL beam or a negative or
 * non-finite temperature.
 */
gr_status gr_beam_set_sampling(gr_beam* beam, float temperature, uint64_t seed);

/*
 * Length penalty, minimum length and banned tokens (beamgrad README,
 * "Features": GNMT length penalty, minimum length, banned tokens; "How it
 * works": the cumulative log-probability is ranked by
 * raw / ((5 + length) / 6) ** alpha).  Later steps rank each candidate by
 * fl32(c / pen(len)) (then by the Gumbel draw when sampling, added to that),
 * pen(len) = (float)pow((5 + len) / 6, alpha) computed in double, len = the
 * hypothesis' tokens including EOS (step + 1 for a live beam's candidate, its
 * own length for a finished beam carried forward); slots keep the raw c.  EOS
 * is not a candidate while step + 1 < min_length; the n_banned token ids at
 * `banned` (host memory, any order, duplicates allowed) never are, with or
 * without a trie.  alpha = 0, min_length <= 1, n_banned = 0 (the defaults)
 * change nothing.  Copies small tables (allocated by gr_beam_init) on
 * `stream` and synchronises it; call it between steps, not while a step of
 * this beam may still run on another stream.
 * Errors: GR_ERR_INVALID_ARG for a NULL beam, a non-finite alpha, a negative
 * min_length or count, a NULL list with n_banned > 0, or a token outside
 * [0, vocab); GR_ERR_HIP if a copy fails.
 */
gr_status gr_beam_set_penalties(gr_beam* beam, float alpha, int32_t min_length, const int32_t* banned,
                                int32_t n_banned, gr_stream stream);

/*
 * Normalisation variants of later steps (the default normalises every live
 * row over its full vocabulary):
 *   GR_NORM_RANGE [lo, hi) -- FlashRec README, "Decoding": lm_head is
 *     evaluated only over the SID token range.  The row normaliser runs over
 *     tokens lo <= v < hi only (only that part of each row is read); tokens
 *     outside the range are never candidates.
 *   GR_NORM_SLICE -- Qwen-2.5-1B-RLCD-Fast model card, "Sub-Vocabulary Logit
 *     Slicing": probabilities normalised over the candidate slice only.  A
 *     trie row's normaliser runs over its node's children (before banned
 *     tokens and the minimum length are applied); the row itself is not
 *     streamed.  Without a trie this equals GR_NORM_FULL.
 *   GR_NORM_NONE -- beamgrad README, the C API example: the decoder takes
 *     log_probs.  The values are log-probabilities already: lse = 0, lp = x
 *     (times 1/T when sampling), and rows are not streamed (only candidates
 *     are read).  gr_beam_backward's path gradients are then gradients with
 *     respect to these values.
 * lse, lp and c keep their definitions with the chosen normaliser; lo and hi
 * are ignored unless mode is GR_NORM_RANGE.  Does not synchronise.  Errors:
 * GR_ERR_INVALID_ARG for a NULL beam, an unknown mode, or a range not inside
 * [0, vocab) or empty.
 */
enum { GR_NORM_FULL = 0, GR_NORM_RANGE = 1, GR_NORM_SLICE = 2, GR_NORM_NONE = 3 };
gr_status gr_beam_set_normalization(gr_beam* beam, int32_t mode, int32_t lo, int32_t hi);

/* ---------------------------------------------------------- backward */

/*
 * Surrogate backward of the search so far (beamgrad README, "How it works":
 * backward holds the selection fixed; the gradient of final beam k's score
 * -- its cumulative log-probability divided by the length penalty -- with
 * respect to log_probs[t, p, v] is 1 / penalty(length_k) for every
 * (t, p, v) on k's path and zero elsewhere; "Features": each step is handed
 * only its own path gradient, never a dense [B, T, K, V] array).  Here
 * log_probs[t] are the values step t ranked by: lp = x/T - lse of row p
 * under the chosen normaliser (with GR_NORM_NONE, the inputs themselves).
 *
 * gr_beam_backward, with steps = the current step index (>= 1) and the
 * current state as the final beams:
 *   d_grad_final  [B, K] device fp32: upstream gradient of each final slot
 *   d_path_slot   [steps, B, K] device int32, out: slot of final beam
 *                 (b, k)'s hypothesis read at step t (the row whose
 *                 log-probability it used), -1 for empty final slots
 *   d_path_token  [steps, B, K] device int32, out: the token it emitted at
 *                 step t; -1 where the beam was carried (finished: that step
 *                 adds nothing) and for empty final slots
 *   d_weight      [B, K] device fp32, out: fl32(grad / pen(len)), len = the
 *                 tokens of the final sequence (EOS included), 0 for empty
 *                 slots; pen is the current length-penalty table (1 when
 *                 alpha = 0)
 * The paths follow the history rows this beam's steps wrote since its last
 * init or reset (after gr_beam_set_state, rows before its step are whatever
 * they held).  Enqueued on `stream`; no synchronisation.  Errors:
 * GR_ERR_INVALID_ARG for NULL pointers, GR_ERR_STATE before the first step.
 *
 * gr_beam_backward_scatter adds step `step`'s log-probability gradient to
 * d_grad (device fp32, row (b, p) at (b*K + p) * grad_row_stride elements,
 * 0 = vocab): for each distinct (p, v) with v >= 0 among the paths at that
 * step in request b, the weights of the final beams through it, summed in
 * fp32 from 0 in ascending k, are added once to d_grad[b][p][v].  Entries
 * outside [0, K) x [0, V) are skipped.  Other elements are not touched.
 * Enqueued on `stream`.  Errors: GR_ERR_INVALID_ARG for NULL pointers, a
 * step outside [0, current step) or a stride below vocab.
 */
gr_status gr_beam_backward(gr_beam* beam, const float* d_grad_final, int32_t* d_path_slot,
                           int32_t* d_path_token, float* d_weight, gr_stream stream);
gr_status gr_beam_backward_scatter(gr_beam* beam, int32_t step, const int32_t* d_path_slot,
                                   const int32_t* d_path_token, const float* d_weight, float* d_grad,
                                   int64_t grad_row_stride, gr_stream stream);

/* ---------------------------------------------------------- observability */

/*
 * Kernel timing: when enabled, every later gr_beam_step records HIP events
 * around each of its kernels on the step's stream.  gr_beam_timing_get
 * synchronises on the last events and returns the accumulated milliseconds
 * of the row kernel (log-softmax normaliser, candidate gather and per-row
 * pre-selection) and of the request kernel (per-request top-K and state
 * update), and the number of timed steps; gr_beam_timing_reset clears them.
 * A fused step (gr_beam_set_fused) counts its row-streaming kernel as row
 * time and its merge kernel, when it has one, as request time; a fused step
 * that is one kernel adds nothing to the request time.
 */
gr_status gr_beam_timing_enable(gr_beam* beam, int32_t enable);
gr_status gr_beam_timing_get(gr_beam* beam, double* row_ms, double* select_ms, int64_t* steps);
gr_status gr_beam_timing_reset(gr_beam* beam);

/* Counters of the last step, copied to the host (synchronises the stream
 * of that step): live rows read, candidates emitted, candidates that passed
 * the per-request bound (fused step: the sum over its workgroups of their
 * K best),
 * requests that took the slow selection path, rows whose candidates the
 * request kernel recomputed because their whole summary passed the bound,
 * and requests whose step ran as the fused kernel (gr_beam_set_fused). */
typedef struct {
    int64_t rows_read;
    int64_t candidates;
    int64_t survivors;
    int64_t slow_path_requests;
    int64_t rescanned_rows;
    int64_t fused_requests;
} gr_step_stats;

gr_status gr_beam_last_stats(gr_beam* beam, gr_step_stats* out);

/* ----------------------------------------------------------------- probes */

/* Read `bytes` (a multiple of 16) from device memory at d_src with 16-byte
 * non-temporal loads, each workgroup one contiguous 64 KB chunk with eight
 * loads in flight per thread (the fastest plain read found on MI355X),
 * folding into d_sink (>= 65536 words): an achievable-bandwidth reference. */
gr_status gr_probe_read(const void* d_src, size_t bytes, uint32_t* d_sink, gr_stream stream);

/* Copy `bytes` (a multiple of 16) from d_src to d_dst; a kernel of known
 * traffic for calibrating memory counters. */
gr_status gr_probe_copy(void* d_dst, const void* d_src, size_t bytes, gr_stream stream);

/* Sampled unconstrained rows are pruned with fast fp32 estimates of the
 * Gumbel variates (the ranking itself always uses the exact fp64-derived
 * variate; FlashRec README, "Serving", the API item: Gumbel top-k without
 * replacement above temperature 0).  This probe
 * writes to the device double at d_out (8 bytes, caller-owned) the largest
 * difference between estimate and exact variate over the Philox words
 * r0 .. r0 + count - 1 (count <= 2^32; all 2^32 words take a few tens of
 * milliseconds), enqueued on `stream`.  GR_ERR_INVALID_ARG on a NULL d_out
 * or a larger count. */
gr_status gr_probe_draw_error(uint32_t r0, uint64_t count, double* d_out, gr_stream stream);

/* The bound on that difference which the pruning assumes. */
double gr_draw_error_bound(void);

/* ------------------------------------------------------------------ misc */

/* Enqueue a copy of `bytes` between any two host or device addresses on
 * `stream` (for reading views into caller-owned buffers). */
gr_status gr_memcpy(void* dst, const void* src, size_t bytes, gr_stream stream);

const char* gr_status_string(gr_status status);
const char* gr_last_error(void);   /* thread-local; never NULL */
const char* gr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GR_H */
