/*
 * ngram.h -- C ABI of the hashed bigram + trigram embedding table with sparse
 * row-wise updates, for AMD Instinct MI355X (gfx950).
 *
 * The method (modded-nanogpt README, technique list: a hashed bigram +
 * trigram embedding table of 84.6M rows with a sign trick, and sparse
 * row-wise embedding updates with beta1 = 0, one second moment per row,
 * every 4 steps; the @classiclarryd post quoted on the airebao.com item about
 * the 39.9 s record: only rows seen in the batch get an optimizer step, beta2
 * is applied retroactively when a row is next used, one optimizer float per
 * 768 parameters; agentic-affairs "NanoGPT Training Record", ablation section:
 * 84.6M rows across a bigram and a trigram channel; amund.blog "My 2nd
 * modded-nanogpt world record attempt", The four improvements, item 4: the
 * accumulated n-gram gradients can be added as each step produces them or in
 * one burst every fourth step, with the same result):
 *
 *   per position i of a micro-step, with n-gram context reset at each EoS,
 *     r_b, s_b = hash_b(t[i-1], t[i]);  r_t, s_t = hash_t(t[i-2], t[i-1], t[i])
 *     out[i]   = s_b W_b[r_b] + s_t W_t[r_t]
 *   per accumulation window (accum_steps micro-steps), per touched row r:
 *     G[r]     = sum of s dY[i] over the window's positions hashed to r
 *   sparse step t (t = 1, 2, ... counts optimizer steps), per touched row:
 *     v[r]     = beta2^(t - t_last[r]) v[r] + (1 - beta2) mean(G[r]^2)
 *     W[r]    -= lr G[r] / (sqrt(v[r]) + eps);   t_last[r] = t
 *
 * Readings of what the pages leave open (the CPU oracle shares them):
 *   hash      SplitMix64 finaliser of (key ^ seed) + 0x9E3779B97F4A7C15; row =
 *             ((z >> 32) * R) >> 32 (Lemire); sign negative iff z & 1.
 *   keys      bigram p1*(V+1) + t, trigram (p2*(V+1) + p1)*(V+1) + t in 64-bit
 *             unsigned arithmetic, V = vocab, a missing token written as V.
 *   context   p1 = t[i-1] unless i == 0 or t[i] is EoS; p2 = t[i-2] unless
 *             i < 2 or t[i] or t[i-1] is EoS.  Every micro-step starts afresh.
 *   forward   one fp32 addition of the two signed rows, then one rounding to
 *             the table dtype (bf16: nearest, ties to even; NaN -> 0x7FC0).
 *   update    no bias correction (fold it into lr and eps), eps outside the
 *             root, no weight decay, gradients summed (not averaged) over the
 *             window.
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers unless marked "host".  The caller owns
 *     every buffer; the library never allocates, frees or synchronises in the
 *     hot calls (ngram_hash, ngram_embed_fwd, ngram_embed_bwd_accum,
 *     ngram_embed_bwd_step, ngram_window_keys, ngram_window_sort,
 *     ngram_window_reduce, ngram_sparse_step, ngram_window_export,
 *     ngram_touched_rows and the _dev step variants).  Those calls only enqueue work on `stream` (a
 *     hipStream_t; NULL = the null stream) and return; they are safe to
 *     capture in a HIP graph (with the _dev step variants, a replay can take
 *     a new step number and learning rate).
 *   - A negative return value is a host-detected error and nothing was
 *     enqueued.  NGRAM_EHIP reports a failed launch.
 *   - Faults only the device can see (token ids outside [0, vocab), more
 *     distinct rows than the window holds, a full burst stash, step numbers
 *     that do not increase, out-of-range device step parameters, burst
 *     windows not ready for their step) set sticky NGRAM_FLAG_* bits in the
 *     workspace, read with ngram_device_status.
 *   - Tables and row-major activations are [rows][dim] with dim = 768; all
 *     row bases must be 16-byte aligned.  Row counts must be below 2^31.
 *   - One workspace serves one table pair; the calls on it must be ordered
 *     (one stream, or event waits where ngram_window_keys / ngram_window_sort
 *     run on another).  Distinct workspaces are independent (the library
 *     keeps no global state).
 */
#ifndef NGRAM_H
#define NGRAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NGRAM_ABI_VERSION 10

/* dtypes of the tables (and of the forward output), and of the upstream
 * gradients dY */
#define NGRAM_DTYPE_F32 0
#define NGRAM_DTYPE_BF16 1

/* how micro-step gradients enter the window (amund.blog, The four
 * improvements, item 4) */
#define NGRAM_MODE_SPREAD 0     /* reduce each micro-step into the window now */
#define NGRAM_MODE_BURST 1      /* keep micro-steps (dY copied into the
                                   workspace); reduce all at step time       */
#define NGRAM_MODE_BURST_REF 2  /* as BURST, but dY is not copied: the caller
                                   keeps every micro-step's dY unchanged until
                                   the window's step (max_tokens <= 2^25)    */

/* status codes */
#define NGRAM_OK 0
#define NGRAM_ENULL -1    /* a required pointer is NULL                     */
#define NGRAM_EALIGN -2   /* a pointer is not aligned as documented         */
#define NGRAM_ECONFIG -3  /* the config is invalid (see ngram_config_check) */
#define NGRAM_ESIZE -4    /* a size is out of range                         */
#define NGRAM_EARG -5     /* a scalar argument is out of range              */
#define NGRAM_EHIP -6     /* the HIP runtime reported an error              */

/* sticky device flags */
#define NGRAM_FLAG_BAD_TOKEN 0x1u   /* a token id outside [0, vocab)          */
#define NGRAM_FLAG_WINDOW_FULL 0x2u /* more distinct rows than window_rows;
                                       the excess rows were dropped          */
#define NGRAM_FLAG_STASH_FULL 0x4u  /* burst mode: more than accum_steps *
                                       max_tokens positions before a step;
                                       the excess micro-step was dropped     */
#define NGRAM_FLAG_STEP_ORDER 0x8u  /* sparse step t <= t_last of a touched
                                       row; that row decays by beta2^0       */
#define NGRAM_FLAG_BAD_PARAMS 0x10u /* step parameters read from device
                                       memory were out of range; that step
                                       changed no row and emptied the window */
#define NGRAM_FLAG_WINDOW_UNREADY 0x20u /* burst modes: a window reached its
                                       reduction with keys recorded ahead
                                       whose gradients never came, or (with
                                       NGRAM_OPT_PRESORT) not sorted since
                                       its last keys; the window was dropped:
                                       no row changed                        */
#define NGRAM_FLAG_KEYS_MISMATCH 0x40u /* burst modes: a micro-step's
                                       gradients came with another T than
                                       its keys recorded ahead; they were not
                                       attached (the window is then dropped
                                       with NGRAM_FLAG_WINDOW_UNREADY)       */

/* options (ngram_config.options) */
#define NGRAM_OPT_PRESORT 0x1  /* burst modes: the caller sorts every window
                                  with ngram_window_sort after its last keys
                                  and before its step, which then skips the
                                  sort (see ngram_window_keys)              */
#define NGRAM_OPT_OUT_F32 0x2  /* the forward writes fp32 whatever the table
                                  dtype: the exact fp32 sum of the two
                                  signed rows, not rounded to bf16          */
#define NGRAM_OPT_DIRECT 0x4   /* one table indexed by the token id itself
                                  (value embeddings, updated on the same
                                  4-step cadence: @classiclarryd post): row
                                  = id, sign +1, no hashing, no context;
                                  rows[0] >= vocab; rows[1], W_t and
                                  state_t are not used (W_t and state_t may
                                  be NULL).  The forward is out[i] =
                                  W_b[t[i]]; an id outside [0, vocab) is
                                  flagged and reads row 0                   */
#define NGRAM_OPT_NEST_ALWAYS 0x8  /* fused reductions (the burst modes'
                                  step, spread mode's fused last micro-
                                  step) sort the bigram keys by (bigram
                                  row, trigram row) and complete trigram
                                  rows of several positions in the bigram
                                  pass at any window size; without it only
                                  reductions of at least 2^20 positions do
                                  (a smaller one sorts faster than it would
                                  gain).  Schedule only: the results are
                                  the same within the stated tolerances     */

typedef struct ngram_config {
    int32_t vocab;       /* V: token ids are valid in [0, V); 50304 in the
                            speedrun (agentic-affairs, benchmark definition) */
    int32_t eos_id;      /* the EoS id that opens each document             */
    int32_t dim;         /* row width; must be 768                          */
    int32_t dtype;       /* NGRAM_DTYPE_F32 or NGRAM_DTYPE_BF16             */
    int64_t rows[2];     /* rows of the bigram [0] and trigram [1] tables,
                            each in [1, 2^31)                               */
    uint64_t seed[2];    /* hash seeds of the two channels                  */
    int64_t max_tokens;  /* largest T of one micro-step, in [1, 2^28]       */
    int32_t accum_steps; /* micro-steps per window, in [1, 64]              */
    int32_t mode;        /* NGRAM_MODE_SPREAD, _BURST or _BURST_REF         */
    int64_t window_rows; /* distinct rows one window can hold per channel;
                            0 = min(max(rows[0], rows[1]),
                                    accum_steps * max_tokens); the result
                            must be below 2^30 - 1                         */
    int32_t dy_dtype;    /* dtype of dY: NGRAM_DTYPE_F32 (0) or
                            NGRAM_DTYPE_BF16 (the gradient a bf16 model
                            returns for a bf16 forward output); window sums
                            are fp32 either way                             */
    int32_t options;     /* NGRAM_OPT_* bits; 0 = none                      */
} ngram_config;

/* Optimizer state of one table row (8 bytes, 8-byte aligned arrays): the
 * second moment v (one float per 768-wide row, the @classiclarryd post) and
 * the optimizer step at which the row was last updated (its pending beta2
 * decay is beta2^(t - t_last)).  Start at {0, 0}. */
typedef struct ngram_row_state {
    float v;
    int32_t t_last;
} ngram_row_state;

/* Step parameters in device memory (16 bytes, 16-byte aligned), for the
 * _dev step entry points: the kernels read them when they run, so a captured
 * HIP graph replays with whatever the caller stored there last (the
 * speedrun's training step is graph-captured: agentic-affairs "NanoGPT
 * Training Record", ablation section).  Valid values as for
 * ngram_sparse_step. */
typedef struct ngram_step_params {
    int32_t t;
    float lr;
    float beta2;
    float eps;
} ngram_step_params;

/* Version of this ABI (NGRAM_ABI_VERSION). */
int ngram_abi_version(void);

/* Static text for a status code (never NULL). */
const char *ngram_status_string(int status);

/* Validates a config on the host.  Returns NGRAM_OK or NGRAM_ECONFIG. */
int ngram_config_check(const ngram_config *cfg);

/* Bytes of device workspace the config needs (host output `bytes`).  The
 * workspace holds the window accumulator (window_rows x 768 fp32 per
 * channel), a row->slot map (8 B per table row), sort buffers, and in burst
 * mode a copy of the window's upstream gradients. */
int ngram_workspace_bytes(const ngram_config *cfg, uint64_t *bytes);

/* Prepares a workspace of `ws_bytes` bytes (256-byte aligned) on `stream`:
 * empty window, no flags.  Must be called once before any other use of `ws`
 * and may be called again to discard a window. */
int ngram_workspace_init(const ngram_config *cfg, void *ws, uint64_t ws_bytes,
                         void *stream);

/* Context + hash of one micro-step (modded-nanogpt README, technique list:
 * hashed bigram + trigram table with sign trick; EoS-aligned batches).
 * tokens: int32 [T], 4-byte aligned.  idx: uint32 [2][T] (bigram row block,
 * then trigram), each entry row | (negative << 31).  ws may be NULL; if not,
 * bad token ids set NGRAM_FLAG_BAD_TOKEN there.  0 <= T <= max_tokens. */
int ngram_hash(const ngram_config *cfg, const int32_t *tokens, int64_t T,
               uint32_t *idx, void *ws, void *stream);

/* Forward of one micro-step: out[i] = s_b W_b[r_b(i)] + s_t W_t[r_t(i)]
 * (same passages as ngram_hash).  W_b, W_t: [rows[c]][768] of cfg->dtype.
 * out: [T][768] of cfg->dtype, or fp32 with NGRAM_OPT_OUT_F32; must not
 * overlap the tables.  ws may be NULL
 * (bad token ids then go unreported; their rows are still valid rows). */
int ngram_embed_fwd(const ngram_config *cfg, const void *W_b, const void *W_t,
                    const int32_t *tokens, int64_t T, void *out, void *ws,
                    void *stream);

/* Backward of one micro-step into the window accumulator (gradients are
 * accumulated over accum_steps micro-steps and applied once: the
 * @classiclarryd post; README technique list).  dY: [T][768] of
 * cfg->dy_dtype, 16-byte aligned, the gradient of `out` for the same tokens.
 * Each position's signed dY row is added to its rows' window sums in fp32.  Spread mode reduces now (dY may be
 * reused once the stream passes this call); burst mode keeps the tokens' rows
 * and a copy of dY in the workspace and reduces at ngram_window_reduce /
 * ngram_sparse_step; burst-by-reference mode keeps the rows and only the
 * address of dY, which must stay unchanged until the window's step. */
int ngram_embed_bwd_accum(const ngram_config *cfg, void *ws,
                          const int32_t *tokens, const void *dY, int64_t T,
                          void *stream);

/* Burst mode: reduce every micro-step kept since the last step into the
 * window accumulator now (ngram_sparse_step does this itself).  Spread mode:
 * nothing to do.  Calling it twice is harmless. */
int ngram_window_reduce(const ngram_config *cfg, void *ws, void *stream);

/* Burst modes: records the sort keys of the window's next micro-step now,
 * from its tokens alone (a window's n-gram rows depend on its tokens, not on
 * its gradients).  The matching ngram_embed_bwd_accum (or
 * ngram_embed_bwd_step), the next one called for this window, then only
 * attaches the micro-step's dY (same T, else NGRAM_FLAG_KEYS_MISMATCH).
 * Micro-steps may be recorded ahead in any number up to accum_steps, and
 * ngram_window_sort can then sort the window on another stream while the
 * forwards and the model run.  A window whose recorded keys never get their
 * gradients is dropped at its step (NGRAM_FLAG_WINDOW_UNREADY).  Order this
 * call before the micro-step's backward (same stream, or an event wait):
 * a backward that runs first keeps the keys itself, and the ones recorded
 * later then belong to a further micro-step.
 * tokens: int32 [T], the same tokens the micro-step's forward gets. */
int ngram_window_keys(const ngram_config *cfg, void *ws, const int32_t *tokens,
                      int64_t T, void *stream);

/* Burst modes: sorts the window's keys recorded so far (by ngram_window_keys
 * or ngram_embed_bwd_accum), finds the distinct rows and splits off the
 * trigram rows that occur once, i.e. everything the step's fused reduction
 * needs besides the gradients.  With NGRAM_OPT_PRESORT the step skips these
 * kernels and requires this call after the window's last keys (else the
 * window is dropped with NGRAM_FLAG_WINDOW_UNREADY); without the option the
 * step sorts again.  Order it before the step on the step's stream (an event
 * wait if it runs on another stream).  Spread mode: nothing to do. */
int ngram_window_sort(const ngram_config *cfg, void *ws, void *stream);

/* Sparse step number t >= 1 on every row the window touched, then empties the
 * window (the @classiclarryd post: optimizer step only for n-gram rows that
 * occurred, beta1 = 0, beta2 applied retroactively, one float per 768
 * parameters).  W_b, W_t: tables of cfg->dtype, updated in place.  state_b,
 * state_t: ngram_row_state [rows[c]] (v and t_last of every row), updated for
 * the touched rows only.  Requires 0 <= beta2 < 1, eps > 0 and finite, lr
 * finite. */
int ngram_sparse_step(const ngram_config *cfg, void *ws, void *W_b, void *W_t,
                      ngram_row_state *state_b, ngram_row_state *state_t,
                      int32_t t, float lr, float beta2, float eps,
                      void *stream);

/* The last micro-step of a window fused with the sparse step: the same as
 * ngram_embed_bwd_accum(tokens, dY, T) followed by ngram_sparse_step(t, ...),
 * but every row this micro-step touches gets its window gradient completed
 * and its step applied in the reduction itself, so its gradient never goes
 * back to memory; the other rows of the window are stepped as usual.  In
 * burst mode the whole window is reduced this way.  Arguments as for those
 * two calls; the window is empty afterwards. */
int ngram_embed_bwd_step(const ngram_config *cfg, void *ws,
                         const int32_t *tokens, const void *dY, int64_t T,
                         void *W_b, void *W_t, ngram_row_state *state_b,
                         ngram_row_state *state_t, int32_t t, float lr,
                         float beta2, float eps, void *stream);

/* ngram_sparse_step and ngram_embed_bwd_step with the step parameters
 * (t, lr, beta2, eps) read from `params` in device memory when the kernels
 * run, for callers that capture a window in a HIP graph and replay it with a
 * new step number and learning rate each time.  The library cannot check
 * device-resident values on the host: out-of-range ones set
 * NGRAM_FLAG_BAD_PARAMS, and that step then writes no table row and no row
 * state (the window is still emptied). */
int ngram_sparse_step_dev(const ngram_config *cfg, void *ws, void *W_b,
                          void *W_t, ngram_row_state *state_b,
                          ngram_row_state *state_t,
                          const ngram_step_params *params, void *stream);

int ngram_embed_bwd_step_dev(const ngram_config *cfg, void *ws,
                             const int32_t *tokens, const void *dY, int64_t T,
                             void *W_b, void *W_t, ngram_row_state *state_b,
                             ngram_row_state *state_t,
                             const ngram_step_params *params, void *stream);

/* Copies the current window of one channel (0 bigram, 1 trigram) to caller
 * buffers: the first min(n, max_rows) rows (uint32, first-touch order:
 * ascending within each reduced micro-step), their gradients G (fp32
 * [max_rows][768], 16-byte aligned; may be NULL), and n itself (uint32,
 * device).  In burst mode call ngram_window_reduce first. */
int ngram_window_export(const ngram_config *cfg, const void *ws, int channel,
                        uint32_t *rows, float *G, int64_t max_rows,
                        uint32_t *count, void *stream);

/* The distinct rows of one channel (0 bigram, 1 trigram) that the current
 * window touches, in ascending order: the rows that receive this window's
 * update and nothing else (the @classiclarryd post quoted on the airebao.com
 * item: only the rows that receive updates are passed on and stepped).
 * Valid after the window's last ngram_embed_bwd_accum (or ngram_window_keys)
 * and before its step; it covers the rows already reduced into the window
 * and, in the burst modes, those of every micro-step kept but not yet
 * reduced.  rows: int32 [max_rows], device, 4-byte aligned; the first
 * min(n, max_rows) rows are written.  count: int64, device, 8-byte aligned:
 * n.  Sync-free (capture-safe); uses the workspace's touched-row bits (one bit
 * per table row, 10.6 MB at 2 x 42.3M rows) and changes nothing else in it.
 * A token-indexed table (NGRAM_OPT_DIRECT) has no channel 1: n = 0. */
int ngram_touched_rows(const ngram_config *cfg, void *ws, int channel,
                       int32_t *rows, int64_t max_rows, int64_t *count,
                       void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one whole
 * accumulation window reduced and stepped in a single call, with no caller
 * workspace.  The same as, on a fresh workspace of cfg in burst-by-reference
 * mode with accum_steps = n_micro and max_tokens = T, calling
 * ngram_embed_bwd_accum for micro-steps 0 .. n_micro - 2 and
 * ngram_embed_bwd_step for the last one (same kernels, same results).
 * tokens: int32 [n_micro][T] (each micro-step starts without context, as in
 * every other call); dY: [n_micro][T][768] of cfg->dy_dtype, 16-byte aligned,
 * read in place while the call's kernels run; tables and row state as for
 * ngram_sparse_step.  cfg's mode, accum_steps, max_tokens, window_rows and
 * NGRAM_OPT_PRESORT are ignored; its tables, hash, dtypes and the other
 * options apply.
 * The window's workspace is a fixed 32 MiB array in the library's device
 * code, one per GPU, held until the process ends; the call allocates
 * nothing.  Limits: 1 <= n_micro <= 64 and n_micro * T <= 65,536 positions,
 * else NGRAM_ESIZE (nothing enqueued); T = 0 does nothing.  The array is
 * shared by every call on the same GPU and is re-initialised at each call:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  flags (device uint32, may be NULL): the
 * call ORs its NGRAM_FLAG_* bits into it when its kernels end.  The current
 * device must be the stream's device. */
int ngram_window_step_noalloc(const ngram_config *cfg, const int32_t *tokens,
                              const void *dY, int64_t T, int32_t n_micro,
                              void *W_b, void *W_t, ngram_row_state *state_b,
                              ngram_row_state *state_t, int32_t t, float lr,
                              float beta2, float eps, uint32_t *flags,
                              void *stream);

/* Kernel groups for ngram_profile_events. */
#define NGRAM_PROF_FWD 0    /* the forward gather-sum kernel              */
#define NGRAM_PROF_SORT 1   /* key build, radix sort, heads and slots     */
#define NGRAM_PROF_REDUCE 2 /* the signed segment-reduction kernel        */
#define NGRAM_PROF_STEP 3   /* the fused sparse step (and window reset)   */
#define NGRAM_PROF_STASH 4  /* burst mode: keeping a micro-step           */
#define NGRAM_PROF_GROUPS 5

/* Measurement hook for benchmarks and profilers: until changed, every call
 * made by this host thread that launches kernels of `group` records
 * `start_event` at the start of that group's first kernel and `stop_event` at
 * the end of its last one (both are hipEvent_t; NULL stops recording).  The
 * events are attached to those kernels' own dispatches on the call's stream
 * (hipExtLaunchKernelGGL), so recording them adds no work to the stream.
 * Thread-local; never used by the library itself. */
int ngram_profile_events(int group, void *start_event, void *stop_event);

/* Synchronises `stream` and writes the sticky device flags to the host word
 * `flags`; clears them if `clear` is nonzero.  Not for use under capture. */
int ngram_device_status(const ngram_config *cfg, const void *ws,
                        uint32_t *flags, int clear, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NGRAM_H */
