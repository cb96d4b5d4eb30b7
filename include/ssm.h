/*
 * ssm.h -- C ABI of the sampled-softmax training loss, for AMD Instinct
 * MI355X (gfx950).  Built into the same libngram.so as ngram.h.
 *
 * The method: for most of training the loss scores only a subset of the
 * vocabulary; a vocabulary entry that does not occur in the batch has its
 * lm_head forward and backward skipped part of the time (the @classiclarryd
 * post quoted on the airebao.com item about the 39.9 s record).  The subset is
 * shared and has a fixed size per phase: 10,240, then 14,336, then 24,576
 * entries, and all 50,304 for the last steps (agentic-affairs.com, "NanoGPT
 * Training Record", Key Optimizations and Ablation Table Results, and
 * Technical Architecture and Implementation Details):
 *
 *   candidate set S, |S| = C:  every id occurring among the targets
 *                              (ascending), then ids that do not occur, in
 *                              the order of a caller-given random
 *                              permutation of [0, V), until |S| = C
 *   z[i][c]   = X[i] . W[S[c]]                          (fp32 from bf16)
 *   loss[i]   = log sum_c exp(z[i][c]) - z[i][slot[i]]  (S[slot[i]] = y[i])
 *   dz[i][c]  = g[i] (exp(z[i][c] - lse[i]) - [c == slot[i]])
 *   dX        = dz W_S;    dW[S[c]] += (dz^T X)[c]      (other rows untouched)
 *
 * Readings of what the pages leave open (the CPU oracle shares them): the
 * fill order above; no bias, scale, cap or sampling correction on the logits;
 * a per-position upstream gradient g (1/T for a mean loss).  Precision: X and
 * W are bf16; the three contractions run on bf16 matrix cores with fp32
 * accumulation; between the forward and the backward each logit is kept as
 * exp(z - M) in fp16 (nearest even; M the largest logit of its row among
 * the 192 candidates of its forward tile, so the kept value lies in (0, 1]);
 * dz is rounded to bf16 (nearest even) before the two backward
 * contractions; lse, loss, dX and dW are fp32.
 *
 * Conventions: device pointers unless marked "host"; the caller owns every
 * buffer; ssm_candidates, ssm_loss_fwd and ssm_loss_bwd only enqueue on
 * `stream` (a hipStream_t, NULL = the null stream) and never allocate, free or
 * synchronise; a negative return is a host-detected error with nothing
 * enqueued.  Row-major [rows][768] activations and tables, 16-byte aligned.
 * Calls on one workspace must be ordered (one stream).
 */
#ifndef SSM_H
#define SSM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 2

#define SSM_OK 0
#define SSM_ENULL -1    /* a required pointer is NULL                          */
#define SSM_EALIGN -2   /* a pointer is not 16-byte (workspace: 256-byte) aligned */
#define SSM_ECONFIG -3  /* dim != 768, vocab < 1, C outside [1, vocab], or
                           max_tokens outside [1, 2^24]                       */
#define SSM_ESIZE -4    /* T outside [0, max_tokens] or a workspace too small  */
#define SSM_EARG -5     /* a scalar argument is out of range                  */
#define SSM_EHIP -6     /* the HIP runtime reported an error                  */

/* sticky device flags (ssm_device_status) */
#define SSM_FLAG_BAD_TARGET 0x1u  /* a target id outside [0, vocab)          */
#define SSM_FLAG_OVERFLOW 0x2u    /* more distinct targets than C            */
#define SSM_FLAG_BAD_PERM 0x4u    /* perm is not a permutation of [0, vocab) */
#define SSM_FLAG_BAD_CAND 0x8u    /* a candidate id outside [0, vocab): row 0
                                     was read in its place                   */
#define SSM_FLAG_BAD_SLOT 0x10u   /* a slot outside [0, C): that position's
                                     loss is NaN and its one-hot term absent */
#define SSM_FLAG_NO_LOGITS 0x20u  /* ssm_loss_bwd found no logits stored by an
                                     ssm_loss_fwd of the same T since the last
                                     ssm_candidates: gradients are zero      */

/* kernel groups for ssm_profile_events */
#define SSM_PROF_CAND 0   /* the candidate-set kernels                        */
#define SSM_PROF_FWD 1    /* forward contraction + per-tile softmax sums      */
#define SSM_PROF_LSE 2    /* per-position log-sum-exp and loss                */
#define SSM_PROF_TRANS 3  /* the backward's operand transposes                */
#define SSM_PROF_DZ 4     /* stored logits -> dz (bf16)                       */
#define SSM_PROF_DX 5     /* dX = dz W_S                                      */
#define SSM_PROF_DW 6     /* dW[S] += dz^T X                                  */
#define SSM_PROF_GROUPS 7

typedef struct ssm_config {
    int32_t vocab;       /* V: ids are valid in [0, V); 50304 in the speedrun */
    int32_t dim;         /* D: must be 768                                     */
    int32_t candidates;  /* C in [1, V]: 10240, 14336, 24576 or 50304 there   */
    int32_t reserved;    /* must be 0                                          */
    int64_t max_tokens;  /* largest T of any call on a workspace              */
} ssm_config;

int ssm_abi_version(void);
const char *ssm_status_string(int status);

/* Workspace size for cfg (host).  About 2 (T+128)(C+128) bytes for what the
 * forward keeps of its logits, 2 (T+128)(C+128) for dz, 16 D (C+128) for dW's
 * split parts, plus 2 D (T + C + 256) bytes of transposed operands and
 * 8 T C/128 bytes of per-tile sums (about 2.3 GB at T = 49,152,
 * C = 10,240). */
int ssm_workspace_bytes(const ssm_config *cfg, uint64_t *bytes);

/* Prepares a workspace (256-byte aligned, ws_bytes from ssm_workspace_bytes)
 * and clears its flags.  Enqueued on stream. */
int ssm_workspace_init(const ssm_config *cfg, void *ws, uint64_t ws_bytes, void *stream);

/* Candidate set of one batch (the reading above).
 *   targets: int32 [T] next-token ids; perm: int32 [V], a permutation of
 *   [0, V) drawn by the caller (the method's randomness, passed in);
 *   cand: int32 [C] out; slot: int32 [T] out, cand[slot[i]] == targets[i].
 * Device faults: an id outside [0, V) (BAD_TARGET), more than C distinct
 * targets (OVERFLOW) or a perm that is not a permutation (BAD_PERM) mark the
 * batch void: cand and slot still hold in-range values, and the next
 * ssm_loss_fwd / ssm_loss_bwd on this workspace write NaN losses and zero
 * gradients.  T = 0 enqueues nothing. */
int ssm_candidates(const ssm_config *cfg, void *ws, const int32_t *targets, int64_t T,
                   const int32_t *perm, int32_t *cand, int32_t *slot, void *stream);

/* Forward: loss and lse (fp32 [T] each) of every position over the
 * candidate set.  X: bf16 [T][768]; W: bf16 [V][768] (the lm_head);
 * cand, slot as from ssm_candidates.  The logits, kept as fp16 exp(z - M)
 * (see Precision above), stay in the workspace for ssm_loss_bwd.  T = 0
 * enqueues nothing. */
int ssm_loss_fwd(const ssm_config *cfg, void *ws, const void *X, const void *W,
                 const int32_t *cand, const int32_t *slot, int64_t T, float *loss,
                 float *lse, void *stream);

/* Backward: dX = dz W_S (fp32 [T][768], overwritten) and dW[cand[c]] +=
 * (dz^T X)[c] (fp32 [V][768]; rows outside the candidate set are not
 * touched).  lse: the forward's; dloss: fp32 [T], the upstream gradient g.
 * dz comes from the logits the last ssm_loss_fwd on this workspace stored:
 * call it after that forward with the same X, W, cand, slot and T (the
 * library checks T and that no ssm_candidates came between, see
 * SSM_FLAG_NO_LOGITS; X and W are the caller's to keep).  dX must not
 * overlap X or dW. */
int ssm_loss_bwd(const ssm_config *cfg, void *ws, const void *X, const void *W,
                 const int32_t *cand, const int32_t *slot, const float *lse,
                 const float *dloss, int64_t T, float *dX, float *dW, void *stream);

/* Reads the sticky flags (host *flags); synchronises the stream.  With
 * clear != 0 the flags are reset afterwards. */
int ssm_device_status(const ssm_config *cfg, const void *ws, uint32_t *flags, int clear,
                      void *stream);

/* Measurement hook (thread-local): raw hipEvent_t start/stop to be recorded
 * around the first and last kernel of `group` on the next calls; NULL
 * detaches. */
int ssm_profile_events(int group, void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
