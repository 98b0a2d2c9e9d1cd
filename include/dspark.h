/*
 * dspark.h -- C ABI of the fused DSpark draft-training loss for AMD gfx950.
 *
 * What is computed (the pages, cited by title and section):
 *   Megatron-Bridge API page "bridge.training.post_training.dspark.loss",
 *   module docstring and `dspark_loss`: the draft's loss sums three terms,
 *   each weighted by slot position -- cross-entropy against the teacher-forced next
 *   token, the raw probability L1 ||p_draft - p_target||_1 (no 1/2), and a
 *   confidence BCE against the label 1 - 0.5 * L1 -- each scaled by the slot
 *   weight exp(-k / loss_decay_gamma); the acceptance accept = 1 - 0.5 * L1 and
 *   tau = sum_k cumprod(accept)_k + 1.  The loss is an unnormalised numerator,
 *   returned with the supervised token count and [numerator, denominator]
 *   report pairs (section "Return contract").
 *   NeMo-RL design doc "DSpark Auxiliary Heads": the draft logits are first
 *   corrected by the Markov head, bias = markov_w2 . markov_w1[prev_id] on
 *   valid slots ("Inputs and Outputs"); the confidence head is a linear
 *   projection of [hidden ; markov embedding] plus a bias ("Checkpoint
 *   Contract" shapes).  TorchSpec pull request #132, PR description: the
 *   teacher is the target lm_head applied to the target's final hidden state.
 *
 * Conventions shared by every entry point:
 *   - R = batch * num_blocks * block_size rows, in (b, n, k) order; the vocab
 *     axis is innermost.  All tensors are dense row-major.
 *   - Every pointer in the structs below is DEVICE memory owned by the caller.
 *     The library allocates nothing and keeps no pointer after a call returns.
 *   - Every device pointer must be 16-byte aligned (DSPARK_ERR_ALIGN).
 *   - Validation is on the host and synchronous; after it the work is enqueued
 *     on `stream` (a hipStream_t; NULL = the legacy default stream) and the
 *     call returns without synchronising.  Data-dependent problems (ids out of
 *     range on a supervised slot, a non-finite loss term) set bits in the
 *     device word `flags` instead of failing.
 *   - Supervised slot mask m = block_keep_mask[b,n] * cumprod_k(eval_mask != 0)
 *     (API page, `DSparkForwardOutput.eval_mask`: a block supervises a
 *     contiguous prefix; TorchSpec #132: realised as a cumprod).  Rows with
 *     m = 0 are never read beyond their mask and ids: NaN/Inf there changes
 *     nothing (Megatron-Bridge PR #5241, merge note: scrub before reducing).
 *   - Calls on one workspace must not overlap; distinct workspaces are
 *     independent.  dspark_loss_bwd must follow dspark_loss_fwd on the same
 *     workspace, same stream order, with the inputs unchanged.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t, passed as an opaque pointer so this header needs no HIP headers. */
typedef void *dspark_stream_t;

/* Element types of the float inputs / of the draft-logit gradient. */
enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 };

/* Status codes (0 = success).  dspark_status_string() describes each. */
enum {
  DSPARK_OK = 0,
  DSPARK_ERR_NULL = -1,       /* a pointer the call needs is NULL */
  DSPARK_ERR_SHAPE = -2,      /* a dimension is <= 0, not a multiple of 8 where required, or inconsistent */
  DSPARK_ERR_DTYPE = -3,      /* dtype / grad_dtype not DSPARK_F32 or DSPARK_BF16 */
  DSPARK_ERR_NO_TARGET = -4,  /* L1 term or confidence head requested without a teacher */
  DSPARK_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than dspark_workspace_size() */
  DSPARK_ERR_ALIGN = -6,      /* a device pointer is not 16-byte aligned */
  DSPARK_ERR_HIP = -7,        /* a HIP launch failed; see dspark_last_hip_error() */
  DSPARK_ERR_SCRATCH = -8     /* the problem needs more than the no-allocation entry point's scratch */
};

/* Bits of dspark_shape.options; an unknown bit makes the shape invalid
 * (DSPARK_ERR_SHAPE, workspace size 0). */
enum {
  /* By default, for bf16 inputs with markov_rank in {32, 64, 128, 256}, R and
   * Vd multiples of 32 and Vd < 2^24, the fp32 Markov-corrected draft logits
   * z + W2 W1[prev] are never stored: each vocabulary sweep (softmax
   * statistics, L1, gradient) recomputes the rank-r bias from W2 and the
   * gathered W1 rows on bf16 MFMA.  This bit instead materialises them once
   * (a GEMM epilogue) in the workspace, 4 R Vd bytes more, and sweeps the
   * stored values: slower on MI355X at the shapes measured, kept for
   * comparison.  Ignored where the default does not apply (fp32 inputs, other
   * ranks: the logits are always stored there) and without a Markov head
   * (the sweeps read z directly). */
  DSPARK_OPT_STORE_DRAFT_LOGITS = 1u,
  /* dspark_loss_bwd's d_markov_w1 (and dspark_shard_bwd_finish's): by default
   * the rows' embedding gradients are scattered with fp32 atomics, so the
   * order of the additions, and the last bits of rows that several slots
   * share, vary from run to run.  This bit adds them as 64-bit fixed-point
   * integers instead (scale from the largest term; each term rounded once to
   * far below a float ulp of the sums), which makes d_markov_w1 bitwise
   * reproducible; workspace + 8 Vt r bytes.  With a non-finite term the
   * gradient falls back to the fp32 atomics (the forward flags the loss). */
  DSPARK_OPT_DETERMINISTIC = 2u
};

/* Bits of the device word dspark_fwd_out.flags (OR-ed, never cleared by bwd). */
enum {
  DSPARK_FLAG_TARGET_ID_RANGE = 1u, /* a supervised slot has target id outside [0, draft_vocab) */
  DSPARK_FLAG_PREV_ID_RANGE = 2u,   /* a supervised slot has prev id outside [0, target_vocab) */
  DSPARK_FLAG_NONFINITE = 4u,       /* a supervised slot produced a non-finite loss term */
  DSPARK_FLAG_NO_TEACHER = 8u       /* CE-only call: L1 is zero by definition, so accept = 1 */
};

typedef struct {
  int64_t batch;          /* B */
  int64_t num_blocks;     /* N: anchor blocks drawn per sequence */
  int64_t block_size;     /* K: draft positions per anchor */
  int64_t draft_vocab;    /* Vd: logits, L1 and target ids live here; multiple of 8 */
  int64_t target_vocab;   /* Vt: rows of markov_w1, range of prev ids (may differ from Vd) */
  int64_t hidden;         /* H: inner size of lm_head / target_hidden; multiple of 8 (0 if unused) */
  int64_t conf_hidden;    /* Hd: confidence-head hidden size; 0 = no confidence head */
  int64_t markov_rank;    /* r: multiple of 8; 0 = no Markov head */
  int32_t with_markov_conf; /* 1: confidence input is [hidden ; markov embedding] (proj [1, Hd + r]) */
  int32_t dtype;          /* DSPARK_F32 or DSPARK_BF16: type of every float input */
  int32_t grad_dtype;     /* type written to d_draft_logits */
  int32_t options;        /* DSPARK_OPT_* bits (0 = defaults); fwd and bwd must pass the same */
} dspark_shape;

/* `dspark_loss` keyword arguments (API page, defaults 0.1 / 0.9 / 1.0 / 4.0). */
typedef struct {
  float ce_alpha;
  float l1_alpha;          /* weight of the RAW L1 (no 1/2) */
  float confidence_alpha;
  float loss_decay_gamma;  /* <= 0 disables the decay (the page's None) */
} dspark_hparams;

/* Forward inputs; shapes use R = B*N*K.  Pointers not needed by the shape may be NULL. */
typedef struct {
  const void *draft_logits;          /* [R, Vd] dtype, required */
  const int32_t *target_ids;         /* [R], required; read on supervised slots only */
  const uint8_t *eval_mask;          /* [R] nonzero = loss-enabled, required */
  const uint8_t *block_keep_mask;    /* [B*N] nonzero = kept, or NULL = all kept */
  const int32_t *prev_ids;           /* [R] ids into markov_w1 rows; required when r > 0 */
  const void *markov_w1;             /* [Vt, r] dtype (markov_head.markov_w1.weight) */
  const void *markov_w2;             /* [Vd, r] dtype (markov_head.markov_w2.weight) */
  const void *target_hidden;         /* [R, H] dtype, target final hidden AFTER its final norm */
  const void *lm_head;               /* [Vd, H] dtype, target lm_head rows of the draft vocab */
  const void *aligned_target_logits; /* [R, Vd] dtype: teacher logits given directly (wins over the two above) */
  const void *conf_hidden;           /* [R, Hd] dtype: confidence-head hidden input */
  const void *conf_w;                /* [1, Hd (+ r)] dtype (confidence_head.proj.weight) */
  const void *conf_b;                /* [1] dtype (confidence_head.proj.bias) */
} dspark_inputs;

typedef struct {
  double *loss;          /* [1] unnormalised weighted numerator (required) */
  int64_t *num_tokens;   /* [1] supervised slot count (required) */
  double *pairs;         /* [10] (num, den) x {ce, l1, confidence, accept rate, tau}; every
                            den is an exact integer (required) */
  float *accept_rate;    /* [R] per-slot accept, 1 on unsupervised slots, or NULL */
  float *row_terms;      /* [R, 4] (ce, l1, bce, confidence logit) per slot, 0 when unsupervised, or NULL */
  uint32_t *flags;       /* [1] DSPARK_FLAG_* bits, OR-ed in (required; caller zeroes it) */
} dspark_fwd_out;

typedef struct {
  void *d_draft_logits;  /* [R, Vd] grad_dtype, required; 0 on unsupervised slots */
  float *d_markov_w1;    /* [Vt, r], required when r > 0 */
  float *d_markov_w2;    /* [Vd, r], required when r > 0 */
  float *d_conf_w;       /* [1, Hd (+ r)], required with a confidence head */
  float *d_conf_b;       /* [1], required with a confidence head */
  float *d_conf_hidden;  /* [R, Hd] or NULL */
} dspark_bwd_out;

/* Bytes of device workspace fwd + bwd need for `shape` (0 on an invalid shape).
 * It holds the fp32 teacher logits, the fp32 Markov-corrected draft logits
 * where they are stored (see DSPARK_OPT_STORE_DRAFT_LOGITS), per-tile softmax
 * statistics, per-row state and the backward scratch. */
size_t dspark_workspace_size(const dspark_shape *shape);

/* Forward: loss numerator, token count, report pairs, optional per-row terms.
 * Teacher: aligned_target_logits if non-NULL, else target_hidden x lm_head^T
 * if both are non-NULL (and H > 0), else none -- then only CE is allowed
 * (l1_alpha == 0 and no confidence head, else DSPARK_ERR_NO_TARGET), the L1
 * output is zeros (API page, `_ce_and_l1_per_token`) and FLAG_NO_TEACHER is set.
 * The workspace must stay untouched until the matching dspark_loss_bwd. */
int dspark_loss_fwd(const dspark_shape *shape, const dspark_hparams *hp, const dspark_inputs *in,
                    void *workspace, size_t workspace_bytes, dspark_fwd_out *out,
                    dspark_stream_t stream);

/* Backward of `loss` with upstream gradient `grad_scale` (Megatron-Core scales
 * by 1 / global num_tokens).  Outputs are overwritten, not accumulated.  The
 * teacher gets no gradient (API page: the teacher arrives detached), and
 * the BCE label is treated as a constant.  With bf16 inputs the Markov weight
 * gradients contract the logit gradient G at the precision of d_draft_logits:
 * grad_dtype bf16 -> the bf16 G that is written out (as a bf16 autograd would;
 * about 2^-10 normwise, like dz itself; R and Vd multiples of 32), grad_dtype
 * fp32 -> G as bf16 high + low parts (about 2^-18). */
int dspark_loss_bwd(const dspark_shape *shape, const dspark_hparams *hp, const dspark_inputs *in,
                    void *workspace, size_t workspace_bytes, float grad_scale,
                    dspark_bwd_out *out, dspark_stream_t stream);

/* Acceptance report alone (API page, `_acceptance_report`): from per-slot
 * accept rates [R] (fp32), eval_mask [R] and block_keep_mask [B*N] (or NULL),
 * writes out4 = {sum m*accept, sum m, sum over kept blocks of
 * (1 + sum_k prod_{j<=k} m_j accept_j), number of kept blocks} as doubles. */
int dspark_accept_report(int64_t batch, int64_t num_blocks, int64_t block_size,
                         const float *accept_rate, const uint8_t *eval_mask,
                         const uint8_t *block_keep_mask, double *out4, dspark_stream_t stream);

/* ---- standalone head ops (draft time) ---------------------------------------
 * The two auxiliary heads of the NeMo-RL design doc "DSpark Auxiliary Heads"
 * ("Inputs and Outputs", "Checkpoint Contract") outside the loss, with the
 * loss's own kernels and parameter layouts.  All pointers are device memory;
 * rows are [rows, ...] row-major; dtype (DSPARK_F32 / DSPARK_BF16) is the type
 * of every float input; outputs are fp32 and overwritten.  valid_mask [rows]
 * (nonzero = valid slot) may be NULL (every slot valid); both ops return zero
 * on invalid slots.  prev_ids [rows] index markov_w1 [target_vocab,
 * markov_rank]; an id outside [0, target_vocab) on a valid slot gives a zero
 * embedding (the loss flags it; these ops do not).
 * Errors: DSPARK_ERR_NULL, _SHAPE (a size < 0, a vocabulary or rank that is not
 * a multiple of 8, draft_hidden < 1), _DTYPE, _ALIGN (16 bytes),
 * _WORKSPACE, _HIP.  Asynchronous on `stream`. */

/* Bytes of workspace dspark_markov_logits needs (the gathered embeddings and
 * the per-tile statistics the projection kernel writes where the op takes it
 * instead of the sweep engine: fp32 inputs, or a rank outside {0, 32, 64,
 * 128, 256}, or a vocabulary from 2^24 on). */
size_t dspark_markov_logits_workspace_size(int64_t rows, int64_t draft_vocab,
                                           int64_t markov_rank, int32_t dtype);

/* Markov head: out [rows, draft_vocab] fp32 = z + W2 W1[prev] on valid slots
 * and 0 on the others ([HEADS] "Inputs and Outputs": the bias applies only
 * where a slot is valid, and each head outputs zeros elsewhere; TorchSpec pull
 * request #132, "Testing": bias == W2(W1[prev])).  markov_rank 0: out = z on
 * valid slots.  z is draft_logits [rows, draft_vocab]. */
int dspark_markov_logits(int64_t rows, int64_t draft_vocab, int64_t target_vocab,
                         int64_t markov_rank, int32_t dtype, const void *draft_logits,
                         const int32_t *prev_ids, const uint8_t *valid_mask,
                         const void *markov_w1, const void *markov_w2, float *out,
                         void *workspace, size_t workspace_bytes, dspark_stream_t stream);

/* Confidence head: out [rows] fp32 = W_c . [h ; e] + b on valid slots and 0
 * on the others, with h = draft_hidden [rows, draft_hidden] and, when
 * with_markov_conf, e = W1[prev]; conf_w is [1, draft_hidden (+ markov_rank)],
 * conf_b [1] ([HEADS] "Checkpoint Contract"; concatenation order [hidden ;
 * embedding]).  With the loss's effective mask as valid_mask this is the
 * loss's own confidence logit, bit for bit.  workspace: at least
 * dspark_confidence_logits_workspace_size() bytes (0 without Markov features,
 * then it may be NULL). */
size_t dspark_confidence_logits_workspace_size(int64_t rows, int64_t markov_rank,
                                               int32_t with_markov_conf, int32_t dtype);
int dspark_confidence_logits(int64_t rows, int64_t draft_hidden, int64_t target_vocab,
                             int64_t markov_rank, int32_t with_markov_conf, int32_t dtype,
                             const void *hidden, const int32_t *prev_ids,
                             const uint8_t *valid_mask, const void *markov_w1,
                             const void *conf_w, const void *conf_b, float *out,
                             void *workspace, size_t workspace_bytes, dspark_stream_t stream);

/* ---- no-allocation variant (for callers that cannot allocate) ---------------
 * For code under HIP graph capture, tight serving loops and harnesses that
 * forbid hipMalloc: dspark_confidence_logits with its workspace replaced by a
 * library-owned device array of DSPARK_NOALLOC_SCRATCH_BYTES per GPU (a
 * file-scope __device__ array, present on every GPU the library runs on until
 * the process ends; nothing is allocated or freed by the call).  Same
 * arguments, results and errors as dspark_confidence_logits without
 * workspace / workspace_bytes; a problem whose workspace
 * (dspark_confidence_logits_workspace_size) exceeds the scratch returns
 * DSPARK_ERR_SCRATCH (with bf16 and markov rank 256: up to about 32000 rows).
 * The stream must belong to the current device.  Every call on one GPU uses
 * that GPU's one scratch array (which keeps the last call's contents; no part
 * of it needs to start at zero): calls that overlap in time on one GPU --
 * concurrent streams, or host threads on one device -- race and must be
 * ordered by the caller. */
#define DSPARK_NOALLOC_SCRATCH_BYTES (16u << 20)
int dspark_confidence_logits_noalloc(int64_t rows, int64_t draft_hidden, int64_t target_vocab,
                                     int64_t markov_rank, int32_t with_markov_conf, int32_t dtype,
                                     const void *hidden, const int32_t *prev_ids,
                                     const uint8_t *valid_mask, const void *markov_w1,
                                     const void *conf_w, const void *conf_b, float *out,
                                     dspark_stream_t stream);

/* ---- batch construction (the step before the loss) --------------------------
 * TorchSpec pull request #132, PR description: slot k of a block is labelled
 * by the token at anchor + k + 1 and every slot is supervised, the eval mask
 * is a running product over the block (so a prefix), the Markov head's
 * previous-token input starts from the anchor, and an anchor is drawn only
 * where both it and its first label are valid.  "Valid" is the loss mask here: an anchor a is kept when
 * 0 <= a, a + 1 < seq_len and loss_mask[a], loss_mask[a + 1] are nonzero.
 * Inputs: input_ids [batch, seq_len] int32, loss_mask [batch, seq_len] (nonzero
 * = supervised position), anchors [batch, num_blocks] int32 (the caller's
 * random draws, e.g. from anchor_ok).  Outputs for row r = (b num_blocks + n)
 * block_size + k: target_ids[r] = input_ids[b, a + k + 1], prev_ids[r] =
 * input_ids[b, a + k] (0 past the end of the sequence), eval_mask[r] = product
 * of loss_mask over positions a + 1 .. a + k + 1 (0 past the end);
 * block_keep[b num_blocks + n]; a dropped block's rows are all 0.
 * anchor_ok [batch, seq_len] (may be NULL): 1 where an anchor may be drawn.
 * The outputs feed dspark_loss_fwd directly.  Errors: DSPARK_ERR_NULL,
 * _SHAPE (a size < 1 or beyond 2^31 rows), _HIP.  Asynchronous on `stream`. */
int dspark_build_blocks(int64_t batch, int64_t seq_len, int64_t num_blocks, int64_t block_size,
                        const int32_t *input_ids, const uint8_t *loss_mask,
                        const int32_t *anchors, int32_t *target_ids, int32_t *prev_ids,
                        uint8_t *eval_mask, uint8_t *block_keep, uint8_t *anchor_ok,
                        dspark_stream_t stream);

/* ---- vocabulary shards (tensor-parallel split of the draft vocabulary) -----
 * NeMo-RL "DSpark Auxiliary Heads" (Markov head) and the loss section of the
 * DSpark page: every vocabulary term of the loss is a sum over columns, and a
 * softmax's log-sum-exp is the log-sum-exp of per-part log-sum-exps, so a
 * caller holding columns [v0, v0 + draft_vocab) of draft_logits,
 * aligned_target_logits / lm_head and markov_w2 computes partials that merge
 * into the unsplit loss exactly (up to rounding).  `shape` describes the
 * shard: draft_vocab is the shard's width; target_ids are shard-local
 * (global id - v0), so an id outside [0, draft_vocab) belongs to another
 * shard (each supervised target must fall in exactly one shard).  Every other
 * input (masks, prev_ids, markov_w1, confidence head) is the same on every
 * shard.  The shape must take the bias sweeps: bf16, markov_rank in
 * {0, 32, 64, 128, 256}, R and draft_vocab multiples of 32 with a Markov head,
 * options without DSPARK_OPT_STORE_DRAFT_LOGITS; else DSPARK_ERR_SHAPE.  The
 * workspace is dspark_workspace_size(shape), one per shard, kept from the
 * first call to the last.  Order per step, with the collectives between:
 *   shard_fwd_stats -> lse parts [G, R, 2] gathered -> shard_merge_lse ->
 *   shard_fwd_terms -> terms [R, 4] summed over shards -> shard_fwd_finish ->
 *   shard_bwd -> d_embed [R, r] summed over shards -> shard_bwd_finish.
 * Asynchronous on `stream`; errors as dspark_loss_fwd. */

/* Step 1: prep rows, E = W1[prev], the shard's teacher logits and per-tile
 * statistics, then lse_part [R, 2] fp32 = (log-sum-exp of z' = z + E W2^T,
 * of T) over the shard's columns; -inf on unsupervised rows and for T without
 * a teacher.  flags [1] as in dspark_fwd_out (the target-id range is not
 * checked: shard-local ids leave it legitimately). */
int dspark_shard_fwd_stats(const dspark_shape *shape, const dspark_hparams *hp,
                           const dspark_inputs *in, void *workspace, size_t workspace_bytes,
                           float *lse_part, uint32_t *flags, dspark_stream_t stream);

/* lse [rows, 2] = log-sum-exp over the `shards` parts of lse_parts
 * [shards, rows, 2] (fp64 inside, -inf when every part is -inf).  Errors:
 * DSPARK_ERR_SHAPE (shards < 1 or > 65536, rows < 0 or >= 2^31), _NULL, _HIP. */
int dspark_shard_merge_lse(int64_t shards, int64_t rows, const float *lse_parts, float *lse,
                           dspark_stream_t stream);

/* Step 2: with the merged lse [R, 2], terms [R, 4] fp64 = this shard's
 * (sum |p - q|, sum p sign(p - q), z'_y if the shard owns the target else 0,
 * 1 if it owns the target else 0) on supervised rows, zeros elsewhere.  The
 * sum over shards is the row's (L1, S, z'_y, number of owners). */
int dspark_shard_fwd_terms(const dspark_shape *shape, const dspark_hparams *hp,
                           const dspark_inputs *in, void *workspace, size_t workspace_bytes,
                           const float *lse, double *terms, dspark_stream_t stream);

/* Step 3: from the shard-summed terms [R, 4], CE = lse_z - z'_y, the
 * confidence head and the reductions: `out` as dspark_loss_fwd (identical on
 * every shard); DSPARK_FLAG_TARGET_ID_RANGE where a supervised row's target
 * has not exactly one owner (a global id outside the vocabulary). */
int dspark_shard_fwd_finish(const dspark_shape *shape, const dspark_hparams *hp,
                            const dspark_inputs *in, void *workspace, size_t workspace_bytes,
                            const double *terms, dspark_fwd_out *out, dspark_stream_t stream);

/* Step 4: the shard's gradients: d_draft_logits [R, draft_vocab] (grad_dtype),
 * d_markov_w2 [draft_vocab, r] (the shard's rows of W2's gradient) and
 * d_embed [R, r] fp32 = the shard's G . W2 term of dloss/dE (0 on unsupervised
 * rows).  d_markov_w2 and d_embed are required when r > 0. */
int dspark_shard_bwd(const dspark_shape *shape, const dspark_hparams *hp, const dspark_inputs *in,
                     void *workspace, size_t workspace_bytes, float grad_scale,
                     void *d_draft_logits, float *d_markov_w2, float *d_embed,
                     dspark_stream_t stream);

/* Step 5: from d_embed summed over the shards, the replicated gradients into
 * out->d_markov_w1, d_conf_w, d_conf_b, d_conf_hidden (as dspark_loss_bwd;
 * out->d_draft_logits and d_markov_w2 are not touched). */
int dspark_shard_bwd_finish(const dspark_shape *shape, const dspark_hparams *hp,
                            const dspark_inputs *in, void *workspace, size_t workspace_bytes,
                            float grad_scale, const float *d_embed, dspark_bwd_out *out,
                            dspark_stream_t stream);

const char *dspark_status_string(int status);
const char *dspark_last_hip_error(void);

/* ---- per-stage GPU timers (a tracing aid; off by default) -------------------
 * When enabled, every fwd / bwd call records a pair of HIP events around each
 * of its stages on the call's stream (adds two event records per stage).
 * dspark_profile_read() waits for all recorded events, adds their elapsed
 * times to per-stage totals, and copies min(n, stage count) totals (ms) and
 * launch counts out; it returns the number of stages.  Enabling or disabling
 * clears the totals.  Process-wide, guarded by a mutex. */
int dspark_profile_enable(int on);
int dspark_profile_read(double *ms, int64_t *counts, int n);
const char *dspark_stage_name(int stage);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
