/*
 * grpo_head.h - C ABI of the fused LM-head GRPO / GSPO loss for MI355X (gfx950).
 *
 * What it computes.  For hidden states H [N, D] and an LM-head weight W [V_r, D]
 * (nn.Linear layout, rows >= V are vocabulary padding), z = H W^T / tau over the
 * real vocabulary [0, V).  The forward returns each token's selected log-prob
 * log p(y_t) = z[t, y_t] - LSE_v z[t, :] without ever storing the [N, V] logits:
 * vocabulary tiles are streamed, each tile leaves a per-token (max, sumexp)
 * partial, and the partials are folded from the identity (-inf, 0) in one fixed
 * order: the tiles split into 8 consecutive runs, each run folded in ascending tile
 * order, then the 8 run results folded in ascending run order (the same order for
 * every call and every shard count, so results are bitwise repeatable; it differs
 * from one left-to-right fold only in fp32 rounding).  It then applies the
 * clipped-ratio objective and reduces it to
 * (loss, policy_loss, kl), and writes the per-token coefficient d loss / d logp_t.
 * The backward recomputes each logit tile, forms
 * dlogits = grad_output * coef_t * (onehot(y_t) - softmax) / tau, and contracts it
 * into dH = dlogits W and dW = dlogits^T H.
 *
 * Sources (page title, section):
 *   - streaming over the vocabulary so only selected-token log-probs are computed,
 *     behind a fused-linear API (hidden states and head weight in, loss out):
 *     Liger-Kernel PR #1160 "[GRPO] add chunked grpo streaming over vocab", Summary.
 *   - padded versus real vocabulary; padded columns masked to -inf before the
 *     per-tile partials; fp32 (max, sumexp) merge in a fixed global tile order and
 *     the (-inf, 0) identity; an explicit active mask or ignore_index, inactive
 *     targets that need not hold ignore_index; fp32 log-prob and LSE outputs:
 *     RL-Kernel PR #291 "Add deterministic DP-aware GRPO loss on the TP-aware
 *     logprob path", commit notes (ShardingSpec, MaskSpec / MaskMode, ReductionSpec,
 *     LogprobOutputSpec).
 *   - the objective is elementwise per token / per sequence; token normalisers
 *     global_active_tokens (masked mean) and per_sequence_then_mean; the
 *     (loss, policy_loss, kl) result; a validation flag that costs a device sync;
 *     no division by zero for a batch with no active token; fail loudly, never a
 *     silent fallback: same page, Overview / Key Changes, commit notes and the
 *     review threads on validation syncs and the zero-active-token guard.
 *   - GSPO: per-token contributions aggregated per segment (index_add), then the
 *     loss, the new_logprobs metric and the unscaled per-token backward
 *     coefficient, with the divisor and grad_output supplied at run time:
 *     Fast-LLM PR #554 "Fuse the GSPO segment seam into compiled blocks", What.
 *   The clipped surrogate is the PPO form (Schulman et al. 2017, eq. 7) with
 *   separate bounds 1 - eps_low and 1 + eps_high; the KL term is the k3 estimator
 *   exp(q - l) - (q - l) - 1 with l = logp, q = ref_logp; the GSPO ratio is
 *   exp of the segment's mean log-ratio (Zheng et al. 2025, eq. 7).
 *
 * Conventions for every entry point.
 *   - Pointers named as buffers are DEVICE pointers on the current HIP device,
 *     except `p` (a host pointer to the parameter block).  The caller owns every
 *     buffer; the library never allocates or frees device memory, keeps no state
 *     between calls and enqueues all work on `stream` (a hipStream_t; NULL is the
 *     null stream).  Calls return as soon as the work is enqueued, unless
 *     p->validate is set.
 *   - Arguments are checked on the host before anything is enqueued; a rejected
 *     call enqueues nothing.  The return value is a grpo_head_status; on a
 *     non-zero status grpo_head_last_error() describes it.
 *   - Results are bitwise identical from run to run for identical inputs: every
 *     reduction has a fixed order and no result depends on atomics (atomic
 *     counters in the workspace only decide which workgroup computes a tile; each
 *     tile is computed whole, in a fixed order).
 *   - Calls that share a workspace must not overlap in time.
 *
 * Layouts.  Row-major, no padding between rows.
 *   H [n_tokens][d_model] and W [v_rows][d_model]: bf16 or fp32 (p->dtype).
 *   y [n_tokens] int64 target ids; mask [n_tokens] uint8 (0 = inactive) or NULL;
 *   sid [n_tokens] int32 sequence / segment id, non-decreasing, in [0, n_seqs);
 *   adv [n_seqs] fp32 advantage per sequence / segment;
 *   old_logp, ref_logp, logp, lse, coef [n_tokens] fp32; counts [n_seqs] int32;
 *   out3 [3] fp32 = {loss, policy_loss, kl}; dH [n_tokens][d_model] and
 *   dW [v_rows][d_model] fp32, or bf16 with p->grad_dtype = GRPO_HEAD_GRAD_BF16.
 */
#ifndef GRPO_HEAD_H
#define GRPO_HEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum grpo_head_status {
  GRPO_HEAD_OK = 0,
  GRPO_HEAD_INVALID_ARGUMENT = 1,   /* null pointer, bad size, bad enum or scalar */
  GRPO_HEAD_WORKSPACE_TOO_SMALL = 2,/* ws_bytes < the matching *_workspace_size() */
  GRPO_HEAD_NO_ACTIVE_TOKENS = 3,   /* validate only: no token is active */
  GRPO_HEAD_TARGET_OUT_OF_RANGE = 4,/* validate only: an active target outside
                                       [0, v_real), or sid decreasing / outside
                                       [0, n_seqs) */
  GRPO_HEAD_NONFINITE = 5,          /* validate only: a non-finite lse, logp, input
                                       log-prob or loss */
  GRPO_HEAD_HIP_ERROR = 6           /* a HIP runtime call or launch failed */
} grpo_head_status;

enum { GRPO_HEAD_BF16 = 0, GRPO_HEAD_F32 = 1 };                  /* p->dtype */
enum { GRPO_HEAD_GRAD_F32 = 0, GRPO_HEAD_GRAD_BF16 = 1 };        /* p->grad_dtype */
enum { GRPO_HEAD_TOKEN_MEAN = 0, GRPO_HEAD_SEQUENCE_MEAN = 1,
       GRPO_HEAD_FIXED_CONSTANT = 2 };                          /* p->reduction */
enum { GRPO_HEAD_LEVEL_TOKEN = 0, GRPO_HEAD_LEVEL_SEQUENCE_GSPO = 1 }; /* p->level */

/* Parameter block, passed by host pointer.
 *   n_tokens     N >= 0.  N = 0 is an empty batch: outputs are written as zeros.
 *   d_model      D > 0, a multiple of 64.
 *   v_real       V >= 1: the real vocabulary; columns [V, v_rows) are padding and
 *                W rows there are never read (they may hold NaN).
 *   v_rows       V_r >= V: rows of W and dW.
 *   n_seqs       S >= 1 (S >= 0 when N = 0): sequences (token level) or packed
 *                segments (GSPO).
 *   ignore_index used only when mask is NULL: token t is active iff
 *                y[t] != ignore_index.  With a mask the mask alone decides and an
 *                inactive token's target is never read.
 *   chunk_tokens backward token-chunk size (rounded up to a multiple of 256);
 *                0 = all tokens in one chunk.  Sets the backward workspace size.
 *   dtype        GRPO_HEAD_BF16 or GRPO_HEAD_F32 (element type of H and W; the
 *                fp32 path keeps its dlogits in fp32, the bf16 path rounds them to
 *                bf16, nearest-even, before the two gradient products).
 *   reduction    token mean over active tokens (global_active_tokens), mean over
 *                sequences (that have an active token) of each sequence's token
 *                mean (per_sequence_then_mean), or the sum over active tokens
 *                divided by the caller's constant norm_const (fixed_constant, the
 *                Dr. GRPO normaliser): RL-Kernel PR #291 "Add deterministic
 *                DP-aware GRPO loss on the TP-aware logprob path", Key Changes
 *                (LossReductionSpec.token_normalizer).  GSPO always uses the
 *                sequence mean and rejects fixed_constant.
 *   level        token-level ratio (GRPO) or segment-level ratio (GSPO).
 *   validate     0: never synchronise.  1: synchronise `stream` once at the end of
 *                the call and check the conditions of statuses 3-5.
 *   inv_tau      1/temperature > 0, applied to the fp32 logit accumulator.
 *   eps_low, eps_high  clip bounds >= 0 (eps_low < 1): ratio clipped to
 *                [1 - eps_low, 1 + eps_high].
 *   beta         KL weight >= 0.  beta > 0 needs ref_logp.
 *   norm_const   fixed_constant only: the divisor C > 0 (finite); ignored otherwise.
 *                The pages name the normaliser without fixing C (Dr. GRPO, Liu et
 *                al. 2025, "Understanding R1-Zero-Like Training", divides by a
 *                constant generation budget).
 *                With fixed_constant a batch without active tokens is not an
 *                error even under validate (same page, review thread on the
 *                zero-active-token guard): the loss is then 0.
 *   accumulate_dw  0: grpo_head_bwd overwrites dW.  1: it adds this call's
 *                gradient to dW (rows [0, v_real); the padding rows are left
 *                as they are), e.g. across micro-batches.  dH is always
 *                overwritten.
 *   grad_dtype   element type of dH and dW: GRPO_HEAD_GRAD_F32 (0, the default)
 *                or GRPO_HEAD_GRAD_BF16 (rounded to nearest even once, after the
 *                fp32 accumulation; with several token chunks or accumulate_dw
 *                the running dW is read back, added in fp32 and rounded again).
 *   reserved     must be 0.
 */
typedef struct grpo_head_params {
  int64_t n_tokens;
  int64_t d_model;
  int64_t v_real;
  int64_t v_rows;
  int64_t n_seqs;
  int64_t ignore_index;
  int64_t chunk_tokens;
  int32_t dtype;
  int32_t reduction;
  int32_t level;
  int32_t validate;
  float inv_tau;
  float eps_low;
  float eps_high;
  float beta;
  float norm_const;
  int32_t accumulate_dw;
  int32_t grad_dtype;
  int32_t reserved;
} grpo_head_params;

/* Bytes of device workspace grpo_head_fwd needs (per-tile partials, target
 * logits, per-sequence totals, tile-queue counters).  0 if p is invalid. */
size_t grpo_head_fwd_workspace_size(const grpo_head_params* p);

/* Bytes of device workspace grpo_head_bwd needs (the bf16 or fp32 dlogits of one
 * token chunk over the 256-padded vocabulary, the chunk's gathered hidden states
 * as rows and transposed, per-token scalars and row indices, and tile-queue
 * counters); also at
 * least grpo_head_fwd_workspace_size(p), so one buffer serves all calls.
 * 0 if p is invalid. */
size_t grpo_head_workspace_size(const grpo_head_params* p);

/* Forward: selected log-prob, LSE, objective and per-token coefficient.
 *   logp[t] = z[t, y_t] - lse[t] for active tokens, 0 for inactive ones;
 *   lse[t]  = LSE over the real vocabulary, for every token;
 *   out3    = {loss, policy_loss, kl}; loss = policy_loss + beta * kl;
 *   coef[t] = d loss / d logp_t (0 for inactive tokens);
 *   counts[s] = number of active tokens of sequence s.
 * ref_logp may be NULL iff beta == 0 (kl is then 0).  old_logp and ref_logp are
 * read for active tokens only.  With level == GSPO the objective stage is the one
 * gspo_segment_reduce runs.
 * Status 0, 1, 2, 6; with validate also 3 (not with fixed_constant), 4, 5
 * (outputs are then still written, but may be meaningless).  With validate == 0
 * an active target outside [0, v_real) gives logp = NaN for that token, and an
 * invalid sid is clamped into [0, n_seqs); neither is reported. */
int grpo_head_fwd(const grpo_head_params* p, const void* H, const void* W, const int64_t* y,
                  const uint8_t* mask, const int32_t* sid, const float* adv,
                  const float* old_logp, const float* ref_logp, float* logp, float* lse,
                  float* out3, float* coef, int32_t* counts, void* ws, size_t ws_bytes,
                  void* stream);

/* Backward from the forward's lse and coef.
 *   dH[t, :] = sum_v G[t, v] W[v, :],  dW[v, :] = sum_t G[t, v] H[t, :] for v < V,
 *   dW[v, :] = 0 for V <= v < v_rows, with
 *   G[t, v] = grad_output * coef[t] * (1[v == y_t] - exp(z[t, v] - lse[t])) * inv_tau
 *   and G[t, :] = 0 for inactive tokens.
 * grad_output is a DEVICE pointer to one fp32 scalar, or NULL for 1.0.
 * dH is overwritten.  dW is overwritten, or with p->accumulate_dw the gradient
 * is added to it (rows [0, v_real) only; the padding rows are not touched).
 * Token chunks are processed in ascending order and dW accumulates them in that
 * order.  Within a chunk only the tokens with a non-zero scale
 * grad_output * coef[t] * inv_tau reach the matrix-core products, in ascending
 * token order (their G rows are the only non-zero ones); the other tokens' dH
 * rows are written as zeros.  dH and dW hold fp32 or bf16 elements
 * (p->grad_dtype).
 * Status 0, 1, 2, 6; with validate also 4 (active target out of range) and 5
 * (non-finite lse or coef). */
int grpo_head_bwd(const grpo_head_params* p, const void* H, const void* W, const int64_t* y,
                  const uint8_t* mask, const float* lse, const float* coef,
                  const float* grad_output, void* dH, void* dW, void* ws, size_t ws_bytes,
                  void* stream);

/* GSPO segment stage alone (no GEMM), from given per-token log-probs.
 *   per segment s with L_s active tokens: rho_s = sum_t m_t (logp_t - old_t) / L_s,
 *   sigma_s = exp(rho_s), c_s = clip(sigma_s, 1 - eps_low, 1 + eps_high),
 *   pol_s = -min(sigma_s A_s, c_s A_s); policy_loss = mean of pol_s over the
 *   S_live segments with L_s > 0; kl = sequence-mean of the token k3 term;
 *   coef_t = m_t / (S_live L_s) * (-A_s sigma_s [sigma_s A_s <= c_s A_s])
 *            + beta * m_t / (S_live L_s) * (1 - exp(ref_t - logp_t)).
 *   seg_mean_logp[s] (may be NULL) = mean active-token logp of segment s, 0 if
 *   L_s = 0 (the new_logprobs metric).
 * p->n_tokens, n_seqs, eps_*, beta, ignore_index and validate are used (the GEMM
 * fields d_model, v_real, v_rows, dtype and inv_tau are ignored, and level is
 * taken as GSPO; the segment mean is the only normaliser, so a reduction of
 * fixed_constant is rejected with status 1, the other reductions are ignored);
 * y is read only when mask is NULL (then it may not be NULL).  Needs
 * gspo_segment_workspace_size(p) bytes of workspace.
 * Status 0, 1, 2, 6; with validate also 3, 4, 5. */
int gspo_segment_reduce(const grpo_head_params* p, const float* logp, const float* old_logp,
                        const float* ref_logp, const uint8_t* mask, const int64_t* y,
                        const int32_t* sid, const float* adv, float* out3, float* coef,
                        float* seg_mean_logp, int32_t* counts, void* ws, size_t ws_bytes,
                        void* stream);

/* Bytes of device workspace gspo_segment_reduce needs (per-segment totals and
 * scalars).  0 if p is invalid. */
size_t gspo_segment_workspace_size(const grpo_head_params* p);

/* Forward-only selected log-probs: the vocabulary-tile stage and the ordered
 * merge of grpo_head_fwd, without the objective.  This is the one log-prob
 * operator a trainer calls for the policy and for the reference policy (and for
 * the old policy before an update): RL-Kernel PR #291 "Add deterministic
 * DP-aware GRPO loss on the TP-aware logprob path", Sequence Diagram(s) (the loss
 * asks the log-prob op for policy and reference log-probs) and the review
 * comment on the log-prob operator's usage example (the op returns logp and
 * lse); Liger-Kernel PR #1160 "[GRPO] add chunked grpo streaming over vocab",
 * conversation (a forward-only selective log-prob test against a reference).
 *   logp[t] = z[t, y_t] - lse[t] for active tokens, 0 for inactive ones;
 *   lse[t]  = LSE over the real vocabulary, for every token.
 * Both are bitwise equal to grpo_head_fwd's logp and lse for the same inputs.
 * Uses p->n_tokens, d_model, v_real, v_rows, ignore_index, dtype, inv_tau and
 * validate; every other field is ignored (n_seqs may be 0).  Needs
 * grpo_head_logp_workspace_size(p) bytes of workspace.
 * Status 0, 1, 2, 6; with validate also 4 (an active target outside
 * [0, v_real)) and 5 (a non-finite lse or logp).  A batch with no active token is
 * not an error here: logp is all zeros and lse is still written. */
int grpo_head_logp(const grpo_head_params* p, const void* H, const void* W, const int64_t* y,
                   const uint8_t* mask, float* logp, float* lse, void* ws, size_t ws_bytes,
                   void* stream);

/* Bytes of device workspace grpo_head_logp needs (per-tile partials and target
 * logits).  0 if p is invalid. */
size_t grpo_head_logp_workspace_size(const grpo_head_params* p);

/* grpo_head_logp without a workspace: for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same outputs, bitwise, as grpo_head_logp; same parameter fields and
 * statuses.  The scratch grpo_head_logp would take from its workspace lives in a
 * static device array of GRPO_HEAD_NOALLOC_SCRATCH_BYTES inside the library: each
 * GPU the library runs on holds one copy until the process ends.  A problem whose
 * grpo_head_logp_workspace_size(p) exceeds that size is rejected with status 1
 * before anything is enqueued (64 MiB holds 8192 tokens of a 151936-row vocabulary
 * with room to spare: about 14100 tokens at that vocabulary).  The call allocates
 * nothing; its first call on a device looks the array's address up
 * (hipGetSymbolAddress; a graph-capturing caller can make that first call before
 * capturing).  Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents: calls that overlap in time on one GPU (other streams or host
 * threads) race and must be serialised by the caller.  Nothing in the array needs
 * to start at zero: each call writes every element it later reads. */
#define GRPO_HEAD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int grpo_head_logp_noalloc(const grpo_head_params* p, const void* H, const void* W,
                           const int64_t* y, const uint8_t* mask, float* logp, float* lse,
                           void* stream);

/* One GPU's share of a vocabulary-parallel forward, part 1: the per-tile
 * partials and the target logits of one vocabulary shard, on the global tile
 * grid, so that a fixed-order merge of all shards' partials (part 2) is bitwise
 * the single-GPU result whatever the number of shards.  RL-Kernel PR #291 "Add
 * deterministic DP-aware GRPO loss on the TP-aware logprob path", commit notes
 * (ShardingSpec; the tile size must divide every shard boundary for cross-degree
 * bitwise equality; the fixed merge order) and the review thread on
 * _local_tile_stats.
 *   The shard is global vocabulary rows [v_begin, v_end), 0 <= v_begin < v_end <=
 *   v_rows; v_begin must be a multiple of 256 (the vocabulary tile) and v_end
 *   either a multiple of 256 or >= v_real.  W_shard points to the shard's first
 *   row (v_end - v_begin rows of d_model elements); rows >= v_real are padding
 *   and never read.  The shard's real rows [v_begin, min(v_end, v_real)) form
 *   n_st = ceil((min(v_end, v_real) - v_begin) / 256) tiles, the global tiles
 *   v_begin/256 .. + n_st - 1 (n_st may be 0 for a shard of padding only).
 *   partials  [n_st][n_tokens] pairs of fp32 (base-2 max, sum of 2^(z log2 e -
 *             max)) = grpo_head_shard_partials_bytes() bytes; the shards' arrays
 *             concatenated in ascending shard order are the global
 *             [ceil(v_real/256)][n_tokens] array part 2 reads.
 *   zy        [n_tokens] fp32, written for every token: z[t, y_t] when y_t lies
 *             in the shard's real rows and token t is active, else +0.0.  Adding
 *             the shards' zy (in any order) gives every target logit exactly.
 * Uses p->n_tokens, d_model, v_real, v_rows, ignore_index, dtype, inv_tau.
 * Status 0, 1, 6.  No workspace. */
int grpo_head_shard_partials(const grpo_head_params* p, int64_t v_begin, int64_t v_end,
                             const void* H, const void* W_shard, const int64_t* y,
                             const uint8_t* mask, void* partials, float* zy, void* stream);

/* Bytes of grpo_head_shard_partials' partials output for that shard; 0 if the
 * parameters or the shard bounds are invalid. */
size_t grpo_head_shard_partials_bytes(const grpo_head_params* p, int64_t v_begin,
                                      int64_t v_end);

/* Part 2: the fixed-order merge of all shards' partials (concatenated in global
 * tile order) into logp and lse, exactly as grpo_head_logp forms them:
 *   logp[t] = zy[t] - lse[t] for active tokens, 0 for inactive ones.
 * Bitwise equal to grpo_head_logp's outputs when the shards tile the vocabulary
 * as part 1 requires.  Uses the same fields as grpo_head_logp.  Status 0, 1, 6. */
int grpo_head_merge_partials(const grpo_head_params* p, const void* partials, const float* zy,
                             const int64_t* y, const uint8_t* mask, float* logp, float* lse,
                             void* stream);

/* Group-relative advantage of each sequence from its scalar reward: the step
 * before the objective, whose adv input it fills.  Sequences come in consecutive
 * groups of group_size (the completions of one prompt).  Per group:
 *   mean = sum_i r_i / G, var = sum_i (r_i - mean)^2 / G (two passes: the mean is
 *   subtracted before squaring), and
 *   adv_i = (r_i - mean) / (sqrt(var) + eps)   (0 when that divisor is 0), or
 *   adv_i = r_i - mean                         with scale_by_std = 0.
 * Sources: RL-Kernel PR #291 "Add deterministic DP-aware GRPO loss on the
 * TP-aware logprob path", Overview (the group-relative advantage acts per
 * sequence) and the review thread on the TWO_PASS variance enum.  The pages fix
 * neither the variance divisor nor eps: the population variance and a caller
 * eps are used.  Each group's sums run in index order, so results are bitwise
 * repeatable.
 *   rewards, adv  [n_seqs] fp32 device buffers (adv may alias rewards);
 *   group_size    G >= 1, dividing n_seqs; n_seqs >= 0 (0: nothing is enqueued);
 *   eps           finite, >= 0;  scale_by_std  0 or 1.
 * Status 0, 1, 6.  No workspace. */
int grpo_group_advantage(const float* rewards, int64_t n_seqs, int64_t group_size, float eps,
                         int32_t scale_by_std, float* adv, void* stream);

/* Stage timing for measurement tools; off by default, process-wide, not for
 * concurrent use from several threads.  `events` holds `n_events` caller-created
 * hipEvent_t handles (cast to void*; NULL entries are skipped), or events == NULL
 * to switch timing off.  The array is copied.  While set, the calls record
 * events on their stream at stage boundaries:
 *   grpo_head_fwd: [0] before the vocabulary-tile launch, [1] after it, [2]
 *                  after the target-logit gather and the merge, [3] after the
 *                  objective stage (grpo_head_logp records [0]-[2] the same way);
 *   grpo_head_bwd: [4] at entry, [5] just before a token chunk's dlogits tile
 *                  launch (after the row compaction and the H gather), [6] after
 *                  that launch (which also forms the target elements), [7] after
 *                  the launch of the two gradient products, dH and dW (with
 *                  several chunks, [5]-[7] describe the last one).
 * So [0]-[1], [5]-[6] and [6]-[7] each bracket one matrix-core launch.
 * Returns GRPO_HEAD_INVALID_ARGUMENT if n_events < 0 or > 16. */
int grpo_head_set_stage_events(void* const* events, int n_events);

/* Description of the last non-zero status returned on the calling thread
 * (thread-local; valid until the next call on that thread).  "" if none. */
const char* grpo_head_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GRPO_HEAD_H */
