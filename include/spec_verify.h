/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) verify step of speculative
 * decoding.
 *
 * One shared library, libspecverify.so, exports the calls below.  They take
 * plain device pointers and sizes; every tensor is device memory owned by the
 * caller.  Every call is asynchronous on the given HIP stream, reads no device
 * memory on the host, never synchronises and allocates nothing, so a caller may
 * capture it in a HIP graph.  Results are bitwise reproducible and do not
 * depend on batch composition: every random draw is keyed by (seed, request id,
 * absolute position), never by batch slot.
 *
 * Layout.  Request r owns the packed rows [qo_indptr[r], qo_indptr[r+1]) of
 * every per-row tensor (the qo_indptr packing of TensorRT-LLM PR #17056,
 * "DSpark confidence scheduling", description).  Its first gamma_r = rows_r - 1
 * rows verify drafted tokens 0..gamma_r-1 and its last row is the bonus row
 * (tokens submitted per request are verify_len + 1: same page, review-pass
 * commit note).  qo_indptr is int32 [R+1], non-decreasing, qo_indptr[0] = 0,
 * qo_indptr[R] = num_rows; every request owns at least its bonus row.
 *
 * Per-request sampling values live in device arrays and are clamped on the
 * device, never reported: T <= 0 or NaN -> greedy; k <= 0 or k >= V -> top-k
 * off; P >= 1 or NaN -> top-p off; P <= 0 -> keep the top token only.
 *
 * Errors.  Every call returns SV_OK (0) or a negative code for a problem the
 * host can see (null pointer, bad size, bad dtype, workspace too small, HIP
 * launch error).  spec_verify_status_string() names a code and
 * spec_verify_last_error() gives a thread-local message for the last failure.
 * Contract violations inside device data (a qo_indptr that does not start at
 * 0, decreases, or does not end at num_rows) are undefined on the fast path;
 * with SV_CHECK the call checks the layout on the device first and refuses a
 * violation instead of reading through it (TensorRT-LLM PR #17056, commit
 * notes on the layout assertions: refuse rather than degrade silently).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sv_stream_t; /* a hipStream_t; NULL is the default stream */

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

enum {
  SV_OK = 0,
  SV_ERR_NULL = -1,      /* a required pointer is NULL                          */
  SV_ERR_SHAPE = -2,     /* a size or leading dimension is out of range         */
  SV_ERR_DTYPE = -3,     /* unknown logit dtype, or a pointer misaligned for it */
  SV_ERR_WORKSPACE = -4, /* workspace missing or smaller than the size query    */
  SV_ERR_HIP = -5        /* a HIP call failed (message in spec_verify_last_error) */
};

/* Flags in sv_sampling.flags. */
enum {
  SV_ALL_GREEDY = 1u, /* every request is greedy: draft_probs may be NULL. The
                         host-side all-greedy skip of the consolidation study,
                         section 6 (sampling prep is inert at temperature 0). */
  SV_CHECK = 2u,      /* check qo_indptr on the device before the call's
                         kernels (one extra single-workgroup launch): qo[0] =
                         0, non-decreasing, qo[R] = num_rows.  The int32 at
                         byte 0 of the workspace receives 0 or the violated
                         SV_LAYOUT_* bits.  A violated layout is refused, not
                         read: spec_verify_rejection_sample then writes
                         accept_len 0, next_token -1 and out_tokens -1 /
                         row_flags 0 on every row, spec_verify_build_target_probs
                         writes row_max / row_lse NaN, row_argmax -1,
                         kept_count -1, kept_idx -1 and leaves probs untouched. */
  SV_LIST_BOUNDED = 4u, /* every sampled request has 0 < top_k <= 4096, so no
                         correction or bonus token is sampled over the whole
                         vocabulary: the call skips the two launches that split
                         such samples over workgroups.  A performance hint only:
                         a request that breaks it is still sampled exactly (by
                         one workgroup). */
  SV_BLOCK_VERIFY = 8u /* spec_verify_rejection_sample verifies sampled requests
                         by block verification (Sun et al., "Block Verification
                         Accelerates Speculative Decoding"; the consolidation
                         study's rejection_sample_method "block", sections 2, 4,
                         6) instead of token by token; greedy requests keep the
                         argmax rule.  See spec_verify_rejection_sample. */
};

/* Bits of the layout check word (SV_CHECK, spec_verify_check_layout). */
enum {
  SV_LAYOUT_START = 1, /* qo_indptr[0] != 0            */
  SV_LAYOUT_ORDER = 2, /* qo_indptr decreases somewhere */
  SV_LAYOUT_END = 4    /* qo_indptr[R] != num_rows      */
};

/* Row flag bits written by spec_verify_rejection_sample (row_flags). */
enum {
  SV_ROW_ACCEPT = 1,      /* this draft row's test accepted its token       */
  SV_ROW_SAMPLED = 2,     /* this row produced the correction / bonus token */
  SV_ROW_RESID_EMPTY = 32 /* residual was zero on the kept set; sampled p   */
};

typedef struct {
  const float* temperature;  /* [R] device; T <= 0 or NaN: greedy                   */
  const int32_t* top_k;      /* [R] device or NULL (off)                            */
  const float* top_p;        /* [R] device or NULL (off)                            */
  const uint32_t* request_id;/* [R] device or NULL (r): Philox counter word         */
  const uint32_t* position0; /* [R] device or NULL (0): absolute position of row 0  */
  uint64_t seed;             /* Philox4x32-10 key                                   */
  uint32_t flags;            /* SV_ALL_GREEDY | SV_CHECK | SV_LIST_BOUNDED |
                                SV_BLOCK_VERIFY                                     */
  const int32_t* row_order;  /* [num_rows] device or NULL (natural order): the order
                                in which rows are scheduled, a permutation of
                                0..num_rows-1 (anything else leaves the results
                                undefined; ids outside the range are skipped).  A
                                load-balance hint: rows that may need the multi-pass
                                exact top-p path (top-k off, top-p on) placed first
                                overlap their extra passes with the other rows. */
} sv_sampling;

/* Bytes of device workspace the calls below need for these sizes (block: the
 * planner's positions per request, 0 when the planner is not used).  The
 * workspace is scratch: its contents need no initialisation.  After a call,
 * the int32 at byte 0 holds the SV_CHECK layout word (when the call had
 * SV_CHECK) and spec_verify_row_diagnostics can read the per-row records;
 * the rest is meaningless.  It must be 256-byte aligned. */
size_t spec_verify_workspace_bytes(int32_t num_rows, int32_t vocab, int32_t num_requests,
                                   int32_t block);

/* Target distribution per row ("Adaptive verification for DFLASH ... built on
 * upstream DSpark", commit note on build_speculative_verify_target_probs):
 * top-k selected on the raw logits, the temperature applied to the selected
 * values only, then top-p over the top-k renormalised distribution, softmax.
 * Ties are broken by lower token id everywhere.
 *   logits     [num_rows, ld_logits] row-major, dt = SV_BF16 or SV_F32
 *   probs      [num_rows, ld_probs] fp32 or NULL: p on the kept set, 0 elsewhere
 *   row_max, row_argmax, row_lse [num_rows] or NULL; lse is log sum exp(x / T_eff)
 *              over the whole row with T_eff = T, or 1 on greedy rows
 *   kept_count [num_rows] or NULL; kept_idx [num_rows, kmax] or NULL: the first
 *              min(kept_count, kmax) kept ids in order (value desc, id asc), then -1.
 *              kmax <= 1024.
 * Returns SV_ERR_SHAPE when ld_logits < vocab, ld_probs < vocab, kmax > 1024. */
int32_t spec_verify_build_target_probs(const void* logits, sv_dtype dt, int64_t ld_logits,
                                       int32_t num_rows, int32_t vocab,
                                       const int32_t* qo_indptr, int32_t num_requests,
                                       const sv_sampling* sp, float* probs, int64_t ld_probs,
                                       float* row_max, int32_t* row_argmax, float* row_lse,
                                       int32_t* kept_count, int32_t* kept_idx, int32_t kmax,
                                       void* workspace, size_t workspace_bytes,
                                       sv_stream_t stream);

/* The fused verify step.  Per draft row: greedy accepts iff the draft equals
 * the target argmax; temperature > 0 runs the ratio test u < min(1, p(d)/q(d))
 * of Leviathan et al. with an fp64 Philox uniform keyed (seed, request id,
 * position0 + j) (consolidation study, sections 2-4).  At the first rejection
 * the row samples the residual max(0, p - q) by an exponential race (Gumbel-max
 * keyed by position); after a full accept the bonus is sampled from p at the
 * row after the last verified draft ("the bonus comes from the last verified
 * row", DFLASH-through-DSpark commit note).  verify_cap (cap-accept) stops
 * acceptance at min(gamma_r, verify_cap[r]) without changing the rule.
 *   draft_tokens [num_rows] int32; the bonus row's entry is ignored; an id
 *              outside [0, V) is never accepted (the row then samples p)
 *   draft_probs [num_rows, ld_q] fp32 draft distributions, only gathered; may
 *              be NULL only with SV_ALL_GREEDY
 *   verify_cap [R] or NULL
 *   accept_len [R]; out_tokens [num_rows]: row s_r + j holds draft j for
 *              j < L, the sampled token at j = L, -1 after; next_token [R]: the
 *              sampled (correction or bonus) token; row_flags [num_rows] or NULL.
 * With SV_BLOCK_VERIFY a sampled request is verified as a block: weights
 * p_0 = 1, p_i = min(p_{i-1} p(d_{i-1}) / q(d_{i-1}), 1); position i passes when
 * u_{i-1} < h_i, h_i = A_i / (A_i + 1 - p_i) with A_i the residual mass
 * sum_x max(p_i p_i(x) - q_i(x), 0) of row i (h = p at the last verified
 * position); accept_len is the last position passed, and the emitted token
 * comes from the residual max(p_L p - q, 0) of row L, or from p when every
 * position passed.  row_flags bit 0 then marks the positions passed.  Rows
 * whose kept set is not a list (top-k and top-p off, or a kept set over 4096)
 * cost one extra pass over the row and its draft probabilities in the finalize.
 * Returns SV_ERR_NULL when draft_probs is NULL without SV_ALL_GREEDY. */
int32_t spec_verify_rejection_sample(const void* target_logits, sv_dtype dt, int64_t ld_logits,
                                     int32_t vocab, const int32_t* qo_indptr,
                                     int32_t num_requests, int32_t num_rows,
                                     const int32_t* draft_tokens, const float* draft_probs,
                                     int64_t ld_q, const int32_t* verify_cap,
                                     const sv_sampling* sp, int32_t* accept_len,
                                     int32_t* out_tokens, int32_t* next_token,
                                     uint8_t* row_flags, void* workspace,
                                     size_t workspace_bytes, sv_stream_t stream);

/* spec_verify_rejection_sample without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The call allocates nothing: its
 * scratch is a static device array of the library, one per device (34 MiB,
 * placed when the library loads on the device and held until the process
 * ends), whose address the first call on each device looks up with that
 * device current.  Limits: num_rows <= 1024 and num_requests <= 1024, else
 * SV_ERR_SHAPE before any launch.  Every call on one device shares that
 * device's array: calls that overlap on one device (two streams, two host
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  Arguments, outputs and other errors are spec_verify_rejection_sample's;
 * SV_CHECK writes its layout word into the shared array, where the caller cannot
 * read it (the refused outputs still show a failed check). */
int32_t spec_verify_rejection_sample_noalloc(const void* target_logits, sv_dtype dt,
                                             int64_t ld_logits, int32_t vocab,
                                             const int32_t* qo_indptr, int32_t num_requests,
                                             int32_t num_rows, const int32_t* draft_tokens,
                                             const float* draft_probs, int64_t ld_q,
                                             const int32_t* verify_cap, const sv_sampling* sp,
                                             int32_t* accept_len, int32_t* out_tokens,
                                             int32_t* next_token, uint8_t* row_flags,
                                             sv_stream_t stream);

/* Confidence planner (method: TensorRT-LLM PR #17056, first commit note): a
 * position's survival is the product of its request's confidences up to it,
 * and one global ranking of all positions by survival, with ties ordered by
 * position and request rather than by value, decides which are verified.
 * Confidences are clamped to [0,1] (NaN -> 0); S[r][j] = c[r][0]*...*c[r][j] in
 * fp32, left to right; all (r, j) are ranked by (S desc, j asc, r asc) and the
 * first min(budget, R*block) are verified.
 *   confidence [R, ld_conf] fp32; verify_len [R] int32; qo_indptr [R+1] int32,
 *   exclusive scan of verify_len + 1 (one bonus row per request), so
 *   qo_indptr[R] = min(budget, R*block) + R is known on the host;
 *   survival [R, block] fp32 or NULL.
 * Requires R * block < 2^31. */
int32_t spec_verify_plan_windows(const float* confidence, int64_t ld_conf, int32_t num_requests,
                                 int32_t block, int32_t budget, int32_t* verify_len,
                                 int32_t* qo_indptr, float* survival, void* workspace,
                                 size_t workspace_bytes, sv_stream_t stream);

/* Verify budget from a step-cost table (method: TensorRT-LLM PR #17056,
 * description).  Survivals and their rank order are spec_verify_plan_windows's.
 * Every b in [0, R*B] is scored: tau(b) = R + the b largest survivals (fp64),
 * the step runs b + R verify rows (bonus rows included), and Theta(b) = tau(b) /
 * cost[b + R]; the largest Theta wins, the smaller b on equal Theta.  Scoring
 * every b (not stopping at the first drop) matters because the cost rises in
 * steps.  Without a table nothing is trimmed.
 *   confidence [R, ld_conf] fp32, device (as spec_verify_plan_windows)
 *   cost       [ncost] fp32, device: step cost by packed verify row count; NULL
 *              or ncost 0: no table.  ncost must reach R*B + R + 1.
 *   budget     [1] int32, device, written: the budget; R*B when there is no
 *              table or it is equal over [R, R*B + R]; -1 when a cost in that
 *              range is non-positive or non-finite
 *   theta      [1] fp64, device, written (NULL: skipped): Theta(budget), 0 with
 *              no table, NaN with an invalid one
 *   workspace  device scratch of at least spec_verify_workspace_bytes(0, 1, R,
 *              block) bytes, 256-byte aligned; needed only when R*B > 4096
 *              (may be NULL otherwise); its contents afterwards are meaningless
 * R*B must be at most 2^20.  Up to 4096 positions one workgroup sorts the
 * survivals in LDS; beyond, three launches (tile sorts, a rank placement by
 * binary search, one scanning workgroup).  No host synchronisation: the budget
 * stays on the device.  Errors (host-side checks, returned before any launch):
 * SV_ERR_SHAPE, SV_ERR_NULL, SV_ERR_WORKSPACE. */
int32_t spec_verify_plan_budget(const float* confidence, int64_t ld_conf, int32_t num_requests,
                                int32_t block, const float* cost, int32_t ncost, int32_t* budget,
                                double* theta, void* workspace, size_t workspace_bytes,
                                sv_stream_t stream);

/* Accepted prefix from per-row accept bytes (greedy accept with precomputed
 * argmax ids, DFLASH-through-DSpark commit note): accept_len[r] = first j <
 * min(gamma_r, verify_cap[r]) with accepted[s_r + j] == 0, else that bound. */
int32_t spec_verify_accept_prefix(const uint8_t* accepted, const int32_t* qo_indptr,
                                  int32_t num_requests, const int32_t* verify_cap,
                                  int32_t* accept_len, sv_stream_t stream);

/* Layout check of a packed qo_indptr (the check SV_CHECK runs inside a call),
 * for callers that build qo_indptr on the device (e.g. with
 * spec_verify_plan_windows) and want the result before any verify call:
 * writes 0 or the violated SV_LAYOUT_* bits to error_word (one int32, device).
 * Reads qo_indptr[0..R] only.  One workgroup, no synchronisation. */
int32_t spec_verify_check_layout(const int32_t* qo_indptr, int32_t num_requests,
                                 int32_t num_rows, int32_t* error_word, sv_stream_t stream);

/* Diagnostics of the decision quantities: after spec_verify_rejection_sample or
 * spec_verify_build_target_probs on this workspace (and before another call
 * reuses it), copy per row the top-k mass Z_K (over the whole row when top-k is
 * off), the kept mass Z_N (both relative to exp(m / T)), p(d) of a tested draft
 * as the ratio test used it, and the row mode (0 unused, 1 greedy, 2 kept list,
 * 3 whole row, 4 kept range, 5 exact path).  Every output [num_rows] device
 * array may be NULL.  These are the values a caller compares against a
 * reference to check that the device decided with enough precision; they are
 * not needed for verification itself. */
int32_t spec_verify_row_diagnostics(const void* workspace, size_t workspace_bytes,
                                    int32_t num_rows, double* row_zk, double* row_zn,
                                    double* row_pd, int32_t* row_mode, sv_stream_t stream);

/* Acceptance and trim statistics of one verify step (TensorRT-LLM PR #17056,
 * commit note on the trim-regret metric: a trimmed request that accepted its
 * entire window was still alive at the cut, so the cut cost acceptance;
 * per-position acceptance as the consolidation study's section 1 reports it,
 * the share of drafts whose first j+1 tokens survived).  Request r verified
 * w_r = verify_len[r] (e.g. the planner's window) of the block's B drafted
 * positions and accepted L_r = accept_len[r] (e.g. spec_verify_rejection_sample's
 * output); device data is clamped: w_r to [0, B], L_r to [0, w_r].
 *   stats [5 + 2B] int64, device:
 *     [0] requests, [1] trimmed (w_r < B), [2] trim regret (trimmed and
 *     L_r == w_r), [3] sum of L_r, [4] sum of w_r,
 *     [5 + j] offered at position j = #{r : w_r > j},
 *     [5 + B + j] accepted at position j = #{r : L_r > j}, for j < B.
 *   The trim-regret rate is stats[2] / stats[1]; the acceptance per draft
 *   token stats[3] / stats[4].  Exact integer counts; one workgroup, no
 *   workspace.  Requires 0 <= B <= 1024 and R * B < 2^31. */
int32_t spec_verify_acceptance_stats(const int32_t* accept_len, const int32_t* verify_len,
                                     int32_t num_requests, int32_t block, int64_t* stats,
                                     sv_stream_t stream);

/* Online acceptance estimator (SGLang PR "Adaptive verification for DFLASH
 * ... built on upstream DSpark", commit notes adding OnlineAcceptanceEstimator
 * and fixing its slope refit): the planner's confidence source for drafts
 * without a trained confidence head.  p_k = sigmoid(slope * x_k + bias_k),
 * x_k = logit(q_max) of the temperature-scaled draft distribution at position
 * k (T = 1 for greedy requests), clamped to +-40; one slope, one intercept per
 * position, starting at 0.5 and -0.2.
 *   state: device doubles, spec_verify_estimator_state_doubles(block) of them,
 *   caller-owned, written by spec_verify_estimator_init; it holds the
 *   coefficients, the IRLS statistics since the last refit and the refit
 *   counter, so no call synchronizes with the host.  Calls on one state must
 *   be ordered (one stream).  block (drafted positions per request) in [1, 64].
 * predict: the draft rows of request r are rows r * block + k of the draft
 *   build's row_max / row_lse (spec_verify_build_target_probs on the draft
 *   logits); temperature [R] or NULL (greedy).  Writes feature [R, block]
 *   fp64 (or NULL) and confidence [R, block] fp32 (or NULL), the planner's
 *   input.
 * observe: after verification, labels positions k < L_r accepted and k = L_r
 *   rejected when L_r < w_r (w_r = verify_len[r] clamped to [0, block], L_r =
 *   accept_len[r] clamped to [0, w_r]), adds them to the Newton statistics at
 *   the current coefficients; every 100th call solves the arrowhead Newton
 *   system with ridge 1e-3, damps each update by n / (n + 50) (n: the labels
 *   behind that coefficient), drops non-finite steps, halves a slope step that
 *   would make the slope negative (at most 8 times, dropped if it still
 *   does), steps the intercepts given the slope step taken, and clears the
 *   statistics.  One workgroup in a fixed order: the same inputs give the
 *   same coefficients. */
size_t spec_verify_estimator_state_doubles(int32_t block);
int32_t spec_verify_estimator_init(double* state, int32_t block, sv_stream_t stream);
int32_t spec_verify_estimator_predict(const float* row_max, const float* row_lse,
                                      const float* temperature, int32_t num_requests,
                                      int32_t block, const double* state, double* feature,
                                      float* confidence, sv_stream_t stream);
int32_t spec_verify_estimator_observe(const double* feature, const int32_t* accept_len,
                                      const int32_t* verify_len, int32_t num_requests,
                                      int32_t block, double* state, sv_stream_t stream);

/* Diagnostics. */
const char* spec_verify_status_string(int32_t code);
const char* spec_verify_last_error(void);

/* Per-kernel timing for measurement: while enabled, every launch of the
 * library first waits for its stream to drain (the host blocks), then
 * records a pair of HIP events around the kernel on the call's stream;
 * read() waits for them and returns, per kernel id, the launch count and the
 * summed milliseconds since the last reset.  Kernel ids: 0 row pass, 1 request
 * finalize, 2 target-probs writer, 3 planner, 4 accept prefix, 5 race
 * segments, 6 race finish, 7 acceptance statistics and estimator, 8 layout
 * check, 9 row diagnostics. */
int32_t spec_verify_profile_enable(int32_t on);
int32_t spec_verify_profile_read(int32_t kernel_id, int64_t* launches, double* total_ms);
int32_t spec_verify_profile_reset(void);

#ifdef __cplusplus
}
#endif
#endif
