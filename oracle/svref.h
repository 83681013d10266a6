/*
 * svref.h -- CPU oracle for the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, single-threaded fp64
 * definition of what the verify step computes.  It shares no code, header,
 * table or constant with the HIP library under rejection_sampling_amd/csrc,
 * and only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  The product path never calls it.
 *
 * Sources (the pages are web pages; citations name page and section):
 *  - "Adaptive verification for DFLASH ... built on upstream DSpark"
 *    (jianc99/sglang PR #8), commit note on build_speculative_verify_target_probs:
 *    top-k is selected on the raw logits and only the selected values are
 *    divided by the temperature; top-k/top-p distribution; deterministic ties.
 *  - Same page, commit note "run DFLASH through the existing DSpark machinery":
 *    every accept path stops at the planned verify length, greedy accept with
 *    precomputed argmax ids, the bonus comes from the last verified row.
 *  - "dspark-upstream-consolidation" study (rtx6kpro), section 2: greedy accepts
 *    iff draft == target argmax; temperature > 0 runs the Leviathan ratio test;
 *    Gumbel noise keyed by position.  Sections 3-4: fp64 acceptance uniforms.
 *  - TensorRT-LLM PR #17056 "DSpark confidence scheduling", first commit note and
 *    description: survival of a position as a running product of confidences,
 *    one batch-wide ranking by survival (ties by position and request) that
 *    decides the verified positions, windows packed with a qo_indptr; the
 *    review-pass note: tokens submitted per request are verify_len + 1.
 *  - Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *    Easy as 1, 2, 3", SC'11.
 *  - Ratio test and residual max(0, p - q): Leviathan, Kalman, Matias, "Fast
 *    Inference from Transformers via Speculative Decoding", ICML 2023.
 *
 * Row layout: request r owns rows [qo_indptr[r], qo_indptr[r+1]).  Its first
 * gamma_r = rows_r - 1 rows verify drafted tokens 0..gamma_r-1; its last row is
 * the bonus row.  All pointers are host pointers.  Every function returns 0 on
 * success and a negative value on a malformed argument.
 */
#ifndef SVREF_H
#define SVREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SVREF_F32 = 0, SVREF_BF16 = 1 };

/* Row flag bits written by svref_rejection_sample. */
enum {
  SVREF_ROW_ACCEPT = 1,     /* this draft row's test accepted its token          */
  SVREF_ROW_SAMPLED = 2,    /* this row produced the emitted correction/bonus    */
  SVREF_ROW_NEAR_RATIO = 4, /* |u - ratio| < 1e-5                                */
  SVREF_ROW_NEAR_TOPP = 8,  /* top-p boundary mass within 1e-6 * Z_K             */
  SVREF_ROW_NEAR_RACE = 16, /* best and second race keys within 1e-6 (relative)  */
  SVREF_ROW_RESID_EMPTY = 32,/* residual was zero on the kept set: raced over p  */
  SVREF_ROW_BAD_DRAFT = 64  /* draft id outside [0, V): rejected                 */
};

/* svref_sampling.flags: verify sampled requests by block verification (Sun et
 * al., "Block Verification Accelerates Speculative Decoding") instead of the
 * token-by-token ratio test; greedy requests keep the argmax rule. */
enum { SVREF_BLOCK_VERIFY = 8 };

typedef struct {
  const float* temperature;  /* [R]  T <= 0 or NaN: greedy                    */
  const int32_t* top_k;      /* [R]  k <= 0 or k >= V: off; NULL: off         */
  const float* top_p;        /* [R]  P >= 1 or NaN: off; P <= 0: top-1; NULL: off */
  const uint32_t* request_id;/* [R]  Philox counter word; NULL: r             */
  const uint32_t* position0; /* [R]  absolute position of window row 0; NULL: 0 */
  uint64_t seed;             /* Philox key                                    */
  uint32_t flags;            /* SVREF_BLOCK_VERIFY or 0                       */
} svref_sampling;

/* Philox4x32-10 block function: out = Philox(key, ctr). */
void svref_philox4x32_10(const uint32_t key[2], const uint32_t ctr[4], uint32_t out[4]);

/* Acceptance uniform in [0,1) for (seed, request id, absolute position). */
double svref_uniform_accept(uint64_t seed, uint32_t request_id, uint32_t position);

/* Race uniform in (0,1) for token `token` under stream `tag` (1 verify, 2 draft). */
double svref_uniform_race(uint64_t seed, uint32_t request_id, uint32_t position,
                          uint32_t tag, uint32_t token);

/* Target distribution per row.  Every output pointer may be NULL.
 *   probs     [rows, ld_probs] fp64, p on the kept set, 0 elsewhere
 *   row_max, row_argmax, row_lse (lse at T_eff = T, or 1 on greedy rows)
 *   kept_count [rows], kept_idx [rows, kmax] in order (value desc, index asc),
 *   row_zn    [rows] mass of the kept set relative to the row max (Z_N)
 *   row_flags [rows] SVREF_ROW_NEAR_TOPP where the top-p boundary is a near tie
 *   row_zk    [rows] mass of the top-k set relative to the row max (Z_K)
 *   kept_lo, kept_hi [rows] the near-tie band of the kept count: the smallest
 *             and largest counts a top-p target anywhere within 1e-6 * Z_K of
 *             P * Z_K gives (equal to kept_count off the band); the row is
 *             flagged SVREF_ROW_NEAR_TOPP exactly when they differ
 *   order_idx [rows, kmax] the first kmax ids of the row order (value desc,
 *             index asc); greedy rows hold the argmax only */
int32_t svref_build_target_probs(const void* logits, int32_t dtype, int64_t ld_logits,
                                 int32_t num_rows, int32_t vocab, const int32_t* qo_indptr,
                                 int32_t num_requests, const svref_sampling* sp, double* probs,
                                 int64_t ld_probs, double* row_max, int32_t* row_argmax,
                                 double* row_lse, int32_t* kept_count, int32_t* kept_idx,
                                 int32_t kmax, double* row_zn, uint8_t* row_flags,
                                 double* row_zk, int32_t* kept_lo, int32_t* kept_hi,
                                 int32_t* order_idx);

/* The verify step.  draft_probs may be NULL only when every request is greedy.
 * verify_cap may be NULL.  row_ratio / row_u (diagnostics, may be NULL) get the
 * ratio and the uniform of each tested draft row (NaN elsewhere); row_zk /
 * row_zn (may be NULL) the masses Z_K and Z_N of every sampled row the step
 * builds (NaN elsewhere). */
int32_t svref_rejection_sample(const void* logits, int32_t dtype, int64_t ld_logits,
                               int32_t vocab, const int32_t* qo_indptr, int32_t num_requests,
                               int32_t num_rows, const int32_t* draft_tokens,
                               const float* draft_probs, int64_t ld_q, const int32_t* verify_cap,
                               const svref_sampling* sp, int32_t* accept_len, int32_t* out_tokens,
                               int32_t* next_token, uint8_t* row_flags, double* row_ratio,
                               double* row_u, double* row_zk, double* row_zn);

/* Confidence planner: survival cumprod (fp32), rank (S desc, j asc, r asc),
 * budget -> verify_len [R], qo_indptr [R+1], survival [R, block] (may be NULL). */
int32_t svref_plan_windows(const float* confidence, int64_t ld_conf, int32_t num_requests,
                           int32_t block, int32_t budget, int32_t* verify_len,
                           int32_t* qo_indptr, float* survival);

/* Accepted prefix length per request from per-row accept bytes. */
int32_t svref_accept_prefix(const uint8_t* accepted, const int32_t* qo_indptr,
                            int32_t num_requests, const int32_t* verify_cap, int32_t* accept_len);

/* Verify budget from a step-cost table (method: TensorRT-LLM PR #17056,
 * description): every budget is scored by tau/cost and the best score wins,
 * since a cost that rises in steps leaves a local peak at each step.
 * Survivals S and their rank order are those of svref_plan_windows.  For a
 * budget b in [0, R*B], tau(b) = R + (sum of the b first survivals in rank
 * order, fp64, in that order) is the expected count of tokens the step emits
 * (accepted drafts plus one bonus or correction token per request), and the
 * step packs b + R verify rows, so Theta(b) = tau(b) / cost[b + R].  The
 * smallest b with the largest Theta wins.  With no table (cost NULL or
 * ncost 0), or a table equal at every count in [R, R*B + R], the budget is
 * R*B: nothing is trimmed.  theta (may be NULL) receives Theta(budget).
 * Returns -3 when the table is shorter than R*B + R + 1 entries or holds a
 * non-finite or non-positive cost in that range. */
int32_t svref_budget_from_costs(const float* confidence, int64_t ld_conf, int32_t num_requests,
                                int32_t block, const float* cost, int32_t ncost,
                                int32_t* budget, double* theta);

/* Acceptance and trim statistics of one verify step (TensorRT-LLM PR #17056,
 * commit note on the trim-regret metric: a trimmed request that accepted its
 * whole window lost acceptance to the cut; the consolidation study, section 1:
 * per-position acceptance is the share of drafts whose first j+1 tokens
 * survived).  Request r verified w_r = verify_len[r] of the block's B drafted
 * positions and accepted L_r = accept_len[r]; w_r is clamped to [0, B] and L_r
 * to [0, w_r].  stats (int64):
 *   [0] requests, [1] trimmed (w_r < B), [2] regret (trimmed and L_r == w_r),
 *   [3] sum L_r, [4] sum w_r,
 *   [5 + j] offered at position j = #{r : w_r > j},
 *   [5 + B + j] accepted at position j = #{r : L_r > j},   j < B. */
int32_t svref_acceptance_stats(const int32_t* accept_len, const int32_t* verify_len,
                               int32_t num_requests, int32_t block, int64_t* stats);

/* Online acceptance estimator (SGLang PR "Adaptive verification for DFLASH",
 * commit notes adding OnlineAcceptanceEstimator and fixing its slope refit):
 * a logistic model p_k = sigmoid(slope * x_k + bias_k) of the acceptance of
 * the drafted token at position k, calibrated while serving.  x_k =
 * logit(q_max) of the temperature-scaled draft distribution at that position
 * (greedy rows at T = 1), clamped to +-40.  One slope shared by all positions,
 * one intercept per position, starting at 0.5 and -0.2.  observe() labels the
 * accepted drafts 1 and the first rejected one 0 and adds them to the Newton
 * (IRLS) statistics at the current coefficients; every SVREF_EST_REFIT calls
 * the arrowhead Newton system is solved with a ridge, each update damped by
 * n / (n + 50), non-finite steps dropped, a slope step that would make the
 * slope negative halved (at most 8 times, dropped if it still crosses zero),
 * the intercepts stepped given the slope step taken, and the statistics
 * cleared. */
#define SVREF_EST_MAXB 64
#define SVREF_EST_REFIT 100
typedef struct {
  int32_t block;                    /* positions per request, <= SVREF_EST_MAXB */
  int32_t calls;                    /* observe calls since the last refit       */
  int32_t refits;                   /* refits so far                            */
  int32_t pad;
  double slope;
  double bias[SVREF_EST_MAXB];
  /* IRLS statistics since the last refit: Hessian (arrowhead), gradient, counts */
  double h_ss, g_s, n_s;
  double h_sk[SVREF_EST_MAXB], h_kk[SVREF_EST_MAXB], g_k[SVREF_EST_MAXB], n_k[SVREF_EST_MAXB];
  /* the last refit's Newton direction before damping (for inspection) */
  double last_ds, last_db[SVREF_EST_MAXB];
} svref_estimator;

int32_t svref_est_init(svref_estimator* est, int32_t block);
/* Feature per row from the draft build's row max m and lse (at T_eff = T, or 1
 * for greedy rows): x = logit(exp(m / T_eff - lse)), clamped to [-40, 40]. */
int32_t svref_est_feature(const float* row_max, const float* row_lse, const float* t_eff,
                          int32_t num_rows, double* x);
/* p = sigmoid(slope * x + bias[k]) for the rows' positions k. */
int32_t svref_est_predict(const svref_estimator* est, const double* x, const int32_t* pos,
                          int32_t n, double* p);
/* One step's observations: request r drafted positions 0..B-1 with features
 * x[r * B + k]; it verified w_r = verify_len[r] (clamped to [0, B]) and
 * accepted L_r = accept_len[r] (clamped to [0, w_r]).  Positions k < L_r are
 * labelled 1 and k = L_r < w_r is labelled 0. */
int32_t svref_est_observe(svref_estimator* est, const double* x, const int32_t* accept_len,
                          const int32_t* verify_len, int32_t num_requests);

/* Harness helper: one exponential-race sample per row from dense fp32
 * probability rows, keyed (seed, request id, position0 + j, tag). */
int32_t svref_sample_probs(const float* probs, int64_t ld_probs, int32_t num_rows, int32_t vocab,
                           const int32_t* qo_indptr, int32_t num_requests,
                           const uint32_t* request_id, const uint32_t* position0, uint64_t seed,
                           uint32_t tag, int32_t* out);

#ifdef __cplusplus
}
#endif
#endif
