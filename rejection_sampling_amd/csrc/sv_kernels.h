// sv_kernels.h -- kernel argument blocks and launch entry points shared by the
// kernel translation units and the host library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.hpp"

namespace sv {

struct RowRec;
struct ListEntry;

// Best (key, id) of one segment of a full-vocabulary race (key <= 0: none).
struct RacePart {
  double key;
  int32_t id;
  int32_t pad;
};

struct VerifyArgs {
  const void* logits;
  int64_t ld_logits;
  int32_t vocab;
  int32_t dtype;          // 0 fp32, 1 bf16
  const int32_t* qo;
  int32_t num_requests;
  int32_t num_rows;
  const int32_t* draft_tokens;
  const float* draft_probs;
  int64_t ld_q;
  const int32_t* verify_cap;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const uint32_t* request_id;
  const uint32_t* position0;
  const int32_t* row_order;   // [num_rows] or NULL: row of each row-pass workgroup
  uint64_t seed;
  int32_t build;          // 1: target-probs build (every row, lse), 0: verify
  RowRec* rec;            // [num_rows]
  ListEntry* list;        // [num_rows, kListCap]
  int32_t* accept_len;
  int32_t* out_tokens;
  int32_t* next_token;
  uint8_t* row_flags;
  // full-vocabulary samples split over workgroups (race_segs 0: finalize runs
  // them in one workgroup)
  int32_t race_segs;      // segments per race at most (kMaxRaceSegs at most)
  int32_t* race_job;      // [num_requests]: 2 * row + residual, or -1
  RacePart* race_part;    // [num_requests, kMaxRaceSegs]
  int32_t* race_nseg;     // one int (workspace): segments per race this call
  double* race_zn;        // [num_requests]: Z_N the split race divides by
  // block verification of sampled requests (0: the token rule)
  int32_t block;
  double* block_w;        // [num_rows, 2]: block weight p_i and test bound h_i per row
  // every row-pass workgroup is resident at once: rows on one CU are kept
  // level by progress-based wave priorities
  int32_t level;
  // layout check word written by check_layout_kernel earlier on the stream,
  // or NULL: when it is nonzero the kernels refuse the call (no qo_indptr
  // read, refused outputs written)
  const int32_t* check;
};

struct BuildOutArgs {
  float* probs;
  int64_t ld_probs;
  float* row_max;
  int32_t* row_argmax;
  float* row_lse;
  int32_t* kept_count;
  int32_t* kept_idx;
  int32_t kmax;
};

struct PlanArgs {
  const float* conf;
  int64_t ld_conf;
  int32_t num_requests;
  int32_t block;
  int32_t budget;
  int32_t* verify_len;
  int32_t* qo_indptr;
  float* survival;
  uint64_t* keys;        // workspace [R * block]
};

__global__ void check_layout_kernel(const int32_t* qo, int32_t R, int32_t rows, int32_t* word);
__global__ void diagnostics_kernel(const RowRec* rec, int32_t rows, double* zk, double* zn,
                                   double* pd, int32_t* mode);
__global__ void row_pass_kernel(VerifyArgs A);
__global__ void finalize_kernel(VerifyArgs A);
__global__ void finalize_block_kernel(VerifyArgs A);
__global__ void race_segment_kernel(VerifyArgs A);
__global__ void race_finish_kernel(VerifyArgs A);
__global__ void build_out_kernel(VerifyArgs A, BuildOutArgs B);
__global__ void plan_kernel(PlanArgs A);
__global__ void budget_kernel(const float* conf, int64_t ld_conf, int32_t R, int32_t B,
                              const float* cost, int32_t* budget, double* theta);
__global__ void budget_tile_kernel(const float* conf, int64_t ld_conf, int32_t R, int32_t B,
                                   uint32_t* tiles);
__global__ void budget_rank_kernel(const uint32_t* tiles, int32_t n, uint32_t* sorted);
__global__ void budget_scan_kernel(const uint32_t* sorted, int32_t R, int32_t n, const float* cost,
                                   int32_t* budget, double* theta);
__global__ void accept_prefix_kernel(const uint8_t* accepted, const int32_t* qo, int32_t R,
                                     const int32_t* verify_cap, int32_t* accept_len);
__global__ void acceptance_stats_kernel(const int32_t* accept_len, const int32_t* verify_len,
                                        int32_t R, int32_t B, int64_t* stats);
__global__ void est_init_kernel(double* st, int32_t B);
__global__ void est_predict_kernel(const float* row_max, const float* row_lse,
                                   const float* temperature, int32_t R, int32_t B,
                                   const double* st, double* feature, float* confidence);
__global__ void est_observe_kernel(const double* feature, const int32_t* accept_len,
                                   const int32_t* verify_len, int32_t R, int32_t B, double* st);

// sizes shared with the host
constexpr int kRowBlock = SV_BLOCK;
constexpr int kRowPassPerCU = 4;     // row-pass workgroups resident per CU (LDS and VGPR bound)
constexpr int kPlanBlock = 1024;
constexpr int kBudgetMaxKeys = 4096; // drafted positions one workgroup sorts in LDS (budget search)
constexpr int kBudgetMaxN = 1 << 20;  // drafted positions of a budget search (tiles of kBudgetMaxKeys)
constexpr size_t kRowRecBytes = 64;
constexpr size_t kWsHeader = 256;    // workspace bytes before the row records (check word)
constexpr int kEstMaxBlock = 64;     // estimator positions per request
constexpr int kEstRefit = 100;       // estimator observe calls per refit
constexpr int kEstStateBase = 6;     // estimator state doubles: 6 + 5 * block
constexpr int kRaceSegElems = 4096;  // vocabulary elements per race segment
constexpr int kMaxRaceSegs = 64;
constexpr int kRaceGrid = 768;      // race-segment workgroups (three per CU resident)

}  // namespace sv
