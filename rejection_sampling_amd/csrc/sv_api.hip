// sv_api.hip -- host side of libspecverify: argument checks, workspace
// carving, launches, status codes and optional per-kernel event timing.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/spec_verify.h"
#include "sv_device.hpp"
#include "sv_kernels.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* what) {
  g_last_error = what;
  return code;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t rec, list, race_job, race_part, race_zn, block_w, keys, total;
};

constexpr Layout layout(int64_t rows, int64_t R, int64_t block) {
  Layout L{};
  L.rec = sv::kWsHeader;  // bytes [0, 4): the layout check word of SV_CHECK; [4, 8): the
                          // split race's segment count
  L.list = L.rec + align256((size_t)rows * sizeof(sv::RowRec));
  L.race_job = L.list + align256((size_t)rows * sv::kListCap * sizeof(sv::ListEntry));
  L.race_part = L.race_job + align256((size_t)R * sizeof(int32_t));
  L.race_zn = L.race_part + align256((size_t)R * sv::kMaxRaceSegs * sizeof(sv::RacePart));
  L.block_w = L.race_zn + align256((size_t)R * sizeof(double));
  L.keys = L.block_w + align256((size_t)rows * 2 * sizeof(double));
  L.total = L.keys + align256((size_t)(R * block) * sizeof(uint64_t)) + 256;
  return L;
}

// ---- scratch of the allocation-free verify entry point
// One copy per device (the runtime places it when the library's code object
// loads on that device; it stays until the process ends), sized for
// kStaticMaxRows rows and kStaticMaxRequests requests.  Host code never uses
// the symbol's name as an address: the device address comes from
// hipGetSymbolAddress, looked up once per device.
constexpr int kStaticMaxRows = 1024;
constexpr int kStaticMaxRequests = 1024;
constexpr size_t kStaticScratchBytes = layout(kStaticMaxRows, kStaticMaxRequests, 0).total;
static_assert(kStaticScratchBytes <= (size_t)34 << 20, "scratch stays modest");

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Workgroups per full-vocabulary race: none when no request can need one
// (every request greedy, or every kept set bounded by a list), else one per
// kRaceSegElems elements (at least two).
int race_segments(int V, uint32_t flags) {
  if (flags & (SV_ALL_GREEDY | SV_LIST_BOUNDED)) return 0;
  int s = (V + sv::kRaceSegElems - 1) / sv::kRaceSegElems;
  if (s > sv::kMaxRaceSegs) s = sv::kMaxRaceSegs;
  return s < 2 ? 0 : s;
}

// ---- optional event timing
struct Prof {
  std::mutex mu;
  bool on = false;
  struct Rec { int id; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;  // reused events (created once)
  int64_t launches[10] = {};
  double ms[10] = {};
};
Prof& prof() {
  static Prof p;
  return p;
}

// Launch a kernel; with timing on, the dispatch itself stamps a pair of
// pooled events (begin and end of the kernel, no extra stream packets).
template <class... KArgs, class... Args>
void launch(int id, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
            Args... args) {
  Prof& p = prof();
  hipEvent_t ev[2] = {nullptr, nullptr};
  {
    std::lock_guard<std::mutex> g(p.mu);
    if (p.on) {
      for (hipEvent_t& e : ev) {
        if (!p.pool.empty()) {
          e = p.pool.back();
          p.pool.pop_back();
        } else if (hipEventCreate(&e) != hipSuccess) {
          e = nullptr;
        }
      }
    }
  }
  if (ev[0] && ev[1]) {
    // the start stamp is taken when the dispatch is processed, which may be
    // while the previous kernel on the stream still runs: let the stream
    // drain first so the pair brackets this kernel alone
    (void)hipStreamSynchronize(s);
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev[0], ev[1], 0, args...);
    std::lock_guard<std::mutex> g(p.mu);
    p.pending.push_back({id, ev[0], ev[1]});
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
    std::lock_guard<std::mutex> g(p.mu);
    for (hipEvent_t e : ev)
      if (e) p.pool.push_back(e);
  }
}

int32_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return SV_ERR_HIP;
  }
  return SV_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Row-pass workgroups resident at once on the current device.
int resident_row_workgroups() {
  static std::atomic<int> cached[64];  // CU count per device (0: not read yet)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int cus = dev < 64 ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus * sv::kRowPassPerCU;
}

}  // namespace

// The allocation-free entry point's scratch (see kStaticScratchBytes).
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

extern "C" {

const char* spec_verify_status_string(int32_t code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "null pointer";
    case SV_ERR_SHAPE: return "bad size or leading dimension";
    case SV_ERR_DTYPE: return "bad dtype or alignment";
    case SV_ERR_WORKSPACE: return "workspace too small";
    case SV_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* spec_verify_last_error(void) { return g_last_error.c_str(); }

size_t spec_verify_workspace_bytes(int32_t num_rows, int32_t vocab, int32_t num_requests,
                                   int32_t block) {
  (void)vocab;
  if (num_rows < 0) num_rows = 0;
  if (num_requests < 0) num_requests = 0;
  if (block < 0) block = 0;
  return layout(num_rows, num_requests, block).total;
}

static int32_t check_common(const void* logits, sv_dtype dt, int64_t ld, int32_t rows, int32_t V,
                            const int32_t* qo, int32_t R, const sv_sampling* sp) {
  if (!sp) return fail(SV_ERR_NULL, "sampling parameters are NULL");
  if (dt != SV_F32 && dt != SV_BF16) return fail(SV_ERR_DTYPE, "unknown logit dtype");
  if (rows < 0 || R < 0) return fail(SV_ERR_SHAPE, "negative row or request count");
  if (V <= 0) return fail(SV_ERR_SHAPE, "vocab must be positive");
  if (ld < V) return fail(SV_ERR_SHAPE, "ld_logits < vocab");
  if (R > 0 && !qo) return fail(SV_ERR_NULL, "qo_indptr is NULL");
  if (rows > 0 && !logits) return fail(SV_ERR_NULL, "logits are NULL");
  if (logits && !aligned(logits, dt == SV_BF16 ? 2 : 4))
    return fail(SV_ERR_DTYPE, "logits pointer misaligned for its dtype");
  if (rows > 0 && R == 0) return fail(SV_ERR_SHAPE, "rows without requests");
  return SV_OK;
}

static sv::VerifyArgs base_args(const void* logits, sv_dtype dt, int64_t ld, int32_t V,
                                const int32_t* qo, int32_t R, int32_t rows,
                                const sv_sampling* sp, void* ws) {
  sv::VerifyArgs A;
  std::memset(&A, 0, sizeof(A));
  A.logits = logits;
  A.ld_logits = ld;
  A.vocab = V;
  A.dtype = dt == SV_BF16 ? 1 : 0;
  A.qo = qo;
  A.num_requests = R;
  A.num_rows = rows;
  A.temperature = sp->temperature;
  A.top_k = sp->top_k;
  A.top_p = sp->top_p;
  A.request_id = sp->request_id;
  A.position0 = sp->position0;
  A.row_order = sp->row_order;
  A.seed = sp->seed;
  Layout L = layout(rows, R, 0);
  A.rec = (sv::RowRec*)((char*)ws + L.rec);
  A.list = (sv::ListEntry*)((char*)ws + L.list);
  A.race_job = (int32_t*)((char*)ws + L.race_job);
  A.race_part = (sv::RacePart*)((char*)ws + L.race_part);
  A.race_zn = (double*)((char*)ws + L.race_zn);
  A.race_nseg = (int32_t*)((char*)ws + 4);  // header bytes [4, 8)
  A.block_w = (double*)((char*)ws + L.block_w);
  A.block = (sp->flags & SV_BLOCK_VERIFY) ? 1 : 0;
  A.check = (sp->flags & SV_CHECK) ? (const int32_t*)ws : nullptr;
  return A;
}

// SV_CHECK: the layout check writes the workspace's check word before the
// call's kernels, which read it and refuse a failed layout.
static int32_t launch_check(const int32_t* qo, int32_t R, int32_t rows, void* ws, hipStream_t s) {
  launch(8, sv::check_layout_kernel, dim3(1), dim3(1024), s, qo, R, rows, (int32_t*)ws);
  return check_launch("layout check");
}

int32_t spec_verify_build_target_probs(const void* logits, sv_dtype dt, int64_t ld_logits,
                                       int32_t num_rows, int32_t vocab,
                                       const int32_t* qo_indptr, int32_t num_requests,
                                       const sv_sampling* sp, float* probs, int64_t ld_probs,
                                       float* row_max, int32_t* row_argmax, float* row_lse,
                                       int32_t* kept_count, int32_t* kept_idx, int32_t kmax,
                                       void* workspace, size_t workspace_bytes,
                                       sv_stream_t stream) {
  int32_t rc = check_common(logits, dt, ld_logits, num_rows, vocab, qo_indptr, num_requests, sp);
  if (rc) return rc;
  if (probs && ld_probs < vocab) return fail(SV_ERR_SHAPE, "ld_probs < vocab");
  if (kmax < 0 || kmax > sv::kKmaxCap) return fail(SV_ERR_SHAPE, "kmax must be in [0, 1024]");
  if (kept_idx && kmax == 0) return fail(SV_ERR_SHAPE, "kept_idx needs kmax > 0");
  if (num_rows == 0) return SV_OK;
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < spec_verify_workspace_bytes(num_rows, vocab, num_requests, 0))
    return fail(SV_ERR_WORKSPACE, "workspace smaller than spec_verify_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(SV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  sv::VerifyArgs A = base_args(logits, dt, ld_logits, vocab, qo_indptr, num_requests, num_rows,
                               sp, workspace);
  A.build = 1;
  if (A.check && (rc = launch_check(qo_indptr, num_requests, num_rows, workspace, s))) return rc;
  launch(0, sv::row_pass_kernel, dim3(num_rows), dim3(sv::kRowBlock), s, A);
  if ((rc = check_launch("row pass"))) return rc;
  sv::BuildOutArgs B;
  B.probs = probs;
  B.ld_probs = ld_probs;
  B.row_max = row_max;
  B.row_argmax = row_argmax;
  B.row_lse = row_lse;
  B.kept_count = kept_count;
  B.kept_idx = kept_idx;
  B.kmax = kept_idx ? kmax : 0;
  launch(2, sv::build_out_kernel, dim3(num_rows), dim3(sv::kRowBlock), s, A, B);
  return check_launch("build outputs");
}

int32_t spec_verify_rejection_sample(const void* target_logits, sv_dtype dt, int64_t ld_logits,
                                     int32_t vocab, const int32_t* qo_indptr,
                                     int32_t num_requests, int32_t num_rows,
                                     const int32_t* draft_tokens, const float* draft_probs,
                                     int64_t ld_q, const int32_t* verify_cap,
                                     const sv_sampling* sp, int32_t* accept_len,
                                     int32_t* out_tokens, int32_t* next_token,
                                     uint8_t* row_flags, void* workspace,
                                     size_t workspace_bytes, sv_stream_t stream) {
  int32_t rc = check_common(target_logits, dt, ld_logits, num_rows, vocab, qo_indptr,
                            num_requests, sp);
  if (rc) return rc;
  if (num_rows > 0 && !draft_tokens) return fail(SV_ERR_NULL, "draft_tokens are NULL");
  if (num_requests > 0 && (!accept_len || !next_token))
    return fail(SV_ERR_NULL, "accept_len / next_token are NULL");
  if (num_rows > 0 && !out_tokens) return fail(SV_ERR_NULL, "out_tokens are NULL");
  if (!draft_probs && !(sp->flags & SV_ALL_GREEDY))
    return fail(SV_ERR_NULL, "draft_probs is NULL without SV_ALL_GREEDY");
  if (draft_probs && ld_q < vocab) return fail(SV_ERR_SHAPE, "ld_q < vocab");
  if (draft_probs && !aligned(draft_probs, 4)) return fail(SV_ERR_DTYPE, "draft_probs misaligned");
  if (num_requests == 0) return SV_OK;
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < spec_verify_workspace_bytes(num_rows, vocab, num_requests, 0))
    return fail(SV_ERR_WORKSPACE, "workspace smaller than spec_verify_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(SV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  sv::VerifyArgs A = base_args(target_logits, dt, ld_logits, vocab, qo_indptr, num_requests,
                               num_rows, sp, workspace);
  A.build = 0;
  A.draft_tokens = draft_tokens;
  A.draft_probs = draft_probs;
  A.ld_q = ld_q;
  A.verify_cap = verify_cap;
  A.accept_len = accept_len;
  A.out_tokens = out_tokens;
  A.next_token = next_token;
  A.row_flags = row_flags;
  if (!draft_probs) A.temperature = nullptr;  // SV_ALL_GREEDY: every request greedy
  A.race_segs = draft_probs ? race_segments(vocab, sp->flags) : 0;
  A.level = num_rows <= resident_row_workgroups() ? 1 : 0;
  if (A.check && (rc = launch_check(qo_indptr, num_requests, num_rows, workspace, s))) return rc;
  if (num_rows > 0) launch(0, sv::row_pass_kernel, dim3(num_rows), dim3(sv::kRowBlock), s, A);
  if ((rc = check_launch("row pass"))) return rc;
  launch(1, A.block ? sv::finalize_block_kernel : sv::finalize_kernel, dim3(num_requests),
         dim3(sv::kRowBlock), s, A);
  if ((rc = check_launch("finalize"))) return rc;
  if (A.race_segs > 0) {
    const int items = A.race_segs * num_requests;
    launch(5, sv::race_segment_kernel, dim3(items < sv::kRaceGrid ? items : sv::kRaceGrid),
           dim3(sv::kRowBlock), s, A);
    if ((rc = check_launch("race segments"))) return rc;
    launch(6, sv::race_finish_kernel, dim3(num_requests), dim3(sv::kRowBlock), s, A);
    if ((rc = check_launch("race finish"))) return rc;
  }
  return SV_OK;
}

int32_t spec_verify_rejection_sample_noalloc(const void* target_logits, sv_dtype dt,
                                             int64_t ld_logits, int32_t vocab,
                                             const int32_t* qo_indptr, int32_t num_requests,
                                             int32_t num_rows, const int32_t* draft_tokens,
                                             const float* draft_probs, int64_t ld_q,
                                             const int32_t* verify_cap, const sv_sampling* sp,
                                             int32_t* accept_len, int32_t* out_tokens,
                                             int32_t* next_token, uint8_t* row_flags,
                                             sv_stream_t stream) {
  if (num_rows > kStaticMaxRows || num_requests > kStaticMaxRequests)
    return fail(SV_ERR_SHAPE, "the allocation-free entry point takes at most 1024 rows and "
                              "1024 requests");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(SV_ERR_HIP, "no current device (or a device index above 63)");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      // first call on this device (it is current): the device's own address
      // of the scratch array
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        g_last_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
        return SV_ERR_HIP;
      }
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return spec_verify_rejection_sample(target_logits, dt, ld_logits, vocab, qo_indptr,
                                      num_requests, num_rows, draft_tokens, draft_probs, ld_q,
                                      verify_cap, sp, accept_len, out_tokens, next_token,
                                      row_flags, ws, kStaticScratchBytes, stream);
}

int32_t spec_verify_plan_windows(const float* confidence, int64_t ld_conf, int32_t num_requests,
                                 int32_t block, int32_t budget, int32_t* verify_len,
                                 int32_t* qo_indptr, float* survival, void* workspace,
                                 size_t workspace_bytes, sv_stream_t stream) {
  if (num_requests < 0 || block < 0) return fail(SV_ERR_SHAPE, "negative size");
  if ((int64_t)num_requests * (int64_t)block >= (int64_t)1 << 31)
    return fail(SV_ERR_SHAPE, "num_requests * block must be < 2^31");
  if (!qo_indptr) return fail(SV_ERR_NULL, "qo_indptr is NULL");
  if (num_requests > 0 && (!verify_len || (block > 0 && !confidence)))
    return fail(SV_ERR_NULL, "confidence / verify_len are NULL");
  if (num_requests > 0 && ld_conf < block) return fail(SV_ERR_SHAPE, "ld_conf < block");
  const Layout L = layout(0, num_requests, block);
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < L.total) return fail(SV_ERR_WORKSPACE, "workspace too small");
  if (!aligned(workspace, 256)) return fail(SV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  sv::PlanArgs A;
  A.conf = confidence;
  A.ld_conf = ld_conf;
  A.num_requests = num_requests;
  A.block = block;
  A.budget = budget;
  A.verify_len = verify_len;
  A.qo_indptr = qo_indptr;
  A.survival = survival;
  A.keys = (uint64_t*)((char*)workspace + L.keys);
  launch(3, sv::plan_kernel, dim3(1), dim3(sv::kPlanBlock), s, A);
  return check_launch("planner");
}

int32_t spec_verify_plan_budget(const float* confidence, int64_t ld_conf, int32_t num_requests,
                                int32_t block, const float* cost, int32_t ncost, int32_t* budget,
                                double* theta, void* workspace, size_t workspace_bytes,
                                sv_stream_t stream) {
  if (num_requests < 0 || block < 0 || ncost < 0) return fail(SV_ERR_SHAPE, "negative size");
  const int64_t n = (int64_t)num_requests * block;
  if (n > sv::kBudgetMaxN) return fail(SV_ERR_SHAPE, "num_requests * block must be <= 2^20");
  if (!budget) return fail(SV_ERR_NULL, "budget is NULL");
  if (n > 0 && !confidence) return fail(SV_ERR_NULL, "confidence is NULL");
  if (num_requests > 0 && ld_conf < block) return fail(SV_ERR_SHAPE, "ld_conf < block");
  if (ncost > 0 && !cost) return fail(SV_ERR_NULL, "cost is NULL with ncost > 0");
  if (cost && ncost > 0 && (int64_t)ncost < n + num_requests + 1)
    return fail(SV_ERR_SHAPE, "cost table shorter than num_requests * block + num_requests + 1");
  hipStream_t s = (hipStream_t)stream;
  const float* tab = ncost > 0 ? cost : nullptr;
  if (n <= sv::kBudgetMaxKeys) {
    launch(3, sv::budget_kernel, dim3(1), dim3(sv::kPlanBlock), s, confidence, ld_conf,
           num_requests, block, tab, budget, theta);
    return check_launch("cost-table budget");
  }
  // tiles and the rank-ordered keys share the planner's key region (8 bytes
  // per position)
  const Layout L = layout(0, num_requests, block);
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL (R * block > 4096)");
  if (workspace_bytes < L.total) return fail(SV_ERR_WORKSPACE, "workspace too small");
  if (!aligned(workspace, 256)) return fail(SV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  uint32_t* tiles = (uint32_t*)((char*)workspace + L.keys);
  uint32_t* sorted = tiles + n;
  const int nt = (int)((n + sv::kBudgetMaxKeys - 1) / sv::kBudgetMaxKeys);
  int32_t rc;
  launch(3, sv::budget_tile_kernel, dim3(nt), dim3(sv::kPlanBlock), s, confidence, ld_conf,
         num_requests, block, tiles);
  if ((rc = check_launch("budget tiles"))) return rc;
  launch(3, sv::budget_rank_kernel, dim3((unsigned)((n + sv::kPlanBlock - 1) / sv::kPlanBlock)),
         dim3(sv::kPlanBlock), s, (const uint32_t*)tiles, (int32_t)n, sorted);
  if ((rc = check_launch("budget ranks"))) return rc;
  launch(3, sv::budget_scan_kernel, dim3(1), dim3(sv::kPlanBlock), s, (const uint32_t*)sorted,
         num_requests, (int32_t)n, tab, budget, theta);
  return check_launch("budget scan");
}

int32_t spec_verify_accept_prefix(const uint8_t* accepted, const int32_t* qo_indptr,
                                  int32_t num_requests, const int32_t* verify_cap,
                                  int32_t* accept_len, sv_stream_t stream) {
  if (num_requests < 0) return fail(SV_ERR_SHAPE, "negative request count");
  if (num_requests == 0) return SV_OK;
  if (!accepted || !qo_indptr || !accept_len) return fail(SV_ERR_NULL, "null pointer");
  hipStream_t s = (hipStream_t)stream;
  launch(4, sv::accept_prefix_kernel, dim3((num_requests + 3) / 4), dim3(256), s, accepted,
         qo_indptr, num_requests, verify_cap, accept_len);
  return check_launch("accept prefix");
}

int32_t spec_verify_check_layout(const int32_t* qo_indptr, int32_t num_requests,
                                 int32_t num_rows, int32_t* error_word, sv_stream_t stream) {
  if (num_requests < 0 || num_rows < 0) return fail(SV_ERR_SHAPE, "negative size");
  if (!qo_indptr || !error_word) return fail(SV_ERR_NULL, "qo_indptr / error_word are NULL");
  launch(8, sv::check_layout_kernel, dim3(1), dim3(1024), (hipStream_t)stream, qo_indptr,
         num_requests, num_rows, error_word);
  return check_launch("layout check");
}

int32_t spec_verify_row_diagnostics(const void* workspace, size_t workspace_bytes,
                                    int32_t num_rows, double* row_zk, double* row_zn,
                                    double* row_pd, int32_t* row_mode, sv_stream_t stream) {
  if (num_rows < 0) return fail(SV_ERR_SHAPE, "negative row count");
  if (num_rows == 0) return SV_OK;
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  const Layout L = layout(num_rows, 0, 0);
  if (workspace_bytes < L.list) return fail(SV_ERR_WORKSPACE, "workspace too small for the rows");
  const int grid = (num_rows + 255) / 256 < 1024 ? (num_rows + 255) / 256 : 1024;
  launch(9, sv::diagnostics_kernel, dim3(grid), dim3(256), (hipStream_t)stream,
         (const sv::RowRec*)((const char*)workspace + L.rec), num_rows, row_zk, row_zn, row_pd,
         row_mode);
  return check_launch("row diagnostics");
}

int32_t spec_verify_acceptance_stats(const int32_t* accept_len, const int32_t* verify_len,
                                     int32_t num_requests, int32_t block, int64_t* stats,
                                     sv_stream_t stream) {
  if (num_requests < 0 || block < 0) return fail(SV_ERR_SHAPE, "negative size");
  if (block > sv::kPlanBlock) return fail(SV_ERR_SHAPE, "block must be <= 1024");
  if ((int64_t)num_requests * (int64_t)block >= (int64_t)1 << 31)
    return fail(SV_ERR_SHAPE, "num_requests * block must be < 2^31");
  if (!stats) return fail(SV_ERR_NULL, "stats is NULL");
  if (num_requests > 0 && (!accept_len || !verify_len))
    return fail(SV_ERR_NULL, "accept_len / verify_len are NULL");
  hipStream_t s = (hipStream_t)stream;
  launch(7, sv::acceptance_stats_kernel, dim3(1), dim3(sv::kPlanBlock), s, accept_len, verify_len,
         num_requests, block, stats);
  return check_launch("acceptance statistics");
}

size_t spec_verify_estimator_state_doubles(int32_t block) {
  return block < 1 ? 0 : (size_t)sv::kEstStateBase + 5 * (size_t)block;
}

static int32_t check_est_block(int32_t block) {
  if (block < 1 || block > sv::kEstMaxBlock) return fail(SV_ERR_SHAPE, "block must be in [1, 64]");
  return SV_OK;
}

int32_t spec_verify_estimator_init(double* state, int32_t block, sv_stream_t stream) {
  int32_t rc = check_est_block(block);
  if (rc) return rc;
  if (!state) return fail(SV_ERR_NULL, "state is NULL");
  launch(7, sv::est_init_kernel, dim3(1), dim3(64), (hipStream_t)stream, state, block);
  return check_launch("estimator init");
}

int32_t spec_verify_estimator_predict(const float* row_max, const float* row_lse,
                                      const float* temperature, int32_t num_requests,
                                      int32_t block, const double* state, double* feature,
                                      float* confidence, sv_stream_t stream) {
  int32_t rc = check_est_block(block);
  if (rc) return rc;
  if (num_requests < 0) return fail(SV_ERR_SHAPE, "negative request count");
  if ((int64_t)num_requests * (int64_t)block >= (int64_t)1 << 31)
    return fail(SV_ERR_SHAPE, "num_requests * block must be < 2^31");
  if (!state) return fail(SV_ERR_NULL, "state is NULL");
  if (num_requests == 0) return SV_OK;
  if (!row_max || !row_lse) return fail(SV_ERR_NULL, "row_max / row_lse are NULL");
  const int64_t n = (int64_t)num_requests * block;
  const int64_t grid = (n + 255) / 256;
  launch(7, sv::est_predict_kernel, dim3((unsigned)(grid < 4096 ? grid : 4096)), dim3(256),
         (hipStream_t)stream, row_max, row_lse, temperature, num_requests, block, state, feature,
         confidence);
  return check_launch("estimator predict");
}

int32_t spec_verify_estimator_observe(const double* feature, const int32_t* accept_len,
                                      const int32_t* verify_len, int32_t num_requests,
                                      int32_t block, double* state, sv_stream_t stream) {
  int32_t rc = check_est_block(block);
  if (rc) return rc;
  if (num_requests < 0) return fail(SV_ERR_SHAPE, "negative request count");
  if ((int64_t)num_requests * (int64_t)block >= (int64_t)1 << 31)
    return fail(SV_ERR_SHAPE, "num_requests * block must be < 2^31");
  if (!state) return fail(SV_ERR_NULL, "state is NULL");
  if (num_requests > 0 && (!feature || !accept_len || !verify_len))
    return fail(SV_ERR_NULL, "feature / accept_len / verify_len are NULL");
  launch(7, sv::est_observe_kernel, dim3(1), dim3(sv::kPlanBlock), (hipStream_t)stream, feature,
         accept_len, verify_len, num_requests, block, state);
  return check_launch("estimator observe");
}

int32_t spec_verify_profile_enable(int32_t on) {
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return SV_OK;
}

int32_t spec_verify_profile_reset(void) {
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (auto& r : p.pending) {
    (void)hipEventSynchronize(r.b);
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.pending.clear();
  for (int k = 0; k < 10; ++k) { p.launches[k] = 0; p.ms[k] = 0.0; }
  return SV_OK;
}

int32_t spec_verify_profile_read(int32_t kernel_id, int64_t* launches, double* total_ms) {
  if (kernel_id < 0 || kernel_id >= 10) return fail(SV_ERR_SHAPE, "kernel id out of range");
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (auto& r : p.pending) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(SV_ERR_HIP, "event synchronize");
    float ms = 0.0f;
    (void)hipEventElapsedTime(&ms, r.a, r.b);
    p.launches[r.id] += 1;
    p.ms[r.id] += ms;
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.pending.clear();
  if (launches) *launches = p.launches[kernel_id];
  if (total_ms) *total_ms = p.ms[kernel_id];
  return SV_OK;
}

}  // extern "C"
