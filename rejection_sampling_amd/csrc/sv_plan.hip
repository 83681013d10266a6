// sv_plan.hip -- confidence planner and accepted-prefix kernels (gfx950).
//
// Planner (TensorRT-LLM PR #17056, first commit note): prefix survival is the
// cumulative product of per-position probabilities, and the batch's verify
// budget is handed out by global survival rank with a value-independent
// tie-break.  Each (r, j) gets one 64-bit key whose ascending order is
// (S desc, j asc, r asc); a radix select finds the budget-th smallest key and
// every request's window is the count of its keys at or below it -- always a
// prefix, since S is non-increasing along j.  One workgroup, no host sync.
#include "sv_device.hpp"
#include "sv_kernels.h"

namespace sv {

constexpr int kPB = kPlanBlock;
constexpr int kPW = kPB / 64;

__device__ __forceinline__ int pblock_exclusive_sum(int v, int* scr, int* total) {
  int incl = wave_inclusive_sum(v);
  __syncthreads();
  if (lane_id() == 63) scr[wave_id()] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kPW; ++w) {
    if (w < wave_id()) base += scr[w];
    tot += scr[w];
  }
  *total = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(kPB) void plan_kernel(PlanArgs A) {
  __shared__ uint32_t hist[256];
  __shared__ int scr[kPW];
  __shared__ int sel_digit, sel_need, sel_exact;
  const int tid = threadIdx.x;
  const int R = A.num_requests, B = A.block;
  const long n = (long)R * B;

  // survival, fp32, left to right; clamp to [0, 1], NaN -> 0
  for (int r = tid; r < R; r += kPB) {
    float acc = 1.0f;
    for (int j = 0; j < B; ++j) {
      float cf = A.conf[(size_t)r * A.ld_conf + j];
      cf = (cf > 0.0f) ? (cf < 1.0f ? cf : 1.0f) : 0.0f;
      acc = (j == 0) ? cf : __fmul_rn(acc, cf);
      if (A.survival) A.survival[(size_t)r * B + j] = acc;
      const uint32_t sb = __float_as_uint(acc);  // acc >= +0: bits order = value order
      A.keys[(size_t)r * B + j] = ((uint64_t)(~sb) << 32) | (uint64_t)(uint32_t)(j * R + r);
    }
  }
  __threadfence_block();
  __syncthreads();

  long take = A.budget < 0 ? 0 : (long)A.budget;
  if (take > n) take = n;
  uint64_t prefix = 0, pmask = 0;
  bool all = take == n, none = take == 0;
  if (!all && !none) {
    int need = (int)take;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kPB) hist[b] = 0u;
      __syncthreads();
      for (long t = tid; t < n; t += kPB) {
        const uint64_t k = A.keys[t];
        if ((k & pmask) == prefix) atomicAdd(&hist[(uint32_t)(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave_id() == 0) {
        const int l = lane_id();  // lane l owns digits 4l .. 4l+3, ascending
        const int h0 = (int)hist[4 * l], h1 = (int)hist[4 * l + 1];
        const int h2 = (int)hist[4 * l + 2], h3 = (int)hist[4 * l + 3];
        const int local = h0 + h1 + h2 + h3;
        const int incl = wave_inclusive_sum(local);
        const int excl = incl - local;
        const uint64_t mk = __ballot(excl < need && need <= incl);
        const int src = __ffsll((unsigned long long)mk) - 1;
        if (l == src) {
          int c = excl, d, hd;
          if (c + h0 >= need) { d = 4 * l; hd = h0; }
          else if ((c += h0) + h1 >= need) { d = 4 * l + 1; hd = h1; }
          else if ((c += h1) + h2 >= need) { d = 4 * l + 2; hd = h2; }
          else { c += h2; d = 4 * l + 3; hd = h3; }
          sel_digit = d;
          sel_need = need - c;
          sel_exact = hd == need - c;
        }
      }
      __syncthreads();
      const int d = sel_digit;
      need = sel_need;
      const int ex = sel_exact;
      prefix |= (uint64_t)d << shift;
      pmask |= (uint64_t)0xFF << shift;
      __syncthreads();
      if (ex) break;
    }
  }

  // windows, then the packed layout (one bonus row per request)
  int carry = 0;
  for (int r0 = 0; r0 < R; r0 += kPB) {
    const int r = r0 + tid;
    int vl = 0;
    if (r < R) {
      if (all) vl = B;
      else if (!none)
        for (int j = 0; j < B; ++j) vl += ((A.keys[(size_t)r * B + j] & pmask) <= prefix) ? 1 : 0;
      A.verify_len[r] = vl;
    }
    int total;
    const int ex = pblock_exclusive_sum(r < R ? vl + 1 : 0, scr, &total);
    if (r < R) A.qo_indptr[r] = carry + ex;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) A.qo_indptr[R] = carry;
}

// One wave per request: accept_len = first j < min(gamma, cap) with a zero byte.
__global__ __launch_bounds__(256) void accept_prefix_kernel(const uint8_t* accepted,
                                                            const int32_t* qo, int32_t R,
                                                            const int32_t* verify_cap,
                                                            int32_t* accept_len) {
  const int r = blockIdx.x * 4 + wave_id();
  if (r >= R) return;
  const int s = qo[r], e = qo[r + 1];
  int gamma = e - s - 1;
  gamma = gamma < 0 ? 0 : gamma;
  int cap = gamma;
  if (verify_cap) {
    const int cv = verify_cap[r];
    cap = cv < 0 ? 0 : (cv > gamma ? gamma : cv);
  }
  int L = cap;
  for (int j0 = 0; j0 < cap; j0 += 64) {
    const int j = j0 + lane_id();
    const bool rej = j < cap && accepted[s + j] == 0;
    const uint64_t mk = __ballot(rej);
    if (mk) {
      L = j0 + __ffsll((unsigned long long)mk) - 1;
      break;
    }
  }
  if (lane_id() == 0) accept_len[r] = L;
}

// Acceptance and trim statistics of one verify step (TensorRT-LLM PR #17056,
// commit note on the trim-regret metric; per-position acceptance as in the
// consolidation study, section 1).  One workgroup: each thread counts its
// requests (trimmed: window below the block; regret: trimmed with the whole
// window accepted) and bins their windows and accepted lengths in LDS; the
// per-position counts are suffix sums of those bins (positions j < w are
// offered, j < L accepted).  Integer counts only, so the result is exact.
__global__ __launch_bounds__(kPlanBlock) void acceptance_stats_kernel(
    const int32_t* accept_len, const int32_t* verify_len, int32_t R, int32_t B, int64_t* stats) {
  __shared__ uint32_t hw[kPB + 1], hl[kPB + 1];  // bins 0..B of windows and accepted lengths
  __shared__ uint32_t tot[4];
  const int tid = threadIdx.x;
  for (int v = tid; v <= B; v += kPB) { hw[v] = 0u; hl[v] = 0u; }
  if (tid < 4) tot[tid] = 0u;
  __syncthreads();
  uint32_t trimmed = 0u, regret = 0u, sum_l = 0u, sum_w = 0u;
  for (int r = tid; r < R; r += kPB) {
    int w = verify_len[r];
    w = w < 0 ? 0 : (w > B ? B : w);
    int L = accept_len[r];
    L = L < 0 ? 0 : (L > w ? w : L);
    if (w < B) {
      trimmed += 1u;
      if (L == w) regret += 1u;
    }
    sum_l += (uint32_t)L;
    sum_w += (uint32_t)w;
    atomicAdd(&hw[w], 1u);
    atomicAdd(&hl[L], 1u);
  }
  atomicAdd(&tot[0], trimmed);
  atomicAdd(&tot[1], regret);
  atomicAdd(&tot[2], sum_l);
  atomicAdd(&tot[3], sum_w);
  __syncthreads();
  // suffix sums over bins 1..B in place: after them hw[v] = #{w >= v}
  for (int d = 1; d < B; d <<= 1) {
    uint32_t a = 0u, b = 0u;
    const int v = tid + 1;
    if (v <= B && v + d <= B) { a = hw[v + d]; b = hl[v + d]; }
    __syncthreads();
    if (v <= B) { hw[v] += a; hl[v] += b; }
    __syncthreads();
  }
  if (tid == 0) {
    stats[0] = R;
    stats[1] = tot[0];
    stats[2] = tot[1];
    stats[3] = tot[2];
    stats[4] = tot[3];
  }
  for (int j = tid; j < B; j += kPB) {
    stats[5 + j] = hw[j + 1];      // offered: w > j
    stats[5 + B + j] = hl[j + 1];  // accepted: L > j
  }
}

// ------------------------------------------------------------ estimator
// Online acceptance estimator (SGLang PR "Adaptive verification for DFLASH",
// commit notes adding OnlineAcceptanceEstimator and fixing its slope refit):
// p_k = sigmoid(slope * x_k + bias_k), x_k = logit(q_max) of the draft
// distribution at position k.  The state is one device array of doubles (see
// EstLayout); a single workgroup applies every update in a fixed order, so
// the same inputs always give the same coefficients, and the refit counter
// lives in the state, so nothing waits on the host.
struct EstLayout {
  int B;
  __device__ __forceinline__ explicit EstLayout(int b) : B(b) {}
  __device__ __forceinline__ int slope() const { return 0; }
  __device__ __forceinline__ int bias(int k) const { return 1 + k; }
  __device__ __forceinline__ int h_ss() const { return 1 + B; }
  __device__ __forceinline__ int g_s() const { return 2 + B; }
  __device__ __forceinline__ int n_s() const { return 3 + B; }
  __device__ __forceinline__ int h_sk(int k) const { return 4 + B + k; }
  __device__ __forceinline__ int h_kk(int k) const { return 4 + 2 * B + k; }
  __device__ __forceinline__ int g_k(int k) const { return 4 + 3 * B + k; }
  __device__ __forceinline__ int n_k(int k) const { return 4 + 4 * B + k; }
  __device__ __forceinline__ int calls() const { return 4 + 5 * B; }
  __device__ __forceinline__ int refits() const { return 5 + 5 * B; }
};

__device__ __forceinline__ double est_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

__global__ void est_init_kernel(double* st, int32_t B) {
  const EstLayout L(B);
  for (int t = threadIdx.x; t < kEstStateBase + 5 * B; t += blockDim.x) st[t] = 0.0;
  __syncthreads();
  if (threadIdx.x == 0) st[L.slope()] = 0.5;
  for (int k = threadIdx.x; k < B; k += blockDim.x) st[L.bias(k)] = -0.2;
}

// Feature and prediction of every drafted position (row r * B + k of the
// draft build): x = logit(exp(m / T - lse)) clamped to [-40, 40], with T = 1
// for greedy requests; confidence = sigmoid(slope * x + bias_k) in fp32, the
// planner's input.
__global__ void est_predict_kernel(const float* row_max, const float* row_lse,
                                   const float* temperature, int32_t R, int32_t B,
                                   const double* st, double* feature, float* confidence) {
  const EstLayout L(B);
  const long long n = (long long)R * B;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const int r = (int)(i / B), k = (int)(i - (long long)r * B);
    const float t = temperature ? temperature[r] : 0.0f;
    const double T = t > 0.0f ? (double)t : 1.0;
    const double lq = (double)row_max[i] / T - (double)row_lse[i];
    double x = lq - log1p(-exp(lq));
    if (!(x <= 40.0)) x = 40.0;
    if (x < -40.0) x = -40.0;
    if (feature) feature[i] = x;
    if (confidence) confidence[i] = (float)est_sigmoid(st[L.slope()] * x + st[L.bias(k)]);
  }
}

// One step's observations (labels 1 for the accepted drafts, 0 for the first
// rejected one) added to the IRLS statistics at the current coefficients;
// every kEstRefit calls the refit.  One workgroup: per position, each wave
// sums its lanes by a DPP scan and the waves' sums are added in wave order.
__global__ __launch_bounds__(kPlanBlock) void est_observe_kernel(
    const double* feature, const int32_t* accept_len, const int32_t* verify_len, int32_t R,
    int32_t B, double* st) {
  const EstLayout L(B);
  __shared__ double part[kPW][4];
  __shared__ double tot[kPW][3];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const double slope = st[L.slope()];
  double h_ss = 0.0, g_s = 0.0, n_s = 0.0;
  for (int k = 0; k < B; ++k) {
    const double bk = st[L.bias(k)];
    double hsk = 0.0, hkk = 0.0, gk = 0.0, nk = 0.0;
    for (int r = tid; r < R; r += kPB) {
      int wr = verify_len[r];
      wr = wr < 0 ? 0 : (wr > B ? B : wr);
      int lr = accept_len[r];
      lr = lr < 0 ? 0 : (lr > wr ? wr : lr);
      const int last = lr < wr ? lr : lr - 1;
      if (k > last) continue;
      const double x = feature[(size_t)r * B + k];
      const double y = k < lr ? 1.0 : 0.0;
      const double p = est_sigmoid(slope * x + bk);
      const double wt = p * (1.0 - p);
      h_ss += wt * x * x;
      hsk += wt * x;
      hkk += wt;
      g_s += (y - p) * x;
      gk += y - p;
      n_s += 1.0;
      nk += 1.0;
    }
    hsk = readlane_d(wave_scan_dpp(hsk), 63);
    hkk = readlane_d(wave_scan_dpp(hkk), 63);
    gk = readlane_d(wave_scan_dpp(gk), 63);
    nk = readlane_d(wave_scan_dpp(nk), 63);
    if (l == 0) { part[w][0] = hsk; part[w][1] = hkk; part[w][2] = gk; part[w][3] = nk; }
    __syncthreads();
    if (tid == 0) {
      double a = 0.0, b = 0.0, c = 0.0, d = 0.0;
      for (int q = 0; q < kPW; ++q) { a += part[q][0]; b += part[q][1]; c += part[q][2]; d += part[q][3]; }
      st[L.h_sk(k)] += a;
      st[L.h_kk(k)] += b;
      st[L.g_k(k)] += c;
      st[L.n_k(k)] += d;
    }
    __syncthreads();
  }
  h_ss = readlane_d(wave_scan_dpp(h_ss), 63);
  g_s = readlane_d(wave_scan_dpp(g_s), 63);
  n_s = readlane_d(wave_scan_dpp(n_s), 63);
  if (l == 0) { tot[w][0] = h_ss; tot[w][1] = g_s; tot[w][2] = n_s; }
  __syncthreads();
  if (tid != 0) return;
  {
    double a = 0.0, b = 0.0, c = 0.0;
    for (int q = 0; q < kPW; ++q) { a += tot[q][0]; b += tot[q][1]; c += tot[q][2]; }
    st[L.h_ss()] += a;
    st[L.g_s()] += b;
    st[L.n_s()] += c;
  }
  st[L.calls()] += 1.0;
  if (st[L.calls()] < (double)kEstRefit) return;
  // refit: arrowhead Newton solve with a ridge (Schur complement on the slope)
  const double ridge = 1e-3;
  double a = st[L.h_ss()] + ridge, g = st[L.g_s()];
  for (int k = 0; k < B; ++k) {
    const double dk = st[L.h_kk(k)] + ridge;
    a -= st[L.h_sk(k)] * st[L.h_sk(k)] / dk;
    g -= st[L.h_sk(k)] * st[L.g_k(k)] / dk;
  }
  const double ns = st[L.n_s()];
  double step = (g / a) * (ns / (ns + 50.0));
  if (!isfinite(step)) step = 0.0;
  const double s0 = st[L.slope()];
  for (int h = 0; h < 8 && s0 + step < 0.0; ++h) step *= 0.5;
  if (s0 + step < 0.0) step = 0.0;
  for (int k = 0; k < B; ++k) {
    const double dk = st[L.h_kk(k)] + ridge;
    const double nk = st[L.n_k(k)];
    double sb = ((st[L.g_k(k)] - st[L.h_sk(k)] * step) / dk) * (nk / (nk + 50.0));
    if (!isfinite(sb)) sb = 0.0;
    st[L.bias(k)] += sb;
  }
  st[L.slope()] = s0 + step;
  st[L.h_ss()] = st[L.g_s()] = st[L.n_s()] = 0.0;
  for (int k = 0; k < B; ++k) st[L.h_sk(k)] = st[L.h_kk(k)] = st[L.g_k(k)] = st[L.n_k(k)] = 0.0;
  st[L.calls()] = 0.0;
  st[L.refits()] += 1.0;
}

}  // namespace sv
