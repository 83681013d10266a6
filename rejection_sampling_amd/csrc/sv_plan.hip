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

}  // namespace sv
