// sv_plan.hip -- confidence planner and accepted-prefix kernels (gfx950).
//
// Planner (method: TensorRT-LLM PR #17056, first commit note).  S[r, j] is
// the running fp32 product of request r's clamped confidences up to position
// j.  Every (r, j) gets one 64-bit key, ordered by S descending, then j, then
// r, so equal values are ranked by position and request, never by value
// noise.  A radix select finds the budget-th smallest key; request r verifies
// the positions whose keys are at or below it, which are always its first
// ones because S never grows along j.  One workgroup, no host sync.
#include "sv_device.hpp"
#include "sv_kernels.h"

namespace sv {

constexpr int kPB = kPlanBlock;
constexpr int kPW = kPB / 64;
constexpr int kKeyRegs = 8;     // planner keys held per thread (n <= 8192 stays in registers)
constexpr int kLdsKeys = 4096;  // planner keys staged in LDS instead of the workspace
constexpr int kConfBatch = 8;   // planner confidences loaded per batch

__device__ __forceinline__ int pblock_exclusive_sum(int v, int* scr, int* total) {
  int incl = wave_scan_dpp(v);
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
  __shared__ uint32_t hist[2][256];  // one counts while the other is cleared
  __shared__ uint64_t lkeys[kLdsKeys];  // n <= kLdsKeys: key of (r, j) at j * R + r
  __shared__ int scr[kPW];
  __shared__ int sel_digit, sel_need, sel_exact;
  const int tid = threadIdx.x;
  const int R = A.num_requests, B = A.block;
  const long n = (long)R * B;
  const bool in_lds = n <= kLdsKeys;

  // survival, fp32, left to right; clamp to [0, 1], NaN -> 0 (confidences
  // loaded kConfBatch at a time so their latencies overlap)
  for (int r = tid; r < R; r += kPB) {
    float acc = 1.0f;
    for (int j0 = 0; j0 < B; j0 += kConfBatch) {
      float c[kConfBatch];
#pragma unroll
      for (int u = 0; u < kConfBatch; ++u)
        c[u] = j0 + u < B ? A.conf[(size_t)r * A.ld_conf + j0 + u] : 0.0f;
#pragma unroll
      for (int u = 0; u < kConfBatch; ++u) {
        const int j = j0 + u;
        if (j >= B) break;
        const float cf = (c[u] > 0.0f) ? (c[u] < 1.0f ? c[u] : 1.0f) : 0.0f;
        acc = (j == 0) ? cf : __fmul_rn(acc, cf);
        if (A.survival) A.survival[(size_t)r * B + j] = acc;
        const uint32_t sb = __float_as_uint(acc);  // acc >= +0: bits order = value order
        const uint64_t key = ((uint64_t)(~sb) << 32) | (uint64_t)(uint32_t)(j * R + r);
        if (in_lds) lkeys[j * R + r] = key;
        else A.keys[(size_t)r * B + j] = key;
      }
    }
  }
  if (!in_lds) __threadfence_block();
  __syncthreads();

  // up to kKeyRegs keys per thread (key t in thread t mod kPB) stay in
  // registers for the select's passes, spread over every wave
  const bool in_regs = n <= (long)kPB * kKeyRegs;
  uint64_t kr[kKeyRegs];
#pragma unroll
  for (int i = 0; i < kKeyRegs; ++i) {
    const long t = tid + (long)i * kPB;
    kr[i] = (in_regs && t < n) ? (in_lds ? lkeys[t] : A.keys[t]) : ~0ull;
  }

  long take = A.budget < 0 ? 0 : (long)A.budget;
  if (take > n) take = n;
  uint64_t prefix = 0, pmask = 0;
  bool all = take == n, none = take == 0;
  if (!all && !none) {
    int need = (int)take;
    for (int b = tid; b < 256; b += kPB) hist[0][b] = 0u;
    __syncthreads();
    int hb = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      uint32_t* h = hist[hb];
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < kKeyRegs; ++i) {
          const long t = tid + (long)i * kPB;
          const bool mine = t < n && (kr[i] & pmask) == prefix;
          const uint32_t dg = (uint32_t)(kr[i] >> shift) & 255u;
          // a wave whose matching keys share one digit adds them in one atomic
          const uint64_t act = __ballot(mine);
          if (act == 0) continue;
          const int first = __ffsll((unsigned long long)act) - 1;
          const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)dg, first);
          if (__ballot(mine && dg != d0) == 0) {
            if (lane_id() == first) atomicAdd(&h[d0], (uint32_t)__popcll(act));
          } else if (mine) {
            atomicAdd(&h[dg], 1u);
          }
        }
      } else {
        for (long t = tid; t < n; t += kPB) {
          const uint64_t k = A.keys[t];
          if ((k & pmask) == prefix) atomicAdd(&h[(uint32_t)(k >> shift) & 255u], 1u);
        }
      }
      // the other buffer was last read before the previous round's second barrier
      for (int b = tid; b < 256; b += kPB) hist[hb ^ 1][b] = 0u;
      __syncthreads();
      if (wave_id() == 0) {
        const int l = lane_id();  // lane l owns digits 4l .. 4l+3, ascending
        const int h0 = (int)h[4 * l], h1 = (int)h[4 * l + 1];
        const int h2 = (int)h[4 * l + 2], h3 = (int)h[4 * l + 3];
        const int local = h0 + h1 + h2 + h3;
        const int incl = wave_scan_dpp(local);
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
      hb ^= 1;
      if (ex) break;
    }
  }

  // windows, then the packed layout (one bonus row per request)
  int carry = 0;
  for (int r0 = 0; r0 < R; r0 += kPB) {
    const int r = r0 + tid;
    int vl = 0;
    if (r < R) {
      if (all)
        vl = B;
      else if (!none)
#pragma unroll 8
        for (int j = 0; j < B; ++j) {
          const uint64_t k = in_lds ? lkeys[j * R + r] : A.keys[(size_t)r * B + j];
          vl += ((k & pmask) <= prefix) ? 1 : 0;
        }
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

// Verify budget from a step-cost table (method: TensorRT-LLM PR #17056,
// description).  Expected tokens per unit of step cost are scored at every
// budget b in [0, R*B]: tau(b) = R + the b largest survivals, the step runs
// b + R verify rows, Theta(b) = tau(b) / cost[b + R].  Every b is scored
// because cost rises in steps, so Theta has a local peak at each step's right
// end; the largest Theta wins, the smaller budget on equal Theta.  The survivals are sorted as 32-bit keys ~bits(S)
// (ascending key = S descending; tau depends on the values only, so the
// planner's index tie-break among equal survivals needs no place in the key),
// summed in that order by a block scan (fp64), and a block argmax picks the
// budget.  Up to kBudgetMaxKeys positions one workgroup sorts them in LDS;
// beyond, tiles of kBudgetMaxKeys are sorted by one workgroup each, every key
// is placed at its global rank by binary search in the other tiles, and one
// workgroup scans the sorted keys.  A table equal over [R, R*B + R], or none,
// gives R*B; a non-positive or non-finite cost in that range gives budget -1.

// Survival of position (r, j): the planner's left-to-right fp32 product of the
// clamped confidences (NaN -> 0), bit for bit.
__device__ __forceinline__ float survival_at(const float* conf, int64_t ld_conf, int r, int j) {
  float acc = 1.0f;
  for (int t = 0; t <= j; ++t) {
    float cf = conf[(size_t)r * ld_conf + t];
    cf = (cf > 0.0f) ? (cf < 1.0f ? cf : 1.0f) : 0.0f;
    acc = (t == 0) ? cf : __fmul_rn(acc, cf);
  }
  return acc;
}

// Ascending bitonic sort of keys[0, np) (np a power of two <= 4 kPB; padding
// 0xFFFFFFFF sorts last) with the keys in registers: thread t owns
// i = t + m * kPB and computes each stage's new value of its own elements.  The
// partner i ^ jj is in the same thread for jj >= kPB, in the same wave for
// jj < 64 (a shuffle), and otherwise read through LDS between barriers.
__device__ void sort_keys_lds(uint32_t* keys, int np) {
  const int tid = threadIdx.x;
  uint32_t kv[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int i = tid + m * kPB;
    kv[m] = i < np ? keys[i] : 0xFFFFFFFFu;
  }
  for (int k = 2; k <= np; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      uint32_t pv[4];
      if (jj >= kPB) {
#pragma unroll
        for (int m = 0; m < 4; ++m) pv[m] = kv[m ^ (jj / kPB)];
      } else if (jj >= 64) {
        __syncthreads();  // the previous readers of keys are done
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (tid + m * kPB < np) keys[tid + m * kPB] = kv[m];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int i = tid + m * kPB;
          pv[m] = i < np ? keys[i ^ jj] : 0xFFFFFFFFu;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) pv[m] = (uint32_t)__shfl_xor((int)kv[m], jj, 64);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = tid + m * kPB;
        const bool keep_min = ((i & k) == 0) == ((i & jj) == 0);  // ascending run, lower index
        const uint32_t lo = kv[m] < pv[m] ? kv[m] : pv[m];
        const uint32_t hi = kv[m] < pv[m] ? pv[m] : kv[m];
        if (i < np) kv[m] = keep_min ? lo : hi;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 4; ++m)
    if (tid + m * kPB < np) keys[tid + m * kPB] = kv[m];
  __syncthreads();
}

// tau scan and block argmax over the n sorted keys key_at(i) (rank i holds the
// (i+1)-th best survival); writes budget and theta.  One workgroup.
template <class KeyAt>
__device__ void budget_argmax(KeyAt&& key_at, int n, int R, const float* cost, int32_t* budget,
                              double* theta) {
  __shared__ double wtot[kPW];
  __shared__ double wth[kPW];
  __shared__ int wb[kPW];
  __shared__ int bad_s, flat_s;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  if (tid == 0) { bad_s = 0; flat_s = 1; }
  __syncthreads();
  if (cost) {
    const float c0 = cost[R];
    for (int t = R + tid; t <= n + R; t += kPB) {
      const float c = cost[t];
      if (!(c > 0.0f) || !isfinite(c)) atomicOr(&bad_s, 1);
      if (c != c0) atomicAnd(&flat_s, 0);
    }
  }
  // thread t holds ranks [t * C, t * C + C): their survivals' sum, then a block scan
  const int C = (n + kPB - 1) / kPB;
  double loc = 0.0;
  for (int c = 0; c < C; ++c) {
    const int i = tid * C + c;
    if (i < n) loc += (double)__uint_as_float(~key_at(i));
  }
  const double incl = wave_scan_dpp(loc);
  if (l == 63) wtot[w] = incl;
  __syncthreads();
  double base = 0.0;
  for (int q = 0; q < w; ++q) base += wtot[q];
  double pre = (double)R + base + (incl - loc);  // tau of the budget before this thread's ranks
  double best_th = -1.0;
  int best_b = 0x7FFFFFFF;
  if (cost) {
    if (tid == 0) { best_th = (double)R / (double)cost[R]; best_b = 0; }
    for (int c = 0; c < C; ++c) {
      const int i = tid * C + c;
      if (i >= n) break;
      const float sv = __uint_as_float(~key_at(i));
      pre += (double)sv;
      // a zero survival on a stair that does not fall leaves Theta where the
      // budget before it had it: that smaller budget keeps the tie (tau is
      // rebuilt per thread, so its rounding must not decide here)
      if (sv == 0.0f && !(cost[i + 1 + R] < cost[i + R])) continue;
      const double th = pre / (double)cost[i + 1 + R];
      if (th > best_th) { best_th = th; best_b = i + 1; }
    }
  }
  // block argmax: larger Theta, then smaller budget
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const double ot = __shfl_xor(best_th, d, 64);
    const int ob = __shfl_xor(best_b, d, 64);
    if (ot > best_th || (ot == best_th && ob < best_b)) { best_th = ot; best_b = ob; }
  }
  if (l == 0) { wth[w] = best_th; wb[w] = best_b; }
  __syncthreads();
  if (tid == 0) {
    double bt = wth[0];
    int bb = wb[0];
    for (int q = 1; q < kPW; ++q)
      if (wth[q] > bt || (wth[q] == bt && wb[q] < bb)) { bt = wth[q]; bb = wb[q]; }
    if (cost && bad_s) {
      bb = -1;
      bt = __builtin_nan("");
    } else if (!cost || flat_s) {
      bb = n;
      double tau = (double)R;
      for (int q = 0; q < kPW; ++q) tau += wtot[q];
      bt = cost ? tau / (double)cost[n + R] : 0.0;
    }
    *budget = bb;
    if (theta) *theta = bt;
  }
}

__global__ __launch_bounds__(kPB) void budget_kernel(const float* conf, int64_t ld_conf, int32_t R,
                                                     int32_t B, const float* cost, int32_t* budget,
                                                     double* theta) {
  __shared__ uint32_t keys[kBudgetMaxKeys];  // ~bits(S): ascending = S descending
  const int tid = threadIdx.x;
  const int n = R * B;
  int np = 1;
  while (np < n) np <<= 1;
  for (int r = tid; r < R; r += kPB) {
    float acc = 1.0f;
    for (int j = 0; j < B; ++j) {
      float cf = conf[(size_t)r * ld_conf + j];
      cf = (cf > 0.0f) ? (cf < 1.0f ? cf : 1.0f) : 0.0f;
      acc = (j == 0) ? cf : __fmul_rn(acc, cf);
      keys[j * R + r] = ~__float_as_uint(acc);  // acc >= +0: bits order = value order
    }
  }
  for (int t = n + tid; t < np; t += kPB) keys[t] = 0xFFFFFFFFu;  // padding sorts last
  __syncthreads();
  sort_keys_lds(keys, np);
  budget_argmax([&](int i) { return keys[i]; }, n, R, cost, budget, theta);
}

// Large batches, step 1: tile t (flat positions t * kBudgetMaxKeys + i, i.e.
// (r, j) = divmod(position, B)) sorted in LDS and written to tiles[t * kBudgetMaxKeys ..].
__global__ __launch_bounds__(kPB) void budget_tile_kernel(const float* conf, int64_t ld_conf,
                                                          int32_t R, int32_t B, uint32_t* tiles) {
  __shared__ uint32_t keys[kBudgetMaxKeys];
  const int n = R * B;
  const int t0 = blockIdx.x * kBudgetMaxKeys;
  const int len = n - t0 < kBudgetMaxKeys ? n - t0 : kBudgetMaxKeys;
  int np = 1;
  while (np < len) np <<= 1;
  for (int i = threadIdx.x; i < np; i += kPB) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < len) {
      const int pidx = t0 + i;
      key = ~__float_as_uint(survival_at(conf, ld_conf, pidx / B, pidx % B));
    }
    keys[i] = key;
  }
  __syncthreads();
  sort_keys_lds(keys, np);
  for (int i = threadIdx.x; i < len; i += kPB) tiles[t0 + i] = keys[i];
}

// Large batches, step 2: key i of tile t goes to its global rank: i, plus the
// keys of every earlier tile at or below it, plus those of every later tile
// strictly below it (equal keys: earlier tiles first), found by binary search.
__global__ __launch_bounds__(kPB) void budget_rank_kernel(const uint32_t* tiles, int32_t n,
                                                          uint32_t* sorted) {
  const int g = blockIdx.x * kPB + threadIdx.x;
  if (g >= n) return;
  const int T = (n + kBudgetMaxKeys - 1) / kBudgetMaxKeys;
  const int t = g / kBudgetMaxKeys;
  const uint32_t k = tiles[g];
  int rank = g - t * kBudgetMaxKeys;
  for (int u = 0; u < T; ++u) {
    if (u == t) continue;
    const uint32_t* tk = tiles + (size_t)u * kBudgetMaxKeys;
    const int len = n - u * kBudgetMaxKeys < kBudgetMaxKeys ? n - u * kBudgetMaxKeys : kBudgetMaxKeys;
    // first index whose key is > k (u < t) or >= k (u > t)
    int lo = 0, hi = len;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const uint32_t km = tk[mid];
      const bool before = u < t ? km <= k : km < k;
      if (before) lo = mid + 1;
      else hi = mid;
    }
    rank += lo;
  }
  sorted[rank] = k;
}

// Large batches, step 3: the scan and argmax over the sorted keys.
__global__ __launch_bounds__(kPB) void budget_scan_kernel(const uint32_t* sorted, int32_t R,
                                                          int32_t n, const float* cost,
                                                          int32_t* budget, double* theta) {
  budget_argmax([&](int i) { return sorted[i]; }, n, R, cost, budget, theta);
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
// consolidation study, section 1).  One workgroup, integer counts only, so the
// result is exact.  Each thread takes its requests (trimmed: window below the
// block; regret: trimmed with the whole window accepted); per position j the
// offered count is #{w > j} and the accepted one #{L > j}: each wave counts
// its 64 requests by a ballot per j (lane j mod 64 keeps the count) until no
// window reaches j, and adds its counts to LDS, one address per lane.
__global__ __launch_bounds__(kPlanBlock) void acceptance_stats_kernel(
    const int32_t* accept_len, const int32_t* verify_len, int32_t R, int32_t B, int64_t* stats) {
  __shared__ uint32_t cw[kPB], cl[kPB];  // per position: offered, accepted
  __shared__ uint32_t tot[kPW][4];
  const int tid = threadIdx.x, wv = wave_id(), l = lane_id();
  for (int j = tid; j < B; j += kPB) { cw[j] = 0u; cl[j] = 0u; }
  __syncthreads();
  int trimmed = 0, regret = 0, sum_l = 0, sum_w = 0;
  for (int r0 = 0; r0 < R; r0 += kPB) {  // the same passes for every wave
    const int r = r0 + tid;
    int w = 0, L = 0;
    if (r < R) {
      w = verify_len[r];
      w = w < 0 ? 0 : (w > B ? B : w);
      L = accept_len[r];
      L = L < 0 ? 0 : (L > w ? w : L);
      if (w < B) {
        trimmed += 1;
        if (L == w) regret += 1;
      }
      sum_l += L;
      sum_w += w;
    }
    bool more = true;
    for (int c = 0; more && c < B; c += 64) {
      uint32_t aw = 0u, al = 0u;
      const int cend = B - c < 64 ? B - c : 64;
      for (int jj = 0; jj < cend; ++jj) {
        const uint64_t bw = __ballot(w > c + jj);
        if (bw == 0) { more = false; break; }  // L <= w: no accepted count either
        const uint64_t bl = __ballot(L > c + jj);
        if (l == jj) { aw = (uint32_t)__popcll(bw); al = (uint32_t)__popcll(bl); }
      }
      if (aw) atomicAdd(&cw[c + l], aw);
      if (al) atomicAdd(&cl[c + l], al);
    }
  }
  trimmed = wave_scan_dpp(trimmed);
  regret = wave_scan_dpp(regret);
  sum_l = wave_scan_dpp(sum_l);
  sum_w = wave_scan_dpp(sum_w);
  if (l == 63) { tot[wv][0] = trimmed; tot[wv][1] = regret; tot[wv][2] = sum_l; tot[wv][3] = sum_w; }
  __syncthreads();
  if (tid < 4) {
    uint32_t v = 0u;
    for (int q = 0; q < kPW; ++q) v += tot[q][tid];
    stats[1 + tid] = v;
  } else if (tid == 4) {
    stats[0] = R;
  }
  for (int j = tid; j < B; j += kPB) {
    stats[5 + j] = cw[j];
    stats[5 + B + j] = cl[j];
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
// every kEstRefit calls the refit.  One workgroup: wave w takes positions
// k = w, w + 16, ... over every request (four requests' inputs loaded per lane
// at once) and sums its lanes by DPP scans; one thread per position adds the
// sums to the stored ones, and the refit runs from LDS.  A fixed order
// throughout, so the same inputs give the same state.
__global__ __launch_bounds__(kPlanBlock) void est_observe_kernel(
    const double* feature, const int32_t* accept_len, const int32_t* verify_len, int32_t R,
    int32_t B, double* st) {
  constexpr int kU = 4;
  const EstLayout L(B);
  __shared__ double part[kEstMaxBlock][7];  // per position: h_sk, h_kk, g_k, n_k, h_ss, g_s, n_s
  __shared__ double fin[kEstMaxBlock][4];   // the statistics after this call
  __shared__ double coef[kEstMaxBlock + 1]; // slope, intercepts
  __shared__ double fin_s[4];               // h_ss, g_s, n_s, calls
  __shared__ double step_s;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  if (tid <= B) coef[tid] = st[tid];  // slope at 0, intercepts at 1..B
  __syncthreads();
  const double slope = coef[0];
  for (int k = w; k < B; k += kPW) {
    const double bk = coef[1 + k];
    double hss = 0.0, gs = 0.0, hsk = 0.0, hkk = 0.0, gk = 0.0, nk = 0.0;
    for (int r0 = 0; r0 < R; r0 += 64 * kU) {
      int wr[kU], lr[kU];
      double x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int r = r0 + 64 * u + l;
        wr[u] = r < R ? verify_len[r] : 0;
        lr[u] = r < R ? accept_len[r] : 0;
        x[u] = r < R ? feature[(size_t)r * B + k] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int wc = wr[u] < 0 ? 0 : (wr[u] > B ? B : wr[u]);
        const int lc = lr[u] < 0 ? 0 : (lr[u] > wc ? wc : lr[u]);
        const int last = lc < wc ? lc : lc - 1;  // an empty window gives -1
        if (k > last) continue;
        const double y = k < lc ? 1.0 : 0.0;
        const double p = est_sigmoid(slope * x[u] + bk);
        const double wt = p * (1.0 - p);
        hss += wt * x[u] * x[u];
        hsk += wt * x[u];
        hkk += wt;
        gs += (y - p) * x[u];
        gk += y - p;
        nk += 1.0;
      }
    }
    hsk = readlane_d(wave_scan_dpp(hsk), 63);
    hkk = readlane_d(wave_scan_dpp(hkk), 63);
    gk = readlane_d(wave_scan_dpp(gk), 63);
    nk = readlane_d(wave_scan_dpp(nk), 63);
    hss = readlane_d(wave_scan_dpp(hss), 63);
    gs = readlane_d(wave_scan_dpp(gs), 63);
    if (l == 0) {
      part[k][0] = hsk; part[k][1] = hkk; part[k][2] = gk; part[k][3] = nk;
      part[k][4] = hss; part[k][5] = gs; part[k][6] = nk;
    }
  }
  __syncthreads();
  if (tid < B) {
    const int k = tid;
    fin[k][0] = st[L.h_sk(k)] + part[k][0];
    fin[k][1] = st[L.h_kk(k)] + part[k][1];
    fin[k][2] = st[L.g_k(k)] + part[k][2];
    fin[k][3] = st[L.n_k(k)] + part[k][3];
  } else if (tid == kPB - 1) {
    double a = 0.0, b = 0.0, c = 0.0;
    for (int k = 0; k < B; ++k) { a += part[k][4]; b += part[k][5]; c += part[k][6]; }
    fin_s[0] = st[L.h_ss()] + a;
    fin_s[1] = st[L.g_s()] + b;
    fin_s[2] = st[L.n_s()] + c;
    fin_s[3] = st[L.calls()] + 1.0;
  }
  __syncthreads();
  const bool refit = fin_s[3] >= (double)kEstRefit;
  if (!refit) {  // store the statistics and the count
    if (tid < B) {
      st[L.h_sk(tid)] = fin[tid][0];
      st[L.h_kk(tid)] = fin[tid][1];
      st[L.g_k(tid)] = fin[tid][2];
      st[L.n_k(tid)] = fin[tid][3];
    } else if (tid == kPB - 1) {
      st[L.h_ss()] = fin_s[0];
      st[L.g_s()] = fin_s[1];
      st[L.n_s()] = fin_s[2];
      st[L.calls()] = fin_s[3];
    }
    return;
  }
  // refit: arrowhead Newton solve with a ridge (Schur complement on the slope)
  if (tid == 0) {
    const double ridge = 1e-3;
    double a = fin_s[0] + ridge, g = fin_s[1];
    for (int k = 0; k < B; ++k) {
      const double dk = fin[k][1] + ridge;
      a -= fin[k][0] * fin[k][0] / dk;
      g -= fin[k][0] * fin[k][2] / dk;
    }
    const double ns = fin_s[2];
    double step = (g / a) * (ns / (ns + 50.0));
    if (!isfinite(step)) step = 0.0;
    const double s0 = coef[0];
    for (int h = 0; h < 8 && s0 + step < 0.0; ++h) step *= 0.5;
    if (s0 + step < 0.0) step = 0.0;
    step_s = step;
    st[L.slope()] = s0 + step;
    st[L.h_ss()] = st[L.g_s()] = st[L.n_s()] = 0.0;
    st[L.calls()] = 0.0;
    st[L.refits()] += 1.0;
  }
  __syncthreads();
  if (tid < B) {  // intercepts: their Newton step given the slope step taken
    const int k = tid;
    const double ridge = 1e-3;
    const double dk = fin[k][1] + ridge;
    const double nk = fin[k][3];
    double sb = ((fin[k][2] - fin[k][0] * step_s) / dk) * (nk / (nk + 50.0));
    if (!isfinite(sb)) sb = 0.0;
    st[L.bias(k)] = coef[1 + k] + sb;
    st[L.h_sk(k)] = st[L.h_kk(k)] = st[L.g_k(k)] = st[L.n_k(k)] = 0.0;
  }
}

}  // namespace sv
