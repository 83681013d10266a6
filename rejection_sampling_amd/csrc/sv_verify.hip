// sv_verify.hip -- verify-step kernels for gfx950.
//
//   row_pass_kernel   one workgroup per packed row: the streaming pass over the
//                     logits, the kept set N of the row (top-k on raw logits,
//                     temperature on the kept values only, then top-p, as the
//                     build_speculative_verify_target_probs note of "Adaptive
//                     verification for DFLASH" describes), p(d) and the ratio
//                     test of the row's draft token (Leviathan et al.; greedy:
//                     argmax match, consolidation study section 2).
//   finalize_kernel   one workgroup per request: the accepted prefix (first
//                     rejected row, capped by verify_cap), then one exponential
//                     race on the single sampled row -- residual max(0, p - q)
//                     after a rejection, p after a full accept.
//   build_out_kernel  one workgroup per row: the outputs of the target-probs
//                     build (max, argmax, lse, kept ids, dense p).
#include <type_traits>

#include "sv_device.hpp"
#include "sv_rowpass.hpp"
#include "sv_kernels.h"

namespace sv {

// ------------------------------------------------------------ exact path
struct ExactOut {
  uint32_t bkey;   // order key (32-bit) of the boundary value of N
  int nb;          // ties at bkey kept
  int nkeep;
  double zk, zn;   // masses relative to exp(m/T)
  int argmax;
  int tie_d;       // ties of the draft value with a smaller id
  int ntie;        // elements of K at bkey (nb of them are kept)
};

__device__ __forceinline__ uint32_t key_of_prefix(uint32_t prefix, bool bf16) {
  if (!bf16) return prefix;
  // top 16 bits are the bf16 order key; rebuild the value, then its fp32 key
  const uint32_t k16 = prefix >> 16;
  const uint32_t u16 = (k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
  return fkey(__uint_as_float(u16 << 16));
}

// Walk 256 bins from the top: the digit d* where above + sum(d > d*) < target
// <= above + sum(d >= d*).  Wave 0 computes; results land in sh.
__device__ inline void walk_bins(const double* val, double above, double target, RowShared& sh,
                                 double* out_above) {
  if (wave_id() == 0) {
    const int l = lane_id();
    const double h0 = val[255 - 4 * l], h1 = val[254 - 4 * l];
    const double h2 = val[253 - 4 * l], h3 = val[252 - 4 * l];
    const double local = (h0 + h1) + (h2 + h3);
    const double incl = wave_inclusive_sum(local);
    const double excl = incl - local;
    const double top = __shfl(incl, 63, 64);
    bool here = above + excl < target && target <= above + incl;
    uint64_t mk = __ballot(here);
    // target beyond the total (rounding): take the last non-empty digit
    if (mk == 0) mk = __ballot(above + excl < above + top && l == 63) | 0;
    int src = mk ? __ffsll((unsigned long long)mk) - 1 : 63;
    if (l == src) {
      double c = above + excl;
      int d;
      if (c + h0 >= target || (h1 == 0 && h2 == 0 && h3 == 0)) d = 255 - 4 * l;
      else if ((c += h0) + h1 >= target || (h2 == 0 && h3 == 0)) d = 254 - 4 * l;
      else if ((c += h1) + h2 >= target || h3 == 0) d = 253 - 4 * l;
      else { c += h2; d = 252 - 4 * l; }
      sh.sel_digit = d;
      sh.zn_shared = c;
    }
  }
  __syncthreads();
  *out_above = sh.zn_shared;
}

template <int DT>
__device__ void exact_kept_set(const void* row, int V, float m, float T, int k_eff, float P,
                               int d, float xd, RowShared& sh, ExactOut& o) {
  constexpr bool kBf = DT == 1;
  const float c = kLog2e / T;
  int lg = 0;
  while ((1ll << lg) < (long long)V + 1) ++lg;
  const double scale = ldexp(1.0, 62 - lg);
  uint64_t* mass = sh.buf;             // 256 x u64
  double* vals = (double*)(sh.buf + 256);  // 256 x double
  const uint32_t keyd = d >= 0 ? fkey(xd) : 0u;
  const int top_shift = 24, low_shift = kBf ? 16 : 0;

  int amin = 0x7FFFFFFF, tied = 0;
  bool first = true;

  // one histogram pass over elements with key >= klo and (key & pmask) == prefix
  auto pass = [&](uint32_t prefix, uint32_t pmask, int shift, uint32_t klo) {
    for (int b = threadIdx.x; b < 256; b += kBlock) { sh.whist[0][b] = 0u; mass[b] = 0ull; }
    __syncthreads();
    const bool fst = first;
    for_each_element_lean<DT>(row, V, [&](float x, int i) {
      const uint32_t key = fkey(x);
      if (fst) {
        if (x == m && i < amin) amin = i;
        if (d >= 0 && i < d && key == keyd) ++tied;
      }
      if (key < klo || (key & pmask) != prefix) return;
      const uint32_t dg = (key >> shift) & 255u;
      atomicAdd(&sh.whist[0][dg], 1u);
      const float w = exp2f((x - m) * c);
      atomicAdd((unsigned long long*)&mass[dg], (unsigned long long)((double)w * scale));
    });
    first = false;
    __syncthreads();
  };

  // ---- top-k phase (count target)
  uint32_t bk = 0;          // 32-bit key of the k-th element (0: top-k off)
  int nbk = 0, cnt_bk = 0;
  double zk = 0.0;          // fixed-point units
  const bool topk_on = k_eff < V;
  if (topk_on) {
    uint32_t prefix = 0, pmask = 0;
    double cnt_above = 0.0, mass_above = 0.0;
    for (int shift = top_shift; shift >= low_shift; shift -= 8) {
      pass(prefix, pmask, shift, 0u);
      for (int b = threadIdx.x; b < 256; b += kBlock) vals[b] = (double)sh.whist[0][b];
      __syncthreads();
      double above;
      walk_bins(vals, cnt_above, (double)k_eff, sh, &above);
      const int dg = sh.sel_digit;
      // mass of the digits strictly above dg
      double mab = 0.0;
      for (int b = threadIdx.x; b < 256; b += kBlock) vals[b] = b > dg ? (double)mass[b] : 0.0;
      __syncthreads();
      mab = block_sum_d(threadIdx.x < 256 ? vals[threadIdx.x] : 0.0, sh.dscr);
      cnt_above = above;
      mass_above += mab;
      cnt_bk = (int)sh.whist[0][dg];
      prefix |= (uint32_t)dg << shift;
      pmask |= 0xFFu << shift;
      __syncthreads();
    }
    bk = key_of_prefix(prefix, kBf);
    nbk = k_eff - (int)cnt_above;
    const float wb = exp2f((key_to_float(bk) - m) * c);
    zk = mass_above + (double)nbk * (double)(unsigned long long)((double)wb * scale);
    o.bkey = bk;
    o.nb = nbk;
    o.ntie = cnt_bk;
    o.nkeep = k_eff;
  }

  // ---- top-p phase (mass target), restricted to K
  const bool topp_on = P < 1.0f;
  if (topp_on) {
    uint32_t prefix = 0, pmask = 0;
    double cnt_above = 0.0, mass_above = 0.0;
    const float wbk = topk_on ? exp2f((key_to_float(bk) - m) * c) : 0.0f;
    const double fx_bk = (double)(unsigned long long)((double)wbk * scale);
    const int excess = topk_on ? cnt_bk - nbk : 0;
    double target = -1.0;
    for (int shift = top_shift; shift >= low_shift; shift -= 8) {
      pass(prefix, pmask, shift, topk_on ? bk : 0u);
      // remove the tied entries at bk that are outside K
      const bool bk_here = topk_on && (bk & pmask) == prefix;
      const int dbk = (int)((bk >> shift) & 255u);
      for (int b = threadIdx.x; b < 256; b += kBlock) {
        double mv = (double)mass[b];
        if (bk_here && b == dbk) mv -= (double)excess * fx_bk;
        vals[b] = mv;
      }
      __syncthreads();
      if (target < 0.0) {
        if (!topk_on) zk = block_sum_d(threadIdx.x < 256 ? vals[threadIdx.x] : 0.0, sh.dscr);
        target = (double)P * zk;
      }
      double above;
      walk_bins(vals, mass_above, target, sh, &above);
      const int dg = sh.sel_digit;
      double cab = 0.0;
      {
        const int b = threadIdx.x;
        double cv = 0.0;
        if (b < 256 && b > dg) {
          cv = (double)sh.whist[0][b];
          if (bk_here && b == dbk) cv -= (double)excess;
        }
        cab = block_sum_d(cv, sh.dscr);
      }
      cnt_above += cab;
      mass_above = above;
      prefix |= (uint32_t)dg << shift;
      pmask |= 0xFFu << shift;
      __syncthreads();
    }
    const uint32_t bp = key_of_prefix(prefix, kBf);
    int avail;
    {
      // ties at bp inside K
      uint32_t hb = sh.whist[0][(bp >> low_shift) & 255u];
      avail = (int)hb;
      if (topk_on && bp == bk) avail = nbk;
    }
    const float wbp = exp2f((key_to_float(bp) - m) * c);
    const double fw = (double)(unsigned long long)((double)wbp * scale);
    double need = fw > 0.0 ? ceil((target - mass_above) / fw) : 1.0;
    int nb = need < 1.0 ? 1 : (need > (double)avail ? avail : (int)need);
    if (nb < 1) nb = 1;
    o.bkey = bp;
    o.nb = nb;
    o.ntie = avail;
    o.nkeep = (int)cnt_above + nb;
    o.zn = (mass_above + (double)nb * fw) / scale;
  } else {
    o.zn = zk / scale;
  }
  o.zk = zk / scale;

  if (first) {
    // no histogram pass ran (cannot happen: callers need top-k or top-p)
    for_each_element_lean<DT>(row, V, [&](float x, int i) {
      if (x == m && i < amin) amin = i;
      if (d >= 0 && i < d && fkey(x) == keyd) ++tied;
    });
  }
  // argmax and tie count: block reductions
  {
    const uint64_t e = ((uint64_t)(uint32_t)(0x7FFFFFFF - amin));
    const uint64_t best = block_max_u64(e, sh.uscr);
    o.argmax = 0x7FFFFFFF - (int)(uint32_t)best;
    o.tie_d = block_sum_i(tied, sh.iscr);
  }
}

// Exact top-p kept set of a bf16 row with top-k off (the same fixed-point
// masses and boundary rule as exact_kept_set), in one histogram pass: each of
// the kNbCodes bf16 values just below the maximum is its own bin (a count; the
// weight is the same for every element of a bin), and the mass of the elements
// further down is summed in registers.  A block scan over the bins from the
// top finds the boundary value; a second pass, when needed, lists the kept set
// (when it fits a list) and collects the ids of the ties at the boundary,
// ranked to give the cut when only some of them are kept.  zk_stream, when
// positive, is the row's mass Z_K (relative to exp(m/T)) that the streaming
// pass already summed: the target is then P times it and the elements below
// the binned values are not visited at all.  Returns false when the boundary
// lies below the binned values or the ties overflow their buffer (the caller
// then runs the general path).
constexpr int kNbCodes = 4 * kBlock;
constexpr int kTieBuf = kWaves * 256;

__device__ __forceinline__ float bf16_code_value(uint32_t k16) {
  const uint32_t u16 = (k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
  return __uint_as_float(u16 << 16);
}

template <int DT>
__device__ __forceinline__ bool exact_topp_codes(const void* row, int V, float m, float T, float P,
                                                 int d, float xd, double zk_stream, bool sorted,
                                                 ListEntry* L, RowShared& sh, ExactOut& o,
                                                 int& tie_cut, bool& listed) {
  static_assert(DT == 1, "bf16 rows only");
  const int tid = threadIdx.x;
  if (!(m > -INFINITY) || !(m < INFINITY)) return false;
  const float c = kLog2e / T;
  int lg = 0;
  while ((1ll << lg) < (long long)V + 1) ++lg;
  const double scale = ldexp(1.0, 62 - lg);
  auto fx = [&](float x) { return (uint64_t)((double)exp2f((x - m) * c) * scale); };
  uint32_t* cnt = (uint32_t*)sh.buf;  // [kNbCodes]
  for (int b = tid; b < kNbCodes; b += kBlock) cnt[b] = 0u;
  if (tid == 0) sh.sel_digit = -1;
  __syncthreads();
  const uint32_t mk16 = fkey(m) >> 16;
  // the lowest binned value: elements below it are summed, not binned
  const float x_lo = mk16 >= (uint32_t)(kNbCodes - 1)
                         ? bf16_code_value(mk16 - (uint32_t)(kNbCodes - 1)) : -INFINITY;
  const bool sum_below = !(zk_stream > 0.0);
  double below = 0.0;  // sum of the fp32 weights of the unbinned elements
  int amin = 0x7FFFFFFF, tied = 0;
  auto count = [&](float x, int i) {
    if (x >= x_lo) {
      atomicAdd(&cnt[mk16 - (fkey(x) >> 16)], 1u);
      if (x == m && i < amin) amin = i;
    } else if (sum_below) {
      below += (double)exp2f((x - m) * c);
    }
  };
  auto elem = [&](float x, int i) {
    count(x, i);
    if (i < d && x == xd) ++tied;
  };
  for_each_vector_deep<DT, 2>(row, V, [&](const float* x, int i0) {
    const float vmax = vec_max<8>(x);
    if (vmax < x_lo) {  // no element is binned
      if (sum_below) {
#pragma unroll
        for (int e = 0; e < 8; ++e) below += (double)exp2f((x[e] - m) * c);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // the bin from the value's bf16 bits (its order code, -0 as +0):
        // in the window iff the bin index is below kNbCodes
        uint32_t h = __float_as_uint(x[e]) >> 16;
        h = h == 0x8000u ? 0u : h;
        const uint32_t code = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
        const uint32_t bin = mk16 - code;
        if (bin < (uint32_t)kNbCodes) atomicAdd(&cnt[bin], 1u);
        else if (sum_below) below += (double)exp2f((x[e] - m) * c);
      }
      if (vmax == m) {  // the lowest id reaching the maximum
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (x[e] == m && i0 + e < amin) amin = i0 + e;
      }
    }
    if (i0 < d && vmax >= xd) {
#pragma unroll
      for (int e = 0; e < 8; ++e) tied += (i0 + e < d && x[e] == xd) ? 1 : 0;
    }
  }, elem);
  __syncthreads();
  // masses of this thread's four bins (from the top), then a block scan
  uint32_t cb[4];
  uint64_t mb[4], loc = 0;
  uint32_t lcnt = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = 4 * tid + q;
    cb[q] = cnt[b];
    mb[q] = cb[q] ? (uint64_t)cb[q] * fx(bf16_code_value(mk16 - (uint32_t)b)) : 0ull;
    loc += mb[q];
    lcnt += cb[q];
  }
  uint64_t incl = loc;
  uint32_t cincl = lcnt;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const uint64_t y = ((uint64_t)__shfl_up((uint32_t)(incl >> 32), s, 64) << 32) |
                       __shfl_up((uint32_t)incl, s, 64);
    const uint32_t yc = __shfl_up(cincl, s, 64);
    if (lane_id() >= s) {
      incl += y;
      cincl += yc;
    }
  }
  const double bsum = wave_sum_d(below);
  uint64_t* wtot = (uint64_t*)sh.mhist;  // [0..3] bin masses, [4..7] counts
  double* wbl = (double*)(sh.mhist + 8);  // [0..3] unbinned weight sums
  if (lane_id() == 63) {
    wtot[wave_id()] = incl;
    wtot[4 + wave_id()] = cincl;
    wbl[wave_id()] = bsum;
  }
  __syncthreads();
  uint64_t base = 0, tot = 0;
  uint32_t cbase = 0;
  double blw = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave_id()) {
      base += wtot[w];
      cbase += (uint32_t)wtot[4 + w];
    }
    tot += wtot[w];
    blw += wbl[w];  // fixed order: deterministic
  }
  // the unbinned elements in the same fixed-point units (their weights are
  // summed in fp64 from fp32 values: within one unit per element of the
  // per-element truncation)
  const double zk_fx = sum_below ? (double)(tot + (uint64_t)(blw * scale)) : zk_stream * scale;
  const double target = (double)P * zk_fx;
  {
    uint64_t above = base + incl - loc;
    uint32_t cab = cbase + cincl - lcnt;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if ((double)above < target && target <= (double)(above + mb[q])) {
        sh.sel_digit = 4 * tid + q;
        sh.sel_entry = above;
        sh.sel_need = (int)cab;
        sh.count = (int)cb[q];
      }
      above += mb[q];
      cab += cb[q];
    }
  }
  __syncthreads();
  const int bstar = sh.sel_digit;
  if (bstar < 0) return false;  // the boundary lies below the binned values
  const uint64_t above = sh.sel_entry;
  const int cnt_above = sh.sel_need;
  const int avail = sh.count;
  const uint32_t bp16 = mk16 - (uint32_t)bstar;
  const float xb = bf16_code_value(bp16);
  const uint64_t fw = fx(xb);
  const double need = ceil((target - (double)above) / (double)fw);
  int nb = need < 1.0 ? 1 : (need > (double)avail ? avail : (int)need);
  if (nb < 1) nb = 1;
  o.bkey = fkey(xb);
  o.nb = nb;
  o.ntie = avail;
  o.nkeep = cnt_above + nb;
  o.zk = zk_fx / scale;
  o.zn = ((double)above + (double)nb * (double)fw) / scale;
  o.argmax = 0x7FFFFFFF - (int)(uint32_t)block_max_u64((uint64_t)(uint32_t)(0x7FFFFFFF - amin),
                                                      sh.uscr);
  o.tie_d = block_sum_i(tied, sh.iscr);
  tie_cut = V;
  listed = false;
  const bool want_list = o.nkeep <= kListCap;
  const bool want_ties = nb < avail;
  if (!want_list && !want_ties) return true;
  if (want_ties && avail > kTieBuf) return false;
  // second pass: kept entries above the boundary (listed rows) and the ties
  int* tie_ids = (int*)&sh.whist[0][0];
  if (tid == 0) {
    sh.count = 0;
    sh.wcount[0] = 0;
    sh.found = V;
  }
  __syncthreads();
  auto elem2 = [&](float x, int i) {
    if (x < xb) return;
    if (x == xb && want_ties) {
      const int t = atomicAdd(&sh.wcount[0], 1);
      if (t < kTieBuf) tie_ids[t] = i;
    } else if (want_list) {
      const int slot = atomicAdd(&sh.count, 1);
      if (slot < kCap) sh.buf[slot] = make_entry(x, i);
    }
  };
  for_each_vector_deep<DT, 2>(row, V, [&](const float* x, int i0) {
    if (vec_max<8>(x) < xb) return;  // the whole vector below the boundary
#pragma unroll
    for (int e = 0; e < 8; ++e) elem2(x[e], i0 + e);
  }, elem2);
  __syncthreads();
  if (want_ties) {
    const int nt = sh.wcount[0];
    if (nt != avail) return false;
    // the nb-th smallest id among the ties: the kept ones lie below it + 1
    for (int t = tid; t < nt; t += kBlock) {
      const int id = tie_ids[t];
      int rank = 0;
      for (int u = 0; u < nt; ++u) rank += tie_ids[u] < id ? 1 : 0;
      if (rank == nb - 1) sh.found = id + 1;
    }
    __syncthreads();
    tie_cut = sh.found;
    if (want_list) {
      for (int t = tid; t < nt; t += kBlock) {
        const int id = tie_ids[t];
        if (id < tie_cut) {
          const int slot = atomicAdd(&sh.count, 1);
          if (slot < kCap) sh.buf[slot] = make_entry(xb, id);
        }
      }
      __syncthreads();
    }
  }
  if (!want_list) return true;
  const int n = sh.count;
  __syncthreads();
  if (n != o.nkeep) return true;  // not listed: the range and the tie cut describe the set
  if (sorted) sort_desc(sh, n);
  for (int t = tid; t < n; t += kBlock) {
    const uint64_t en = sh.buf[t];
    ListEntry le;
    le.idx = entry_idx(en);
    le.x = entry_val(en);
    L[t] = le;
  }
  listed = true;
  return true;
}

// -------------------------------------------------------- row pass kernel
// ----------------------------------------------------------------- races
// Exponential race: winner = argmax over weight_v / E_v, E_v = -ln U_v; ties
// go to the lower id.  Reduces (key, id) pairs across the block.
struct RaceBest {
  double key;
  int id;
};
__device__ __forceinline__ bool race_better(double k1, int i1, double k2, int i2) {
  return k1 > k2 || (k1 == k2 && i1 < i2);
}
__device__ inline RaceBest block_race_best(RaceBest b, RowShared& sh) {
#pragma unroll
  for (int dd = 32; dd >= 1; dd >>= 1) {
    const double ok = __shfl_xor(b.key, dd, 64);
    const int oi = __shfl_xor(b.id, dd, 64);
    if (race_better(ok, oi, b.key, b.id)) { b.key = ok; b.id = oi; }
  }
  __syncthreads();
  if (lane_id() == 0) {
    sh.dscr[wave_id()] = b.key;
    sh.iscr[wave_id()] = b.id;
  }
  __syncthreads();
  RaceBest r = {sh.dscr[0], sh.iscr[0]};
  for (int w = 1; w < kWaves; ++w)
    if (race_better(sh.dscr[w], sh.iscr[w], r.key, r.id)) { r.key = sh.dscr[w]; r.id = sh.iscr[w]; }
  __syncthreads();
  return r;
}

// One step of the wave arg-max below: the (key, id) of the lane CTRL reads,
// taken when better (lanes without a source read key -1).
template <int CTRL, int ROWS>
__device__ __forceinline__ void best_step_dpp(double& key, int& id) {
  const int klo = __builtin_amdgcn_update_dpp(0, __double2loint(key), CTRL, ROWS, 0xF, false);
  const int khi =
      __builtin_amdgcn_update_dpp(__double2hiint(-1.0), __double2hiint(key), CTRL, ROWS, 0xF, false);
  const int oi = __builtin_amdgcn_update_dpp(0x7FFFFFFF, id, CTRL, ROWS, 0xF, false);
  const double ok = __hiloint2double(khi, klo);
  if (race_better(ok, oi, key, id)) {
    key = ok;
    id = oi;
  }
}
// Best (key desc, id asc) over a fully active wave, returned in every lane:
// a prefix arg-max by DPP row shifts and row broadcasts, read at lane 63.
__device__ __forceinline__ RaceBest wave_best_dpp(RaceBest b) {
  best_step_dpp<0x111, 0xF>(b.key, b.id);
  best_step_dpp<0x112, 0xF>(b.key, b.id);
  best_step_dpp<0x114, 0xF>(b.key, b.id);
  best_step_dpp<0x118, 0xF>(b.key, b.id);
  best_step_dpp<0x142, 0xA>(b.key, b.id);
  best_step_dpp<0x143, 0xC>(b.key, b.id);
  RaceBest r;
  r.key = readlane_d(b.key, 63);
  r.id = __builtin_amdgcn_readlane(b.id, 63);
  return r;
}

__device__ __forceinline__ double race_e(uint64_t seed, uint32_t rid, uint32_t pos, uint32_t v) {
  return -log(race_uniform(seed, rid, pos, 1u, v));
}

// LDS areas of the vector-candidate finish, past the wave regions (entries of
// 8 bytes; each wave holds at most kThreshVec candidates when streaming ends
// without overflow).
constexpr int kVecGatherOff = kWaves * kVecStride;         // gathered candidates
constexpr int kVecGatherCap = kWaves * kThreshVec;
constexpr int kVecGIdxOff = kVecGatherOff + kVecGatherCap;  // their data slots (int)
constexpr int kVecSortOff = kVecGIdxOff + kVecGatherCap / 2;
constexpr int kVecSIdxOff = kVecSortOff + 64;               // 64 ints
constexpr int kVecElemOff = kVecGatherOff;                  // reuses the gather area
constexpr int kVecElemCap = kVecSortOff - kVecElemOff;
static_assert(kVecSIdxOff + 32 <= kCap, "LDS layout");
static_assert(kVecElemCap >= 64 * 8 + 16, "room for k vectors and the scalar ends");
static_assert(kVecElemOff + kVecElemCap <= kVecSortOff, "elements stay clear of the sorted area");

// The best min(n, k) of src[0, n) (distinct entries), by rank counting, to
// dst[rank] (with their companions); wave-local.  Returns min(n, k).
__device__ __forceinline__ int wave_rank_top(const uint64_t* src, const int* srci, int n, int k,
                                             uint64_t* dst, int* dsti) {
  const int l = lane_id();
  if (n <= 64) {  // one entry per lane, the others read by lane broadcast
    const uint64_t mine = l < n ? src[l] : 0ull;
    const int comp = (srci && l < n) ? srci[l] : 0;
    const uint32_t mlo = (uint32_t)mine, mhi = (uint32_t)(mine >> 32);
    int rank = 0;
    for (int u = 0; u < n; ++u) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)mlo, u);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)mhi, u);
      rank += (((uint64_t)hi << 32) | (uint64_t)lo) > mine ? 1 : 0;
    }
    wave_lds_sync();
    if (l < n && rank < k) {
      dst[rank] = mine;
      if (srci) dsti[rank] = comp;
    }
    wave_lds_sync();
    return n < k ? n : k;
  }
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int f = j0 + l;
    const uint64_t mine = f < n ? src[f] : 0ull;
    int rank = 0;
    for (int u = 0; u < n; ++u) rank += src[u] > mine ? 1 : 0;
    if (f < n && rank < k) {
      dst[rank] = mine;
      if (srci) dsti[rank] = srci[f];
    }
  }
  wave_lds_sync();
  return n < k ? n : k;
}

// Shrink src[0, n) (n > 64) toward `k` <= 64 entries by the lane-threshold
// rule, then exactly to k by radix select if still above 64.
__device__ __forceinline__ int wave_shrink(uint64_t* src, int* srci, int n, int k, uint32_t* hist) {
  uint32_t b1 = 0u, b2 = 0u;
  for (int e = lane_id(); e < n; e += 64) {
    const uint32_t key = (uint32_t)(src[e] >> 32);
    if (key > b1) { b2 = b1; b1 = key; } else if (key > b2) { b2 = key; }
  }
  const uint32_t tk = wave_threshold_key(b1, b2, k);
  if (tk != 0u) n = wave_keep_ge(src, n, tk, srci);
  return n;
}

// Top-k rows with k <= 64 are finished by wave 0 once the block's streaming
// is done: the best k vectors among the wave candidates, their elements (and
// the unvectorised head and tail) at or above the k-th vector max, the best k
// of those in order (vec_topk_select), then the kept set (vec_kept).

// One kept entry per lane of wave 0 after the vector-candidate finish.
struct VecKept {
  float x;    // logit
  int id;     // token
  double w;   // exp((x - m) / T); 0 past nkeep
  double q;   // q(id), gathered when the row is tested
  int nkeep;
  double zn;
};

// The best min(k, #finite) elements of the vector candidates (wave 0), sorted
// by (value desc, id asc) into sh.buf[kVecSortOff, +n).  Returns n, or -1 when
// the candidates cannot certify them (a pile of ties beyond the element area)
// or, with need_k, when fewer than k elements are finite.
template <int DT>
__device__ __forceinline__ int vec_topk_select(int V, int k, bool need_k, const RowSplit<DT>& sp,
                                               RowShared& sh) {
  constexpr int PE = Vec<DT>::kEpv;
  constexpr float kNegInf = -__builtin_huge_valf();
  const int l = lane_id();
  uint64_t* C = sh.buf + kVecGatherOff;
  int* CI = (int*)(sh.buf + kVecGIdxOff);
  uint64_t* S = sh.buf + kVecSortOff;
  int* SI = (int*)(sh.buf + kVecSIdxOff);
  uint64_t* E = sh.buf + kVecElemOff;
  uint32_t* hist = sh.whist[0];

  // vectors below the best wave threshold have k better vectors in that wave
  float tb = sh.wtau[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) tb = fmaxf(tb, sh.wtau[w]);
  const uint32_t tkey = fkey(tb);
  static_assert(kThreshVec <= 128, "two gather rounds per wave segment");
  uint64_t cv[kWaves][2];  // every read issued before the first use
  int cnt[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    cnt[w] = sh.wcount[w];
    if (cnt[w] > 128) return -1;  // not reached: segments end at or below kThreshVec
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int e = r * 64 + l;
      cv[w][r] = e < cnt[w] ? sh.buf[w * kVecStride + e] : 0ull;
    }
  }
  int nc = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const bool kp = r * 64 + l < cnt[w] && (uint32_t)(cv[w][r] >> 32) >= tkey;
      const uint64_t mk = __ballot(kp);
      if (kp) {
        const int slot = nc + lanes_below(mk);
        C[slot] = cv[w][r];
        CI[slot] = w * kVecCap + r * 64 + l;
      }
      nc += __popcll(mk);
    }
  wave_lds_sync();
  if (nc > 128) {  // many ties: shrink toward k first
    nc = wave_shrink(C, CI, nc, k, hist);
    if (nc > 128) {
      nc = wave_rank_top(C, CI, nc, k, S, SI);
      for (int t = l; t < nc; t += 64) {
        C[t] = S[t];
        CI[t] = SI[t];
      }
      wave_lds_sync();
    }
  }
  // up to two candidates per lane; the k-th largest key by a ballot radix
  // select (fewer than k candidates: no wave ever dropped a finite vector)
  bool has[2];
  uint64_t vent[2];
  int di[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    has[r] = r * 64 + l < nc;
    vent[r] = has[r] ? C[r * 64 + l] : 0ull;
    di[r] = has[r] ? CI[r * 64 + l] : 0;
  }
  const uint32_t tk =
      nc >= k ? wave_kth_key(has[0] ? (uint32_t)(vent[0] >> 32) : 0u,
                             has[1] ? (uint32_t)(vent[1] >> 32) : 0u, k, DT == 1 ? 16 : 0)
              : 0u;
  // every vector at or above the k-th key (ties included) holds the top-k;
  // at least k elements reach its value
  const float tv = tk != 0u ? key_to_float(tk) : kNegInf;
  float x[2][PE];
  int id0[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    has[r] = has[r] && (uint32_t)(vent[r] >> 32) >= tk;
    const uint4* dat = (const uint4*)(sh.buf + (di[r] / kVecCap) * kVecStride + kVecDatOff);
    Vec<DT>::unpack(has[r] ? dat[di[r] % kVecCap] : make_uint4(0u, 0u, 0u, 0u), x[r]);
    id0[r] = sp.head + entry_idx(vent[r]) * PE;
  }
  const int ntail = V - sp.tail0;
  const bool hs = l < sp.head;
  const bool ts = l >= 32 && l - 32 < ntail;
  const float xs = hs ? sh.endx[l] : (ts ? sh.endx[8 + l - 32] : kNegInf);
  const int is = hs ? l : sp.tail0 + l - 32;
  wave_lds_sync();  // gather area read: E may overwrite it

  // each lane counts its passing elements; one wave scan gives its slots
  int ecnt = 0;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int e = 0; e < PE; ++e) ecnt += (has[r] && x[r][e] >= tv) ? 1 : 0;
  const bool sp_in = (hs || ts) && xs >= tv;
  ecnt += sp_in ? 1 : 0;
  const int eincl = wave_scan_dpp(ecnt);
  const int ne = __builtin_amdgcn_readlane(eincl, 63);
  if ((need_k && ne < k) || ne > kVecElemCap) return -1;  // too few finite, or a pile of ties
  {
    int slot = eincl - ecnt;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < PE; ++e)
        if (has[r] && x[r][e] >= tv) E[slot++] = make_entry(x[r][e], id0[r] + e);
    if (sp_in) E[slot] = make_entry(xs, is);
  }
  wave_lds_sync();
  int nel = ne;
  if (nel > 64) nel = wave_shrink(E, nullptr, nel, k, hist);
  if (nel > 64) {
    wave_compact(E, hist, nel, k);
    nel = k;
  }
  const int nt = wave_rank_top(E, nullptr, nel, k, S, nullptr);
  const uint64_t fin = __ballot(l < nt && entry_val(S[l < nt ? l : 0]) > kNegInf);
  const int nf = __popcll(fin);  // sorted: the finite ones come first
  if (need_k && nf < k) return -1;  // fewer than k finite elements
  return nf;
}

// Kept set of a top-k row from its k best elements (lane l < k holds the
// l-th, `el`): fp64 weights relative to the row max m, the top-p walk over the
// k-set (top-k sampling, then nucleus sampling on the truncated
// distribution), p(d), the kept list and the per-lane kept entries.
__device__ __forceinline__ void vec_kept(uint64_t el, int k, float m, float T, bool topp_on,
                                         float P, int d, const float* qrow, RowRec& out,
                                         double& pd, ListEntry* L, VecKept& kk) {
  const int l = lane_id();
  const bool valid = l < k;
  const float xv = entry_val(el);
  const int idv = entry_idx(el);
  // q on the kept candidates, issued early: a rejected row races over p - q
  const double qv = (qrow && valid) ? (double)qrow[idv] : 0.0;
  const double wgt = valid ? exp(((double)xv - (double)m) / (double)T) : 0.0;
  const double incl = wave_scan_dpp(wgt);
  const double excl = wave_prev_d(incl);
  const double zk = readlane_d(incl, k - 1);
  const double target = topp_on ? (double)P * zk : 2.0 * zk + 1.0;
  const uint64_t stop = __ballot(valid && !(excl < target));
  int nkeep = stop ? __ffsll((unsigned long long)stop) - 1 : k;
  if (nkeep < 1) nkeep = 1;
  const double zn = readlane_d(incl, nkeep - 1);
  const uint64_t fm = __ballot(l < nkeep && idv == d);
  pd = fm ? readlane_d(wgt, __ffsll((unsigned long long)fm) - 1) / zn : 0.0;
  out.a = __builtin_amdgcn_readlane(idv, 0);
  out.zk = zk;
  out.zn = zn;
  out.nkeep = nkeep;
  out.mode = kModeList;
  if (l < nkeep) {
    ListEntry le;
    le.idx = idv;
    le.x = xv;
    L[l] = le;
  }
  kk.x = xv;
  kk.id = idv;
  kk.w = l < nkeep ? wgt : 0.0;
  kk.q = qv;
  kk.nkeep = nkeep;
  kk.zn = zn;
}

// Both steps on one row; false when the row needs the exact path (fewer than
// k finite elements, or ties the candidates cannot certify).
template <int DT>
__device__ __forceinline__ bool topk_vec_finish(int V, int k, float m, float T, bool topp_on,
                                                float P, int d, const RowSplit<DT>& sp,
                                                const float* qrow, RowShared& sh, RowRec& out,
                                                double& pd, ListEntry* L, VecKept& kk) {
  if (vec_topk_select<DT>(V, k, true, sp, sh) < 0) return false;
  const uint64_t el = lane_id() < k ? sh.buf[kVecSortOff + lane_id()] : 0ull;
  vec_kept(el, k, m, T, topp_on, P, d, qrow, out, pd, L, kk);
  return true;
}

// The race of list_race over the kept set held one entry per lane (wave 0):
// weights p (residual = false) or max(0, p - q); an empty residual falls
// back to p and sets `empty`.  Returns the token (-1 when every weight is 0).
__device__ __forceinline__ int wave_kept_race(const VecKept& kk, bool residual, uint64_t seed,
                                              uint32_t rid, uint32_t pos, bool& empty) {
  const bool valid = lane_id() < kk.nkeep;
  const double p = valid ? kk.w / kk.zn : 0.0;
  const double e = valid ? race_e(seed, rid, pos, (uint32_t)kk.id) : 1.0;
  auto best = [&](double wgt) {
    RaceBest b = {-1.0, 0x7FFFFFFF};
    if (valid && wgt > 0.0) { b.key = wgt / e; b.id = kk.id; }
    return wave_best_dpp(b);
  };
  empty = false;
  RaceBest b = best(residual ? p - kk.q : p);
  if (residual && !(b.key > 0.0)) {
    empty = true;
    b = best(p);
  }
  return b.key > 0.0 ? b.id : -1;
}

template <int DT>
__device__ __forceinline__ void resolve_pending(const VerifyArgs& A, int i, int r, int j,
                                                bool tested, bool bonus, RowShared& sh);

// Top-p rows (top-k off): every element above the largest wave threshold T*
// lies in a candidate vector whose max is above T* (each wave dropped only
// vectors at or below its own threshold).  Those vectors are re-read and their
// elements above T* written to sh.buf[0, n) as entries; returns n, or -1 when
// they do not fit (the row then takes the exact path).  Block level.
constexpr int kMatVecPerThread = 8;

// Fixed-point mass walk over bf16 values by their 16-bit order codes: counts
// per code in the window [code0, code0 + kCodeBins) (one 32-bit LDS atomic per
// item, spread over the codes), the mass of a code being its count times the
// fixed-point weight of its value (as an item-by-item sum would give).  Wave 0
// walks the bins from the top to the first code where the running mass
// reaches target.  Block level; the counts live in sh.mhist.  Returns false
// when an item falls outside the window or the items stay below target;
// otherwise sets code, the mass and item count above it, and its count.
constexpr int kCodeBins = 512;
struct CodeWalk {
  uint32_t code;
  double above;
  int cnt_above, count;
  double total;  // the mass of every counted item (-1 when an item left the window)
};
// The walk over counts already in sh.mhist (block level).
__device__ __forceinline__ bool code_walk_bins(RowShared& sh, uint32_t code0, float m, float c,
                                               double scale, double target, CodeWalk& o) {
  const uint32_t* cnt = (const uint32_t*)sh.mhist;
  if (wave_id() == 0) {
    const int l = lane_id();
    constexpr int kPer = kCodeBins / 64;
    double h[kPer];
    int cc[kPer];
    double loc = 0.0;
    int cloc = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int b = kCodeBins - 1 - kPer * l - q;  // lane 0 holds the top codes
      cc[q] = (int)cnt[b];
      h[q] = 0.0;
      if (cc[q] > 0) {
        const float v = bf16_code_value(code0 + (uint32_t)b);
        const unsigned long long wf = (unsigned long long)((double)exp2f((v - m) * c) * scale);
        h[q] = (double)((unsigned long long)cc[q] * wf);
      }
      loc += h[q];
      cloc += cc[q];
    }
    const double incl = wave_inclusive_sum(loc);
    const int cincl = wave_inclusive_sum(cloc);
    const double excl = incl - loc;
    const uint64_t mk = __ballot(excl < target && target <= incl);
    if (l == 0) sh.sel_exact = mk ? 1 : 0;
    if (l == 63) sh.dscr[0] = incl;
    if (mk) {
      const int src = __ffsll((unsigned long long)mk) - 1;
      if (l == src) {
        double acc = excl;
        int cacc = cincl - cloc, q = 0;
        while (q < kPer - 1 && !(acc + h[q] >= target)) {
          acc += h[q];
          cacc += cc[q];
          ++q;
        }
        sh.sel_digit = kCodeBins - 1 - kPer * l - q;
        sh.zn_shared = acc;
        sh.sel_need = cacc;
        sh.count = cc[q];
      }
    }
  }
  __syncthreads();
  const bool ok = sh.sel_exact != 0;
  o.total = sh.dscr[0];
  if (ok) {
    o.code = code0 + (uint32_t)sh.sel_digit;
    o.above = sh.zn_shared;
    o.cnt_above = sh.sel_need;
    o.count = sh.count;
  }
  __syncthreads();
  return ok;
}

// Counts of the items' codes (key16_at(t) for t < nitems; 0xFFFFFFFF skips an
// item), then the walk.
template <class KeyAt>
__device__ __forceinline__ bool code_walk(RowShared& sh, KeyAt&& key16_at, int nitems,
                                          uint32_t code0, float m, float c, double scale,
                                          double target, CodeWalk& o) {
  uint32_t* cnt = (uint32_t*)sh.mhist;
  for (int b = threadIdx.x; b < kCodeBins; b += kBlock) cnt[b] = 0u;
  if (threadIdx.x == 0) sh.found = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < nitems; t += kBlock) {
    const uint32_t k = key16_at(t);
    if (k == 0xFFFFFFFFu) continue;
    const uint32_t b = k - code0;
    if (b < (uint32_t)kCodeBins) atomicAdd(&cnt[b], 1u);
    else sh.found = 1;  // outside the window
  }
  __syncthreads();
  if (sh.found) {
    o.total = -1.0;
    return false;
  }
  return code_walk_bins(sh, code0, m, c, scale, target, o);
}

// Lower bound on the top-p boundary from the candidate vectors' maxima (bf16
// rows): the vectors whose maximum is at least v hold, in their maxima alone,
// a mass M(v) that is at most the mass of all elements at least v, so when
// M(v) reaches the target the boundary value is at least v.  The code walk
// over the maxima of the entries above T* gives the largest such v.  Every
// element the selection needs is then in a vector whose maximum reaches v.
template <int DT>
__device__ __forceinline__ int topp_certified(const void* row, int V, float m, float T, float P,
                                              double Z, RowShared& sh, uint32_t& code_lo) {
  constexpr int PE = Vec<DT>::kEpv;
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  float tstar = sh.wtau[0];
  bool fits = sh.wcount[0] <= kTopPEnd;
#pragma unroll
  for (int q = 1; q < kWaves; ++q) {
    tstar = fmaxf(tstar, sh.wtau[q]);
    fits = fits && sh.wcount[q] <= kTopPEnd;
  }
  if (!fits) return -1;  // (segments end the stream with at most kTopPEnd entries)
  const uint32_t tkey = fkey(tstar);
  // elements at or above klo go to the selection: those above T*, or (bf16)
  // those at or above the vector-maximum mass bound
  uint32_t klo = tkey == 0xFFFFFFFFu ? 0xFFFFFFFFu : tkey + 1u;
  code_lo = 0xFFFFFFFFu;
  if (DT == 1 && tkey != 0xFFFFFFFFu) {
    const uint32_t code0 = tkey >> 16;
    const uint32_t cmax = fkey(m) >> 16;
    if (cmax >= code0 && cmax - code0 < (uint32_t)kCodeBins) {
      int lg = 0;
      while ((1ll << lg) < (long long)V + 1) ++lg;
      const double scale = ldexp(1.0, 62 - lg);
      auto vkey16 = [&](int g) -> uint32_t {
        const int q = g / kTopPEnd, j = g - q * kTopPEnd;
        if (j >= sh.wcount[q]) return 0xFFFFFFFFu;
        const uint32_t key = (uint32_t)(sh.buf[q * kWaveCap + j] >> 32);
        return key > tkey ? (key >> 16) : 0xFFFFFFFFu;
      };
      CodeWalk cw;
      const double target = (double)P * Z * scale;
      if (code_walk(sh, vkey16, kWaves * kTopPEnd, code0, m, kLog2e / T, scale, target, cw)) {
        klo = key_of_prefix(cw.code << 16, true);
        code_lo = cw.code;
      } else {
        // every element above T* lies in one of these vectors (or is one of
        // the at most 16 head and tail elements) and weighs at most its
        // vector's maximum: when eight times the maxima's mass, the head and
        // tail at full weight and a unit per truncated weight stay below the
        // target, the certified elements cannot reach it
        if (cw.total >= 0.0 && 8.0 * cw.total + 16.0 * scale + 8.0 * kWaves * kTopPEnd < target)
          return -1;
        code_lo = code0;  // every element above T* has a code at least this
      }
    }
  }
  // fkey(x) >= klo, as a float compare (the next float above T* when no bound)
  const float vlo = key_to_float(klo);
  static_assert(kWaves * kTopPEnd == kBlock * kMatVecPerThread, "one re-read slot per entry");
  uint4 raw[kMatVecPerThread];
  int vid[kMatVecPerThread];
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < kMatVecPerThread; ++r) {
    const int g = r * kBlock + tid;
    const int q = g / kTopPEnd, j = g - q * kTopPEnd;
    vid[r] = -1;
    raw[r] = make_uint4(0u, 0u, 0u, 0u);
    if (j < sh.wcount[q]) {
      const uint64_t e = sh.buf[q * kWaveCap + j];
      if ((uint32_t)(e >> 32) >= klo) {
        vid[r] = entry_idx(e);
        raw[r] = __ldg(sp.vbase + vid[r]);
      }
    }
  }
  // the unvectorised head and tail elements are candidates too
  const int ntail = V - sp.tail0;
  const bool hs = tid < sp.head;
  const bool ts = tid >= 8 && tid - 8 < ntail;
  const int is = hs ? tid : sp.tail0 + tid - 8;
  const float xs = (hs || ts) ? Vec<DT>::load1(row, is) : 0.0f;
  const bool sp_in = (hs || ts) && xs >= vlo;
#pragma unroll
  for (int r = 0; r < kMatVecPerThread; ++r) {
    float x[PE];
    Vec<DT>::unpack(raw[r], x);
#pragma unroll
    for (int e = 0; e < PE; ++e) cnt += (vid[r] >= 0 && x[e] >= vlo) ? 1 : 0;
  }
  cnt += sp_in ? 1 : 0;
  int total;
  int pos = block_exclusive_sum(cnt, sh.iscr, &total);  // every candidate entry read
  if (total > kCap) return -1;
#pragma unroll
  for (int r = 0; r < kMatVecPerThread; ++r) {
    float x[PE];
    Vec<DT>::unpack(raw[r], x);
    const int id0 = sp.head + vid[r] * PE;
#pragma unroll
    for (int e = 0; e < PE; ++e)
      if (vid[r] >= 0 && x[e] >= vlo) sh.buf[pos++] = make_entry(x[e], id0 + e);
  }
  if (sp_in) sh.buf[pos++] = make_entry(xs, is);
  __syncthreads();
  return total;
}

// Top-p kept set among the n certified elements in sh.buf (block level):
// the boundary value by a fixed-point mass walk over 8-bit digits of the order
// key (exact integer sums, no sort), ties at the boundary by id, then the kept
// entries compacted to sh.buf[0, nkeep) (sorted only when `sorted`).  Returns
// false when the certified mass does not reach P * Z.  code_lo, when not
// 0xFFFFFFFF, is a bf16 code at or below every entry's code.
struct TopPOut {
  int nkeep, a;
  double zn, pd;
};
template <int DT>
__device__ __forceinline__ bool topp_select(RowShared& sh, int n, float m, float T, float P,
                                            double Z, int d, bool sorted, uint32_t code_lo,
                                            TopPOut& o) {
  constexpr bool kBf = DT == 1;
  const int tid = threadIdx.x;
  const float c = kLog2e / T;
  int lg = 0;
  while ((1 << lg) < n + 1) ++lg;
  const double scale = ldexp(1.0, 62 - lg);
  // fixed-point weight of an entry (fp32 exp2, as the exact path)
  auto wfx = [&](uint64_t e) {
    return (unsigned long long)((double)exp2f((entry_val(e) - m) * c) * scale);
  };
  const double target = (double)P * Z * scale;
  unsigned long long* mh = (unsigned long long*)sh.mhist;
  uint32_t* ch = sh.whist[0];
  uint32_t prefix = 0, pmask = 0;
  double above = 0.0;
  int above_cnt = 0, avail = 0;
  int nlev = kBf ? 2 : 4;
  bool walked = false;
  if (kBf && n > 0) {
    // one walk over the values' codes, in a window from the smallest code
    uint32_t code0 = code_lo;
    if (code0 == 0xFFFFFFFFu) {
      uint32_t cmin = 0xFFFFu;
      for (int t = tid; t < n; t += kBlock) {
        const uint32_t k16 = (uint32_t)(sh.buf[t] >> 48);
        cmin = k16 < cmin ? k16 : cmin;
      }
      code0 = (uint32_t)block_min_u64(cmin, sh.uscr);
    }
    CodeWalk cw;
    if (code_walk(sh, [&](int t) { return (uint32_t)(sh.buf[t] >> 48); }, n, code0, m, c, scale,
                  target, cw)) {
      above = cw.above;
      above_cnt = cw.cnt_above;
      avail = cw.count;
      prefix = cw.code << 16;
      nlev = 0;
      walked = true;
    }
  }
  if (!walked) {
    double wsum = 0.0;
    for (int t = tid; t < n; t += kBlock) wsum += (double)wfx(sh.buf[t]);
    if (block_sum_d(wsum, sh.dscr) < target) return false;
  }
  for (int lev = 0; lev < nlev; ++lev) {
    const int shift = 24 - 8 * lev;
    for (int b = tid; b < 256; b += kBlock) { ch[b] = 0u; mh[b] = 0ull; }
    __syncthreads();
    for (int t = tid; t < n; t += kBlock) {
      const uint64_t e = sh.buf[t];
      const uint32_t key = (uint32_t)(e >> 32);
      if ((key & pmask) == prefix) {
        const uint32_t dg = (key >> shift) & 255u;
        atomicAdd(&ch[dg], 1u);
        atomicAdd(&mh[dg], wfx(e));
      }
    }
    __syncthreads();
    if (wave_id() == 0) {
      // digit (from the top) where the running mass first reaches the target
      const int l = lane_id();
      double h[4];
      int cc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = (double)mh[255 - 4 * l - q];
        cc[q] = (int)ch[255 - 4 * l - q];
      }
      const double loc = (h[0] + h[1]) + (h[2] + h[3]);
      const int cloc = (cc[0] + cc[1]) + (cc[2] + cc[3]);
      const double incl = wave_inclusive_sum(loc);
      const int cincl = wave_inclusive_sum(cloc);
      const double excl = incl - loc;
      const int cexcl = cincl - cloc;
      uint64_t mk = __ballot(above + excl < target && target <= above + incl);
      if (mk == 0) mk = __ballot(l == 63);  // rounding past the total: the lowest digit
      const int src = __ffsll((unsigned long long)mk) - 1;
      if (l == src) {
        double acc = above + excl;
        int cacc = cexcl, q = 0;
        while (q < 3 && !(acc + h[q] >= target)) { acc += h[q]; cacc += cc[q]; ++q; }
        sh.sel_digit = 255 - 4 * l - q;
        sh.zn_shared = acc;
        sh.sel_need = above_cnt + cacc;
        sh.sel_exact = cc[q];
      }
    }
    __syncthreads();
    above = sh.zn_shared;
    above_cnt = sh.sel_need;
    avail = sh.sel_exact;
    prefix |= (uint32_t)sh.sel_digit << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  // the final bin holds one value; its elements keep in id order while the
  // mass before them is below the target
  uint32_t bkey = prefix;
  if (kBf) {
    const uint32_t k16 = prefix >> 16;
    const uint32_t u16 = (k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
    bkey = fkey(__uint_as_float(u16 << 16));
  }
  const double wb = (double)(unsigned long long)((double)exp2f((key_to_float(bkey) - m) * c) * scale);
  const double need = wb > 0.0 ? ceil((target - above) / wb) : 1.0;
  int nb = need < 1.0 ? 1 : (need > (double)avail ? avail : (int)need);
  if (nb < 1) nb = 1;
  // id just past the nb-th tie (all ties when none drops): the tie ids are
  // gathered (spare histogram space) and ranked among themselves
  if (tid == 0) sh.found = 0x7FFFFFFF;
  __syncthreads();
  constexpr int kTieCap = (kWaves - 1) * 256;
  if (nb < avail && avail <= kTieCap) {
    // the tie ids in any order (they are ranked among themselves next)
    int* tie_id = (int*)sh.whist[1];
    if (tid == 0) sh.count = 0;
    __syncthreads();
    for (int t = tid; t < n; t += kBlock) {
      const uint64_t e = sh.buf[t];
      if ((uint32_t)(e >> 32) == bkey) tie_id[atomicAdd(&sh.count, 1)] = entry_idx(e);
    }
    __syncthreads();
    for (int t = tid; t < avail; t += kBlock) {
      const int id = tie_id[t];
      int rank = 0;
      for (int u = 0; u < avail; ++u) rank += tie_id[u] < id ? 1 : 0;
      if (rank == nb - 1) sh.found = id + 1;
    }
  } else if (nb < avail) {
    for (int t = tid; t < n; t += kBlock) {
      const uint64_t e = sh.buf[t];
      if ((uint32_t)(e >> 32) != bkey) continue;
      const int id = entry_idx(e);
      int rank = 0;
      for (int u = 0; u < n; ++u) {
        const uint64_t o2 = sh.buf[u];
        rank += ((uint32_t)(o2 >> 32) == bkey && entry_idx(o2) < id) ? 1 : 0;
      }
      if (rank == nb - 1) sh.found = id + 1;
    }
  }
  __syncthreads();
  const int cut = sh.found;
  // compact the kept entries to the front: every entry is read first (at most
  // kCap / kBlock per thread), then the kept ones are appended.  Their order
  // in the buffer is not used (sorted below when asked; the race over them
  // reduces by key and id), while the weight sums keep each thread's fixed
  // order of entries.
  constexpr int kPer = kCap / kBlock;
  uint64_t ev[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int t = q * kBlock + tid;
    ev[q] = t < n ? sh.buf[t] : 0ull;
  }
  if (tid == 0) sh.count = 0;
  __syncthreads();  // every entry read
  double zloc = 0.0, pdl = 0.0;
  uint64_t best = 0ull;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int t = q * kBlock + tid;
    const uint64_t e = ev[q];
    const uint32_t key = (uint32_t)(e >> 32);
    if (t < n && (key > bkey || (key == bkey && entry_idx(e) < cut))) {
      sh.buf[atomicAdd(&sh.count, 1)] = e;
      const double w = exp(((double)entry_val(e) - (double)m) / (double)T);
      zloc += w;
      if (entry_idx(e) == d) pdl = w;
      best = e > best ? e : best;
    }
  }
  __syncthreads();
  const int pos0 = sh.count;
  const double zn = block_sum_d(zloc, sh.dscr);
  const double pdw = block_sum_d(pdl, sh.dscr);
  o.a = entry_idx(block_max_u64(best, sh.uscr));
  o.nkeep = pos0;
  o.zn = zn;
  o.pd = pdw / zn;
  if (sorted) sort_desc(sh, pos0);
  __syncthreads();
  return true;
}

// Race of list_race over the sorted kept entries sh.buf[0, nkeep) (block
// level); an all-zero residual falls back to p and sets `empty`.
__device__ __forceinline__ int block_kept_race(int nkeep, float m, double zn, float T,
                                               const float* qrow, bool residual, uint64_t seed,
                                               uint32_t rid, uint32_t pos, RowShared& sh,
                                               bool& empty) {
  const double Td = T;
  auto run = [&](bool resid) {
    RaceBest b = {-1.0, 0x7FFFFFFF};
    // four entries per thread at a time, their draft probabilities loaded first
    for (int t0 = threadIdx.x; t0 < nkeep; t0 += 4 * kBlock) {
      uint64_t en[4];
      float qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u * kBlock;
        en[u] = t < nkeep ? sh.buf[t] : 0ull;
        qv[u] = (resid && t < nkeep) ? qrow[entry_idx(en[u])] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t0 + u * kBlock >= nkeep) break;
        const int id = entry_idx(en[u]);
        double wgt = exp(((double)entry_val(en[u]) - (double)m) / Td) / zn;
        if (resid) wgt = wgt - (double)qv[u];
        if (!(wgt > 0.0)) continue;
        const double key = wgt / race_e(seed, rid, pos, (uint32_t)id);
        if (race_better(key, id, b.key, b.id)) { b.key = key; b.id = id; }
      }
    }
    return block_race_best(b, sh);
  };
  empty = false;
  RaceBest b = run(residual);
  if (residual && !(b.key > 0.0)) {
    empty = true;
    b = run(false);
  }
  return b.key > 0.0 ? b.id : -1;
}

// Per-request sampling parameters after the device-side clamps: T <= 0 or
// NaN is greedy, k <= 0 or >= V is off, P >= 1 is off, P <= 0 keeps the top
// token only.
struct RowParams {
  float T, P;
  int k_eff;
  bool greedy, topp_on;
};
__device__ __forceinline__ RowParams row_params(const VerifyArgs& A, int r) {
  RowParams p;
  const int V = A.vocab;
  p.T = A.temperature ? A.temperature[r] : 0.0f;
  p.greedy = !(p.T > 0.0f);
  const int k = A.top_k ? A.top_k[r] : 0;
  p.P = A.top_p ? A.top_p[r] : 1.0f;
  p.k_eff = (k > 0 && k < V) ? k : V;
  p.topp_on = p.P < 1.0f;
  if (!(p.P > 0.0f) && !(p.P != p.P)) {  // P <= 0: keep only the top token
    p.k_eff = 1;
    p.topp_on = false;
  }
  return p;
}
// What the exact path of a row needs to know up front: the row max and the
// streamed Z_K (0 when none), its request's sampling values, its draft token
// with that token's logit and draft probability, and the uniform's key.  The
// rest of the row's record is read from the workspace at the end.
struct PendingIn {
  float m;
  double zk;
  RowParams rp;
  int d;
  float xd, qd;
  uint32_t rid, pos0;
};

template <int DT>
__device__ __forceinline__ void resolve_pending_in(const VerifyArgs& A, int i, int j, bool tested,
                                                   bool bonus, const PendingIn& in, RowShared& sh);

// Greedy verify with every tested draft: accept iff it equals the argmax.
__device__ __forceinline__ void greedy_record(RowRec& out, float m, int a, bool tested, int d,
                                              bool d_ok) {
  out.m = m;
  out.a = a;
  out.mode = kModeGreedy;
  out.nkeep = 1;
  out.zn = out.zk = 1.0;
  if (tested) {
    out.flags |= kRecTested;
    if (!d_ok) out.flags |= kRecBadDraft;
    if (d == a) out.flags |= kRecAccept;
    out.pd = d == a ? 1.0 : 0.0;
  }
}

template <int DT>
__device__ __forceinline__ void row_pass(const VerifyArgs& A, RowShared& sh) {
  if (A.check && *A.check != 0) return;  // refused: qo_indptr failed the layout check
  const int i = A.row_order ? A.row_order[blockIdx.x] : (int)blockIdx.x;
  if (i < 0 || i >= A.num_rows) return;
  const int tid = threadIdx.x;
  const int V = A.vocab;
  const void* row = (const char*)A.logits + (size_t)i * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
  const int r = row_to_request(A.qo, A.num_requests, A.num_rows, i);
  const int s = A.qo[r], e = A.qo[r + 1];
  const int j = i - s;
  const int gamma = e - s - 1;
  int cap_eff = gamma;
  if (A.verify_cap) {
    int cv = A.verify_cap[r];
    cap_eff = cv < 0 ? 0 : (cv > gamma ? gamma : cv);
  }
  RowRec* rec = A.rec + i;
  const bool tested = !A.build && j < cap_eff;
  const bool used = A.build || j <= cap_eff;
  if (!used) {
    if (tid == 0) {
      RowRec z = {};
      z.mode = kModeSkip;
      *rec = z;
    }
    return;
  }
  const RowParams rp = row_params(A, r);
  const float T = rp.T;
  const bool greedy = rp.greedy;
  const float P = rp.P;
  int k_eff = rp.k_eff;
  bool topp_on = rp.topp_on;
  const float teff = greedy ? 1.0f : T;
  const float c = kLog2e / teff;
  const int d = tested ? A.draft_tokens[i] : -1;
  const bool d_ok = d >= 0 && d < V;
  // q(d) is read now so its latency hides behind the stream
  const float qd = (!greedy && d_ok && A.draft_probs)
                       ? A.draft_probs[(size_t)i * (size_t)A.ld_q + d] : 0.0f;
  const uint32_t rid = A.request_id ? A.request_id[r] : (uint32_t)r;
  const uint32_t pos0 = A.position0 ? A.position0[r] : 0u;

  RowRec out = {};
  out.lse = 0.0f;
  out.pd = 0.0;
  const bool need_sum_build = A.build != 0;
  StreamAcc acc;

  if (tid == 0) sh.woverflow = 0;
  if (tid < kWaves) sh.wtau[tid] = -__int_as_float(0x7F800000);
  __syncthreads();

  // ------------------------------------------------ greedy rows
  if (greedy) {
    if (need_sum_build) stream_row<DT, false, true, true>(row, V, c, 1, 1, 0, sh, acc, A.level != 0);
    else stream_row<DT, false, false, true>(row, V, c, 1, 1, 0, sh, acc, A.level != 0);
    const float m = block_max_f(acc.mx, sh.fscr);
    const uint64_t cand = acc.mx == m ? (uint64_t)(uint32_t)(0x7FFFFFFF - acc.bi) : 0ull;
    const int a = 0x7FFFFFFF - (int)(uint32_t)block_max_u64(cand, sh.uscr);
    if (need_sum_build) {
      const double part = acc.s * exp2((double)(acc.mx - m) * (double)c);
      const double Z = block_sum_d(part, sh.dscr);
      out.lse = (float)((double)m / (double)teff + log(Z));
    }
    greedy_record(out, m, a, tested, d, d_ok);
    if (tid == 0) *rec = out;
    return;
  }

  // ------------------------------------------------ sampled rows
  const bool all_mode = k_eff == V && !topp_on;
  // vector candidates on the verify path; the build path also sums the row
  // and takes the element buffer (fewer live registers than both together)
  const bool vec_mode = !need_sum_build && k_eff < V && k_eff <= kTopkVec;
  const bool topk_mode = k_eff < V && k_eff <= kTopkFast && !vec_mode;
  const bool topp_mode = k_eff == V && topp_on;
  const bool buf_mode = topk_mode || topp_mode;
  const bool need_sum = need_sum_build || all_mode || topp_mode;
  int keep, thresh, ramp;
  if (topk_mode) {
    keep = k_eff;
    thresh = 2 * keep < 128 ? 128 : (2 * keep > 512 ? 512 : 2 * keep);
    ramp = keep > 64 ? 1 : 0;
  } else {
    keep = kKeepTopP;
    thresh = kThreshTopP;
    ramp = 2;
  }
  if (vec_mode) {
    stream_row<DT, false, false, false, 1>(row, V, c, k_eff, kThreshVec, 0, sh, acc, A.level != 0);
  } else if (all_mode) {
    if (need_sum_build) stream_row<DT, false, true, true>(row, V, c, 1, 1, 0, sh, acc, A.level != 0);
    else stream_row<DT, false, true, false>(row, V, c, 1, 1, 0, sh, acc, A.level != 0);
  } else if (topp_mode) {
    stream_row<DT, false, true, false, 2>(row, V, c, keep, thresh, 0, sh, acc, A.level != 0);
  } else if (buf_mode) {
    if (need_sum) stream_row<DT, true, true, false>(row, V, c, keep, thresh, ramp, sh, acc, A.level != 0);
    else stream_row<DT, true, false, false>(row, V, c, keep, thresh, ramp, sh, acc, A.level != 0);
  } else {
    if (need_sum) stream_row<DT, false, true, false>(row, V, c, 1, 1, 0, sh, acc, A.level != 0);
    else stream_row<DT, false, false, false>(row, V, c, 1, 1, 0, sh, acc, A.level != 0);
  }
  const float m = block_max_f(acc.mx, sh.fscr);
  double Z = 0.0;
  if (need_sum) {
    const double part = acc.s * exp2((double)(acc.mx - m) * (double)c);
    Z = block_sum_d(part, sh.dscr);
    out.lse = (float)((double)m / (double)T + log(Z));
  }
  out.m = m;
  const double Td = (double)T;
  double pd = 0.0;
  bool exact = !buf_mode && !all_mode && !vec_mode;
  VecKept kk = {};
  uint32_t cert_code0 = 0xFFFFFFFFu;  // lowest bf16 code of the certified elements (or unknown)

  if (vec_mode) {
    if (sh.woverflow) {
      exact = true;
    } else {
      // one wave finishes the row; the others wait only to join an exact
      // fallback (wave 1 draws the ratio-test uniform meanwhile)
      if (wave_id() == 1 && lane_id() == 0 && tested)
        sh.dscr[1] = accept_uniform(A.seed, rid, pos0 + (uint32_t)j);
      if (wave_id() == 0) {
        ListEntry* L = A.list + (size_t)i * kListCap;
        const float* qrow = tested ? A.draft_probs + (size_t)i * (size_t)A.ld_q : nullptr;
        const bool ok = topk_vec_finish<DT>(V, k_eff, m, T, topp_on, P, d_ok ? d : -1,
                                            RowSplit<DT>(row, V), qrow, sh, out, pd, L, kk);
        if (lane_id() == 0) sh.found = ok ? 1 : 0;
      }
      __syncthreads();
      if (!sh.found) exact = true;
      else if (wave_id() != 0) return;
    }
  } else if (all_mode) {
    if (need_sum_build) {
      const uint64_t cand = acc.mx == m ? (uint64_t)(uint32_t)(0x7FFFFFFF - acc.bi) : 0ull;
      out.a = 0x7FFFFFFF - (int)(uint32_t)block_max_u64(cand, sh.uscr);
    } else {
      out.a = -1;  // not needed on the verify path
    }
    out.mode = kModeAll;
    out.nkeep = V;
    out.zk = out.zn = Z;
    if (d_ok) {
      const float xd = Vec<DT>::load1(row, d);
      pd = exp(((double)xd - (double)m) / Td) / Z;
    }
  } else if (buf_mode) {
    __syncthreads();  // segments, counts and thresholds final
    int n = 0;
    if (sh.woverflow) {
      exact = true;
    } else if (topp_mode) {
      n = topp_certified<DT>(row, V, m, T, P, Z, sh, cert_code0);
      if (n < 0) exact = true;
    } else {
      n = merge_segments(sh);
      if (n < k_eff) {
        exact = true;  // fewer finite candidates than k
      } else if (n > k_eff) {
        compact_top(sh, n, k_eff);
        n = k_eff;
      }
    }
    if (!exact && topp_mode) {
      TopPOut tp;
      if (!topp_select<DT>(sh, n, m, T, P, Z, d_ok ? d : -1, A.build != 0, cert_code0, tp)) {
        exact = true;  // the certified candidates do not reach the top-p mass
      } else {
        out.a = tp.a;
        out.zk = Z;
        out.zn = tp.zn;
        out.nkeep = tp.nkeep;
        pd = tp.pd;
        out.mode = kModeList;
        ListEntry* L = A.list + (size_t)i * kListCap;
        for (int t = tid; t < tp.nkeep; t += kBlock) {
          const uint64_t v = sh.buf[t];
          ListEntry le;
          le.idx = entry_idx(v);
          le.x = entry_val(v);
          L[t] = le;
        }
      }
    } else if (!exact) {
      sort_desc(sh, n);
      // fp64 weights and prefix masses over contiguous per-thread chunks
      const int ch = (n + kBlock - 1) / kBlock;
      const int t0 = tid * ch;
      double loc = 0.0;
      for (int t = t0; t < t0 + ch && t < n; ++t)
        loc += exp(((double)entry_val(sh.buf[t]) - (double)m) / Td);
      double total;
      const double base = block_exclusive_sum_d(loc, sh.dscr, &total);
      const double zk = topk_mode ? total : Z;
      const double target = topp_on ? (double)P * zk : 2.0 * total + 1.0;
      // kept count: entries whose exclusive prefix mass is below the target
      int kept_loc = 0;
      double run = base;
      for (int t = t0; t < t0 + ch && t < n; ++t) {
        const double w = exp(((double)entry_val(sh.buf[t]) - (double)m) / Td);
        if (run < target) ++kept_loc;
        run += w;
      }
      int nkeep = block_sum_i(kept_loc, sh.iscr);
      if (nkeep < 1) nkeep = 1;
      if (topp_mode && total < target) {
        exact = true;  // the certified candidates do not reach the top-p mass
      } else {
        // Z_N = prefix mass through entry nkeep-1
        if (tid == 0) { sh.zn_shared = 0.0; sh.found = -1; }
        __syncthreads();
        run = base;
        for (int t = t0; t < t0 + ch && t < n; ++t) {
          const double w = exp(((double)entry_val(sh.buf[t]) - (double)m) / Td);
          run += w;
          if (t == nkeep - 1) sh.zn_shared = run;
          if (d_ok && t < nkeep && entry_idx(sh.buf[t]) == d) sh.found = t;
        }
        __syncthreads();
        const double zn = sh.zn_shared;
        const int fd = sh.found;
        out.a = entry_idx(sh.buf[0]);
        out.zk = zk;
        out.zn = zn;
        out.nkeep = nkeep;
        if (fd >= 0) pd = exp(((double)entry_val(sh.buf[fd]) - (double)m) / Td) / zn;
        if (nkeep <= kListCap) {
          out.mode = kModeList;
          ListEntry* L = A.list + (size_t)i * kListCap;
          for (int t = tid; t < nkeep; t += kBlock) {
            const uint64_t v = sh.buf[t];
            ListEntry le;
            le.idx = entry_idx(v);
            le.x = entry_val(v);
            L[t] = le;
          }
        } else {
          out.mode = kModeRange;
          const uint32_t bkey = (uint32_t)(sh.buf[nkeep - 1] >> 32);
          int ties = 0;
          for (int t = tid; t < nkeep; t += kBlock) ties += ((uint32_t)(sh.buf[t] >> 32) == bkey);
          out.bkey = bkey;
          out.nb = block_sum_i(ties, sh.iscr);
        }
      }
    }
  }

  if (exact) {
    // the multi-pass exact path, run by this row's workgroup; Z_K of the
    // stream goes with the record (0 when the row summed nothing)
    out.mode = kModePending;
    out.zk = need_sum ? Z : 0.0;
    // (the record and the request's values are read back by the exact path:
    // handing them over in registers raised the whole kernel's register count
    // and slowed the streaming loop of every other row)
    if (tid == 0) *rec = out;
    __threadfence_block();
    __syncthreads();
    resolve_pending<DT>(A, i, r, j, tested, !A.build && j == cap_eff, sh);
    return;
  }

  if (tested) {
    out.flags |= kRecTested;
    out.pd = pd;
    if (!d_ok) {
      out.flags |= kRecBadDraft;
    } else {
      const double q = (double)qd;
      const double ratio = q > 0.0 ? fmin(1.0, pd / q) : (pd > 0.0 ? 1.0 : 0.0);
      const double u = vec_mode && !exact ? sh.dscr[1] : accept_uniform(A.seed, rid, pos0 + (uint32_t)j);
      if (u < ratio) out.flags |= kRecAccept;
    }
  }
  // the token this row emits if it is its request's emit row: after a
  // rejection (residual race; p for an out-of-range draft) or as the bonus
  const bool rejected = tested && !(out.flags & kRecAccept);
  // (a block-verified request's token depends on the whole block: its
  // finalize races it)
  if ((rejected || (!A.build && j == cap_eff)) && !A.block) {
    bool empty = false;
    if (vec_mode) {
      out.sample = wave_kept_race(kk, rejected && d_ok, A.seed, rid, pos0 + (uint32_t)j, empty);
      out.flags |= kRecSampled | (empty ? kRecResidEmpty : 0);
    } else if (buf_mode && out.mode == kModeList) {
      const float* qrow = A.draft_probs + (size_t)i * (size_t)A.ld_q;
      out.sample = block_kept_race(out.nkeep, m, out.zn, T, qrow, rejected && d_ok, A.seed, rid,
                                   pos0 + (uint32_t)j, sh, empty);
      out.flags |= kRecSampled | (empty ? kRecResidEmpty : 0);
    }
  }
  if (tid == 0) *rec = out;
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void row_pass_kernel(VerifyArgs A) {
  __shared__ RowShared sh;
  if (A.dtype == 1) row_pass<1>(A, sh);
  else row_pass<0>(A, sh);
}

// ------------------------------------------------------ pending rows
// Exact kept set of a row the streaming pass could not settle (candidate
// overflow, a top-p mass beyond the buffer, or top-k above the buffer), then
// p(d) and the ratio test of its draft.  Rewrites the row record.
// The exact path of a pending row, its inputs loaded from the record and the
// request's arrays (the finalize and build kernels).
template <int DT>
__device__ __forceinline__ void resolve_pending(const VerifyArgs& A, int i, int r, int j,
                                                bool tested, bool bonus, RowShared& sh) {
  PendingIn in;
  in.m = A.rec[i].m;
  in.zk = A.rec[i].zk;
  in.rp = row_params(A, r);
  in.d = tested ? A.draft_tokens[i] : -1;
  const bool d_ok = in.d >= 0 && in.d < A.vocab;
  const void* row = (const char*)A.logits + (size_t)i * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
  in.xd = d_ok ? Vec<DT>::load1(row, in.d) : 0.0f;
  in.qd = tested && d_ok ? A.draft_probs[(size_t)i * (size_t)A.ld_q + in.d] : 0.0f;
  in.rid = A.request_id ? A.request_id[r] : (uint32_t)r;
  in.pos0 = A.position0 ? A.position0[r] : 0u;
  resolve_pending_in<DT>(A, i, j, tested, bonus, in, sh);
}

template <int DT>
__device__ __forceinline__ void resolve_pending_in(const VerifyArgs& A, int i, int j, bool tested,
                                                   bool bonus, const PendingIn& in, RowShared& sh) {
  const int V = A.vocab;
  const float T = in.rp.T;
  const int k_eff = in.rp.k_eff;
  const bool topp_on = in.rp.topp_on;
  const float P = in.rp.P;
  const void* row = (const char*)A.logits + (size_t)i * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
  const int d = in.d;
  const bool d_ok = d >= 0 && d < V;
  const float xd = in.xd;
  ExactOut eo;
  bool listed = false, done = false;
  int tie_cut = V;
  if constexpr (DT == 1) {
    if (k_eff == V && topp_on) {
      int tcut = V;
      done = exact_topp_codes<DT>(row, V, in.m, T, P, d_ok ? d : -1, xd, in.zk, A.build != 0,
                                  A.list + (size_t)i * kListCap, sh, eo, tcut, listed);
      tie_cut = tcut;
    }
  }
  if (!done) {
    exact_kept_set<DT>(row, V, in.m, T, k_eff, topp_on ? P : 1.0f, d_ok ? d : -1, xd, sh, eo);
    // one ranked pass: the kept entries (when they fit a list) and the id
    // just past the last kept tie at the boundary; a kept set that fits
    // becomes an explicit list, sorted
    const uint32_t bkey = eo.bkey;
    const int nb = eo.nb;
    const bool fits = eo.nkeep <= kListCap;
    if (threadIdx.x == 0) {
      sh.count = 0;
      sh.found = V;
    }
    __syncthreads();
    for_each_element_ranked<DT>(
        row, V, [&](float x) { return fkey(x) == bkey; },
        [&](float x, int v, int rank) {
          const uint32_t key = fkey(x);
          if (key == bkey && rank == nb - 1) sh.found = v + 1;
          if (fits && (key > bkey || (key == bkey && rank < nb))) {
            const int slot = atomicAdd(&sh.count, 1);
            if (slot < kCap) sh.buf[slot] = make_entry(x, v);
          }
        },
        sh);
    __syncthreads();
    const int n = sh.count;
    tie_cut = sh.found;
    __syncthreads();
    if (fits && n == eo.nkeep) {
      sort_desc(sh, n);
      ListEntry* L = A.list + (size_t)i * kListCap;
      for (int t = threadIdx.x; t < n; t += kBlock) {
        const uint64_t en = sh.buf[t];
        ListEntry le;
        le.idx = entry_idx(en);
        le.x = entry_val(en);
        L[t] = le;
      }
      listed = true;
    }
  }
  RowRec out = A.rec[i];  // the row's record as the streaming pass left it
  out.tie_cut = tie_cut;
  out.mode = listed ? kModeList : kModeRange;
  out.a = eo.argmax;
  out.bkey = eo.bkey;
  out.nb = eo.nb;
  out.nkeep = eo.nkeep;
  out.zk = eo.zk;
  out.zn = eo.zn;
  out.flags |= kRecExact | kRecTieCut;
  double pd = 0.0;
  if (d_ok) {
    const uint32_t kd = fkey(xd);
    const bool in = kd > eo.bkey || (kd == eo.bkey && eo.tie_d < eo.nb);
    pd = in ? exp(((double)xd - (double)out.m) / (double)T) / eo.zn : 0.0;
  }
  const uint32_t rid = in.rid;
  const uint32_t pos0 = in.pos0;
  if (tested) {
    out.flags |= kRecTested;
    out.pd = pd;
    if (!d_ok) {
      out.flags |= kRecBadDraft;
    } else {
      const double q = (double)in.qd;
      const double ratio = q > 0.0 ? fmin(1.0, pd / q) : (pd > 0.0 ? 1.0 : 0.0);
      const double u = accept_uniform(A.seed, rid, pos0 + (uint32_t)j);
      if (u < ratio) out.flags |= kRecAccept;
    }
  }
  // the emitted token if this row is its request's emit row (listed sets only)
  const bool rejected = tested && !(out.flags & kRecAccept);
  if (listed && (rejected || bonus) && !A.block) {
    bool empty = false;
    const float* qrow = A.draft_probs + (size_t)i * (size_t)A.ld_q;
    out.sample = block_kept_race(out.nkeep, out.m, out.zn, T, qrow, rejected && d_ok, A.seed,
                                 rid, pos0 + (uint32_t)j, sh, empty);
    out.flags |= kRecSampled | (empty ? kRecResidEmpty : 0);
  }
  __syncthreads();
  if (threadIdx.x == 0) A.rec[i] = out;
  __threadfence_block();
  __syncthreads();
}

// fp32 screening bound for the stream race: |log2 key_32 - log2 key| < kEta.
constexpr float kEta = 0.0078125f;     // 2^-7, in log2 units
constexpr float kRelP = 1.0e-4f;       // relative error bound of p_32
constexpr int kSlots = 8;              // candidate slots per thread

__device__ __forceinline__ float race_log2e32(uint64_t seed, uint32_t rid, uint32_t pos,
                                              uint32_t v) {
  const uint32_t w = race_word(seed, rid, pos, 1u, v);
  const float U = (float)(2u * (w >> 9) + 1u) * 0x1.0p-24f;
  const float E = U > 0.5f ? -log1pf(-(1.0f - U)) : -logf(U);
  return log2f(E);
}

// Race over the whole row (kModeAll / kModeRange), weights p (residual=false)
// or max(0, p - q).  Returns id (-1 when every weight is zero).
template <int DT>
__device__ int stream_race(const void* row, int V, const RowRec& rr, float T, const float* qrow,
                           bool residual, uint64_t seed, uint32_t rid, uint32_t pos,
                           RowShared& sh) {
  const float c = kLog2e / T;
  const double Td = T;
  const float l2zn = (float)log2(rr.zn);
  const bool range = rr.mode == kModeRange;
  const uint32_t bkey = rr.bkey;
  const int nb = rr.nb;
  int* slot_id = (int*)sh.buf;                       // [kBlock * kSlots]
  float* slot_up = (float*)(slot_id + kBlock * kSlots);
  int nslot = 0;
  float best_lo = -INFINITY;
  const int tid = threadIdx.x;
  auto visit = [&](float x, int v, int rank) {
    const uint32_t key = fkey(x);
    const bool in = !range || key > bkey || (key == bkey && rank < nb);
    if (!in) return;
    const float y = (x - rr.m) * c;          // log2 of the weight relative to the max
    // -log2 E_v <= 24 (race uniforms lie in [2^-24, 1 - 2^-24]): an element whose
    // weight cannot beat the best lower bound even then needs no uniform
    if (!(y - (residual ? l2zn : 0.0f) + 24.0f + 2.0f * kEta >= best_lo)) return;
    float lo, up;
    if (!residual) {
      if (!(y > -1.0e30f)) return;
      const float l2e = race_log2e32(seed, rid, pos, (uint32_t)v);
      const float kap = y - l2e;
      lo = kap - kEta;
      up = kap + kEta;
    } else {
      const float p32 = exp2f(y - l2zn);
      const float q = qrow[v];
      const float rhi = p32 * (1.0f + kRelP) - q;
      if (!(rhi > 0.0f)) return;
      const float rlo = p32 * (1.0f - kRelP) - q;
      const float l2e = race_log2e32(seed, rid, pos, (uint32_t)v);
      up = log2f(rhi) - l2e + kEta;
      lo = rlo > 0.0f ? log2f(rlo) - l2e - kEta : -INFINITY;
    }
    if (up >= best_lo) {
      if (nslot == kSlots) {
        // drop slots that can no longer win
        const float bl = fmaxf(best_lo, lo);
        int w = 0;
        for (int s2 = 0; s2 < kSlots; ++s2) {
          const int sid = slot_id[tid * kSlots + s2];
          const float su = slot_up[tid * kSlots + s2];
          if (su >= bl) {
            slot_id[tid * kSlots + w] = sid;
            slot_up[tid * kSlots + w] = su;
            ++w;
          }
        }
        nslot = w;
      }
      if (nslot < kSlots) {
        slot_id[tid * kSlots + nslot] = v;
        slot_up[tid * kSlots + nslot] = up;
        ++nslot;
      } else {
        // more than kSlots candidates within the screening band of each other:
        // replace the smallest upper bound
        int ws = 0;
        for (int s2 = 1; s2 < kSlots; ++s2)
          if (slot_up[tid * kSlots + s2] < slot_up[tid * kSlots + ws]) ws = s2;
        if (slot_up[tid * kSlots + ws] < up) {
          slot_id[tid * kSlots + ws] = v;
          slot_up[tid * kSlots + ws] = up;
        }
      }
    }
    best_lo = fmaxf(best_lo, lo);
  };
  if (range) {
    for_each_element_ranked<DT>(row, V, [&](float x) { return fkey(x) == bkey; }, visit, sh);
  } else {
    for_each_element<DT>(row, V, [&](float x, int v) { visit(x, v, 0); });
  }
  // block-wide best lower bound, then exact fp64 keys of the slots above it
  const float B = block_max_f(best_lo, sh.fscr);
  RaceBest b = {-1.0, 0x7FFFFFFF};
  for (int s2 = 0; s2 < nslot; ++s2) {
    if (slot_up[tid * kSlots + s2] < B) continue;
    const int v = slot_id[tid * kSlots + s2];
    const double x = (double)Vec<DT>::load1(row, v);
    double wgt = exp((x - (double)rr.m) / Td) / rr.zn;
    if (residual) wgt = wgt - (double)qrow[v];
    if (!(wgt > 0.0)) continue;
    const double key = wgt / race_e(seed, rid, pos, (uint32_t)v);
    if (race_better(key, v, b.key, b.id)) { b.key = key; b.id = v; }
  }
  __syncthreads();
  RaceBest w = block_race_best(b, sh);
  return w.key > 0.0 ? w.id : -1;
}

// fp32 bounds on log2 of an element's race key (weight / E, E = -ln U) for
// the rows whose kept set is the whole row or a key range: lo <= log2 key <=
// up within kEta of the exact value, from one Philox call per four
// consecutive tokens (cached).  An element whose best possible key is below a
// bound `bl` needs no uniform (-log2 E <= 24: race uniforms lie in
// [2^-24, 1 - 2^-24]).
struct RaceBounds {
  float m, c, l2zn;      // max, log2(e)/T, log2 Z_N (residual) or 0
  uint32_t kmin;         // kept keys: > kmin, or == kmin with id < tie_cut
  int tie_cut;
  bool residual;
  const float* qrow;
  uint32_t k0, k1, rid, pos;
  uint32_t gcache;
  uint4 oc;

  __device__ __forceinline__ RaceBounds(float m_, double zn, float T, uint32_t kmin_, int tie_cut_,
                                        bool residual_, const float* qrow_, uint64_t seed,
                                        uint32_t rid_, uint32_t pos_)
      : m(m_), c(kLog2e / T), l2zn(residual_ ? (float)log2(zn) : 0.0f), kmin(kmin_),
        tie_cut(tie_cut_), residual(residual_), qrow(qrow_), k0((uint32_t)seed),
        k1((uint32_t)(seed >> 32)), rid(rid_), pos(pos_), gcache(0xFFFFFFFFu),
        oc(make_uint4(0u, 0u, 0u, 0u)) {}

  // log2 weight bound of a whole vector from its maximum
  __device__ __forceinline__ bool vector_may_reach(float vmax, float bl) const {
    return (vmax - m) * c - l2zn + 24.0f + 2.0f * kEta >= bl;
  }

  // false when the element is outside the kept range or cannot reach bl
  __device__ __forceinline__ bool bounds(float x, int v, float bl, float& lo, float& up) {
    return bounds(x, v, residual ? qrow[v] : 0.0f, bl, lo, up);
  }
  // the same with the element's draft probability q (residual rows) given
  __device__ __forceinline__ bool bounds(float x, int v, float q, float bl, float& lo, float& up) {
    float y;
    if (!prefilter(x, v, bl, y)) return false;
    const uint32_t g = (uint32_t)v >> 2;
    if (g != gcache) {
      oc = philox4x32_10(k0, k1, make_uint4(pos, rid, 1u, g));
      gcache = g;
    }
    const uint32_t ln = (uint32_t)v & 3u;
    const uint32_t wv = ln == 0 ? oc.x : (ln == 1 ? oc.y : (ln == 2 ? oc.z : oc.w));
    return from_word(y, wv, q, bl, lo, up);
  }
  // Generator block of group g (elements 4g .. 4g+3).
  __device__ __forceinline__ uint4 words(uint32_t g) const {
    return philox4x32_10(k0, k1, make_uint4(pos, rid, 1u, g));
  }
  // The checks that need no generator word: y = log2 of p (residual) or of
  // the relative weight; false when the element is outside the kept range or
  // cannot reach bl even with E at its smallest.
  __device__ __forceinline__ bool prefilter(float x, int v, float bl, float& y) const {
    y = (x - m) * c - l2zn;
    if (!(y + 24.0f + 2.0f * kEta >= bl)) return false;
    const uint32_t key = fkey(x);
    return !(key < kmin || (key == kmin && v >= tie_cut));
  }
  // The checks on the generator word wv that need no logarithm: false when
  // the element cannot reach bl.
  __device__ __forceinline__ bool cheap(float y, uint32_t wv, float q, float bl) const {
    // E = -ln U >= 1 - U = D 2^-24 (D an integer in [1, 2^24)), so log2 E >=
    // floor(log2 D) - 24
    const uint32_t Dlt = 0x1000000u - (2u * (wv >> 9) + 1u);
    const int e_lo = 7 - (int)__clz(Dlt);
    if (!(y + (residual ? 2.0e-4f : 0.0f) - (float)e_lo + 2.0f * kEta >= bl)) return false;
    if (residual) {
      // the residual's upper bound with q: the key is at most rhi / 2^e_lo
      // (an exact scaling by a power of two while the result stays normal)
      const float rhi = exp2f(y) * (1.0f + 2.0f * kRelP) - q;  // 2 kRelP: room for the rounding of the difference
      if (!(rhi > 0.0f)) return false;
      if (bl > -100.0f && ldexpf(rhi, -e_lo) < exp2f(bl - 2.0f * kEta)) return false;
    }
    return true;
  }
  // The bounds with the logarithms (after cheap() passed).
  __device__ __forceinline__ bool full(float y, uint32_t wv, float q, float bl, float& lo,
                                      float& up) const {
    constexpr float kNegInf = -__builtin_huge_valf();
    // log2 E, E = -ln U, within far less than kEta: a short series for U near 1
    const float U = (float)(2u * (wv >> 9) + 1u) * 0x1.0p-24f;
    const float dlt = 1.0f - U;  // exact
    const float E = dlt < 0x1.0p-10f ? dlt * (1.0f + 0.5f * dlt)
                                     : -__builtin_amdgcn_logf(U) * 0.6931471805599453f;
    const float l2e = __builtin_amdgcn_logf(E);
    if (!residual) {
      lo = y - l2e - kEta;
      up = y - l2e + kEta;
      return true;
    }
    if (!(y + 2.0e-4f - l2e + kEta >= bl)) return false;  // even with q = 0
    const float p32 = exp2f(y);
    const float rhi = p32 * (1.0f + 2.0f * kRelP) - q;
    const float rlo = p32 * (1.0f - 2.0f * kRelP) - q;
    up = log2f(rhi) - l2e + kEta;
    lo = rlo > 0.0f ? log2f(rlo) - l2e - kEta : kNegInf;
    return true;
  }
  // Bounds from the element's generator word wv.
  __device__ __forceinline__ bool from_word(float y, uint32_t wv, float q, float bl, float& lo,
                                           float& up) const {
    return cheap(y, wv, q, bl) && full(y, wv, q, bl, lo, up);
  }
};

// Exact fp64 race key of element v (value x) of a full or range row.
__device__ __forceinline__ void race_exact(float x, int v, float m, double zn, double Td,
                                           const float* qrow, bool residual, uint64_t seed,
                                           uint32_t rid, uint32_t pos, RaceBest& b) {
  double wgt = exp(((double)x - (double)m) / Td) / zn;
  if (residual) wgt = wgt - (double)qrow[v];
  if (!(wgt > 0.0)) return;
  const double key = wgt / race_e(seed, rid, pos, (uint32_t)v);
  if (race_better(key, v, b.key, b.id)) {
    b.key = key;
    b.id = v;
  }
}

// Candidates of one thread while streaming: its two best upper bounds, the
// largest upper bound it dropped, and its best lower bound.
struct RaceTop2 {
  float best_lo, up1, up2, dropped;
  int id1, id2;
  __device__ __forceinline__ RaceTop2()
      : best_lo(-__builtin_huge_valf()), up1(-__builtin_huge_valf()),
        up2(-__builtin_huge_valf()), dropped(-__builtin_huge_valf()), id1(-1), id2(-1) {}
  __device__ __forceinline__ void add(float lo, float up, int v) {
    best_lo = fmaxf(best_lo, lo);
    if (up > up1) {
      dropped = fmaxf(dropped, up2);
      up2 = up1;
      id2 = id1;
      up1 = up;
      id1 = v;
    } else if (up > up2) {
      dropped = fmaxf(dropped, up2);
      up2 = up;
      id2 = v;
    } else {
      dropped = fmaxf(dropped, up);
    }
  }
};

// Race over every element of an all-mode row (or a range row) by one
// workgroup.  When every dropped bound is below the block's best lower bound
// B, the winner is among the kept candidates with upper bound >= B, which are
// evaluated exactly in fp64.  Returns -2 when that does not hold (the caller
// falls back).
template <int DT>
__device__ int stream_race_all(const void* row, int V, float m, double zn, uint32_t kmin,
                               int tie_cut, float T, const float* qrow, bool residual,
                               uint64_t seed, uint32_t rid, uint32_t pos, RowShared& sh) {
  constexpr int P = Vec<DT>::kEpv;
  constexpr float kNegInf = -__builtin_huge_valf();
  RaceBounds rb(m, zn, T, kmin, tie_cut, residual, qrow, seed, rid, pos);
  RaceTop2 t2;
  auto elem = [&](float x, int v) {
    float lo, up;
    if (rb.bounds(x, v, t2.best_lo, lo, up)) t2.add(lo, up, v);
  };
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  if (tid < sp.head) elem(Vec<DT>::load1(row, tid), tid);
  for (int vi = tid; vi < sp.nvec; vi += kBlock) {
    float x[P];
    Vec<DT>::unpack(__ldg(sp.vbase + vi), x);
    // whole vectors below the bound skip their uniforms
    if (!rb.vector_may_reach(vec_max<P>(x), t2.best_lo)) continue;
    const int b = sp.head + vi * P;
#pragma unroll
    for (int e = 0; e < P; ++e) elem(x[e], b + e);
  }
  if (sp.tail0 + tid < V) elem(Vec<DT>::load1(row, sp.tail0 + tid), sp.tail0 + tid);
  const float B = block_max_f(t2.best_lo, sh.fscr);
  const float D = block_max_f(t2.dropped, sh.fscr);
  if (D > kNegInf && !(D < B)) return -2;
  RaceBest b = {-1.0, 0x7FFFFFFF};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int v = t == 0 ? t2.id1 : t2.id2;
    const float u = t == 0 ? t2.up1 : t2.up2;
    if (v < 0 || !(u >= B)) continue;
    race_exact(Vec<DT>::load1(row, v), v, m, zn, (double)T, qrow, residual, seed, rid, pos, b);
  }
  const RaceBest w = block_race_best(b, sh);
  return w.key > 0.0 ? w.id : -1;
}

// One segment of a full-vocabulary race: item (r, s) of the race grid (a
// grid-stride loop over requests x segments; items of requests without a
// race end at once).  The same bounds as stream_race_all, with the next three
// vectors (and the next vector's draft probabilities) in flight while one is
// screened; the segment's exact winner goes to race_part[r, s].  When a
// dropped bound reaches the segment's best lower bound B, a second pass over
// the segment evaluates exactly every element whose upper bound reaches B.
template <int DT>
__device__ __forceinline__ void race_segment(const VerifyArgs& A, int r, int sg, int S,
                                             RowShared& sh) {
  constexpr int P = Vec<DT>::kEpv;
  constexpr float kNegInf = -__builtin_huge_valf();
  const int job = A.race_job[r];
  const int is = job >> 1;
  const bool residual = (job & 1) != 0;
  const RowRec rr = A.rec[is];
  const int V = A.vocab;
  const float T = A.temperature[r];
  const uint32_t rid = A.request_id ? A.request_id[r] : (uint32_t)r;
  const uint32_t pos = (A.position0 ? A.position0[r] : 0u) + (uint32_t)(is - A.qo[r]);
  const uint64_t seed = A.seed;
  const void* row = (const char*)A.logits + (size_t)is * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
  const float* qrow = A.draft_probs + (size_t)is * (size_t)A.ld_q;
  const bool range = rr.mode == kModeRange;
  const double zn = A.race_zn[r];  // Z_N, or Z_N / p_tau for a block-verified residual
  RaceBounds rb(rr.m, zn, T, range ? rr.bkey : 0u, range ? rr.tie_cut : 0x7FFFFFFF,
                residual, qrow, seed, rid, pos);
  const RowSplit<DT> sp(row, V);
  const int v0 = (int)((long long)sp.nvec * sg / S);
  const int v1 = (int)((long long)sp.nvec * (sg + 1) / S);
  const int tid = threadIdx.x;
  const double Td = T;
  RaceTop2 t2;
  RaceBest b = {-1.0, 0x7FFFFFFF};
  float B = kNegInf;
  bool second = false;
  // first pass: bounds against the thread's best lower bound; second pass:
  // the ids of the elements whose upper bound reaches B, listed in LDS
  int* cand = (int*)sh.buf;
  constexpr int kCandCap = 2 * kCap;
  auto visit = [&](float x, int v, float q) {
    float lo, up;
    if (!second) {
      if (rb.bounds(x, v, q, t2.best_lo, lo, up)) t2.add(lo, up, v);
    } else if (rb.bounds(x, v, q, B, lo, up) && up >= B) {
      const int slot = atomicAdd(&sh.count, 1);
      if (slot < kCandCap) cand[slot] = v;
    }
  };
  // visit with the element's generator word given
  auto visit_w = [&](float x, int v, float q, uint32_t wv) {
    float lo, up, y;
    const float bl = second ? B : t2.best_lo;
    if (!rb.prefilter(x, v, bl, y) || !rb.from_word(y, wv, q, bl, lo, up)) return;
    if (!second) {
      t2.add(lo, up, v);
    } else if (up >= B) {
      const int slot = atomicAdd(&sh.count, 1);
      if (slot < kCandCap) cand[slot] = v;
    }
  };
  // loads past the segment's end read its last vector again (not used), so
  // every iteration issues the same loads and each wait covers only the
  // vector being visited
  const int vlast = v1 - 1;
  // q of a vector's elements in 16-byte loads when the row's q starts on 16
  // bytes at the first vector (the same for every vector of the row)
  const bool qvec = residual && P % 4 == 0 && ((uintptr_t)(qrow + sp.head) & 15u) == 0;
  auto qload = [&](int vi, float* q) {
    const int vq = vi < v1 ? vi : vlast;
    if (qvec) {
      const float4* qp = (const float4*)(qrow + sp.head + vq * P);
#pragma unroll
      for (int h = 0; h < P / 4; ++h) {
        const float4 t = __ldg(qp + h);
        q[4 * h] = t.x;
        q[(4 * h + 1) % P] = t.y;
        q[(4 * h + 2) % P] = t.z;
        q[(4 * h + 3) % P] = t.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < P; ++e) q[e] = residual ? qrow[sp.head + vq * P + e] : 0.0f;
    }
  };
  for (int pass = 0; pass < 2; ++pass) {
    if (sg == 0 && tid < sp.head)
      visit(Vec<DT>::load1(row, tid), tid, residual ? qrow[tid] : 0.0f);
    const bool any = v1 > v0;  // an empty segment loads nothing
    auto vload = [&](int v) { return __ldg(sp.vbase + (v < v1 ? v : vlast)); };
    // one vector of this lane (vi; past the segment's end it only takes part
    // in the wave's ballots and bound sharing)
    auto vec_step = [&](int vi, const uint4& w, const float* q) {
      float x[P];
      Vec<DT>::unpack(w, x);
      const bool act = vi < v1 && rb.vector_may_reach(vec_max<P>(x), second ? B : t2.best_lo);
      const int e0 = sp.head + vi * P;
      if ((e0 & 3) == 0) {  // the same in every lane (the row's head offset)
        // the vector is whole groups of four: each group's generator block
        // once per vector (the same block in every lane, so the wave runs it
        // once), one block live at a time
#pragma unroll 1
        for (int gh = 0; gh < P / 4; ++gh) {
          if (!__ballot(act)) break;
          const uint4 o = rb.words((uint32_t)(e0 >> 2) + (uint32_t)gh);
          const uint32_t ws[4] = {o.x, o.y, o.z, o.w};
          float xs[4], qs[4];
          if (DT == 1) {
            const uint32_t w01 = gh == 0 ? w.x : w.z, w23 = gh == 0 ? w.y : w.w;
            xs[0] = bf16_lo(w01);
            xs[1] = bf16_hi(w01);
            xs[2] = bf16_lo(w23);
            xs[3] = bf16_hi(w23);
#pragma unroll
            for (int t = 0; t < 4; ++t) qs[t] = gh == 0 ? q[t] : q[(4 + t) % P];
          } else {
            xs[0] = __uint_as_float(w.x);
            xs[1] = __uint_as_float(w.y);
            xs[2] = __uint_as_float(w.z);
            xs[3] = __uint_as_float(w.w);
#pragma unroll
            for (int t = 0; t < 4; ++t) qs[t] = q[t % P];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (act) visit_w(xs[t], e0 + 4 * gh + t, qs[t], ws[t]);
        }
      } else if (act) {
        {
          // a vector across group boundaries (rows that do not start on a
          // group of four): each element's block on its own, no state kept
          auto word_of = [&](int v) {
            const uint4 o = rb.words((uint32_t)v >> 2);
            const int ln = v & 3;
            return ln == 0 ? o.x : (ln == 1 ? o.y : (ln == 2 ? o.z : o.w));
          };
#pragma unroll 1
          for (int h = 0; h < 4; ++h) {
            const uint32_t wd = h == 0 ? w.x : (h == 1 ? w.y : (h == 2 ? w.z : w.w));
            if (DT == 1) {
              const float qlo = h == 0 ? q[0] : (h == 1 ? q[2] : (h == 2 ? q[4] : q[6 % P]));
              const float qhi = h == 0 ? q[1] : (h == 1 ? q[3] : (h == 2 ? q[5] : q[7 % P]));
              visit_w(bf16_lo(wd), e0 + 2 * h, qlo, word_of(e0 + 2 * h));
              visit_w(bf16_hi(wd), e0 + 2 * h + 1, qhi, word_of(e0 + 2 * h + 1));
            } else {
              const float qlo = h == 0 ? q[0] : (h == 1 ? q[1 % P] : (h == 2 ? q[2 % P] : q[3 % P]));
              visit_w(__uint_as_float(wd), e0 + h, qlo, word_of(e0 + h));
            }
          }
        }
      }
      // every lane's best lower bound belongs to an element of this segment
      // that its own lane keeps (or whose drop forces the second pass), so
      // the wave's best is a valid filter for every lane
      if (!second) t2.best_lo = wave_max_f(t2.best_lo);
    };
    // two load buffers in turn, each consumed in place (no register copies
    // of loads in flight), the trip count the same in every lane of a wave
    int vi = v0 + tid;
    uint4 wa = make_uint4(0u, 0u, 0u, 0u), wb = wa;
    float qa[P], qb[P];
#pragma unroll
    for (int e = 0; e < P; ++e) qa[e] = qb[e] = 0.0f;
    if (any) {
      wa = vload(vi);
      qload(vi, qa);
    }
    for (; vi - lane_id() < v1; vi += 2 * kBlock) {
      wb = vload(vi + kBlock);
      qload(vi + kBlock, qb);
      vec_step(vi, wa, qa);
      wa = vload(vi + 2 * kBlock);
      qload(vi + 2 * kBlock, qa);
      vec_step(vi + kBlock, wb, qb);
    }

    if (sg == S - 1 && sp.tail0 + tid < V)
      visit(Vec<DT>::load1(row, sp.tail0 + tid), sp.tail0 + tid,
            residual ? qrow[sp.tail0 + tid] : 0.0f);
    if (pass == 1) {
      __syncthreads();
      const int nc = sh.count;
      if (nc <= kCandCap) {
        for (int t = tid; t < nc; t += kBlock) {
          const int v = cand[t];
          race_exact(Vec<DT>::load1(row, v), v, rr.m, zn, Td, qrow, residual, seed, rid, pos, b);
        }
      } else {
        // more candidates than the list holds: every element of the segment
        // whose bound reaches B, evaluated in place
        const int e_lo = sg == 0 ? 0 : sp.head + v0 * P;
        const int e_hi = sg == S - 1 ? V : sp.head + v1 * P;
        rb.gcache = 0xFFFFFFFFu;
        for (int v = e_lo + tid; v < e_hi; v += kBlock) {
          const float x = Vec<DT>::load1(row, v);
          float lo, up;
          if (rb.bounds(x, v, B, lo, up) && up >= B)
            race_exact(x, v, rr.m, zn, Td, qrow, residual, seed, rid, pos, b);
        }
      }
      break;
    }
    B = block_max_f(t2.best_lo, sh.fscr);
    const float D = block_max_f(t2.dropped, sh.fscr);
    if (D > kNegInf && !(D < B)) {
      second = true;  // a dropped candidate may win: go over the segment again
      rb.gcache = 0xFFFFFFFFu;
      if (tid == 0) sh.count = 0;
      __syncthreads();
      continue;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int v = t == 0 ? t2.id1 : t2.id2;
      const float u = t == 0 ? t2.up1 : t2.up2;
      if (v < 0 || !(u >= B)) continue;
      race_exact(Vec<DT>::load1(row, v), v, rr.m, zn, Td, qrow, residual, seed, rid, pos, b);
    }
    break;
  }
  const RaceBest w = block_race_best(b, sh);
  if (tid == 0) {
    RacePart pt;
    pt.key = w.key;
    pt.id = w.id;
    pt.pad = 0;
    A.race_part[(size_t)r * kMaxRaceSegs + sg] = pt;
  }
}

// Winner of a split race: the best segment (ties to the lower id).  A residual
// that is zero everywhere falls back to p, raced by this workgroup.
template <int DT>
__device__ __forceinline__ void race_finish(const VerifyArgs& A, RowShared& sh) {
  const int r = blockIdx.x;
  const int job = A.race_job[r];
  if (job < 0) return;
  const int is = job >> 1;
  const bool residual = (job & 1) != 0;
  const int S = *A.race_nseg;  // as the segment kernel split the races
  RaceBest b = {-1.0, 0x7FFFFFFF};
  for (int t = threadIdx.x; t < S; t += kBlock) {
    const RacePart pt = A.race_part[(size_t)r * kMaxRaceSegs + t];
    if (pt.key > 0.0 && race_better(pt.key, pt.id, b.key, b.id)) {
      b.key = pt.key;
      b.id = pt.id;
    }
  }
  const RaceBest w = block_race_best(b, sh);
  int sample = w.key > 0.0 ? w.id : -1;
  bool empty = false;
  if (residual && sample < 0) {
    empty = true;
    const RowRec rr = A.rec[is];
    const float T = A.temperature[r];
    const uint32_t rid = A.request_id ? A.request_id[r] : (uint32_t)r;
    const uint32_t pos = (A.position0 ? A.position0[r] : 0u) + (uint32_t)(is - A.qo[r]);
    const void* row = (const char*)A.logits + (size_t)is * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
    const bool range = rr.mode == kModeRange;
    sample = stream_race_all<DT>(row, A.vocab, rr.m, rr.zn, range ? rr.bkey : 0u,
                                 range ? rr.tie_cut : 0x7FFFFFFF, T, nullptr, false, A.seed, rid,
                                 pos, sh);
    if (sample == -2)
      sample = stream_race<DT>(row, A.vocab, rr, T, nullptr, false, A.seed, rid, pos, sh);
  }
  if (threadIdx.x == 0) {
    A.out_tokens[is] = sample;
    A.next_token[r] = sample;
    if (A.row_flags) A.row_flags[is] = (uint8_t)(2 | (empty ? 32 : 0));
  }
}

// Race over an explicit kept list (kModeList), fp64 throughout.
__device__ int list_race(const ListEntry* L, const RowRec& rr, float T, const float* qrow,
                         bool residual, uint64_t seed, uint32_t rid, uint32_t pos, RowShared& sh) {
  const double Td = T;
  RaceBest b = {-1.0, 0x7FFFFFFF};
  for (int t = threadIdx.x; t < rr.nkeep; t += kBlock) {
    const ListEntry le = L[t];
    double wgt = exp(((double)le.x - (double)rr.m) / Td) / rr.zn;
    if (residual) wgt = wgt - (double)qrow[le.idx];
    if (!(wgt > 0.0)) continue;
    const double key = wgt / race_e(seed, rid, pos, (uint32_t)le.idx);
    if (race_better(key, le.idx, b.key, b.id)) { b.key = key; b.id = le.idx; }
  }
  RaceBest w = block_race_best(b, sh);
  return w.key > 0.0 ? w.id : -1;
}

// ------------------------------------------------ block verification
// Test bound of one block position from its residual mass A and weight p.
__device__ __forceinline__ double block_bound(double a, double p) {
  const double den = a + 1.0 - p;
  return den > 0.0 ? a / den : 1.0;  // 0 / 0: p = 1 and the row's p and q agree
}

// Residual mass sum max(w p(x) - q(x), 0) of this thread's share of a row whose
// kept set is the whole row or a key range (every thread must call it: the
// ranked walk synchronises the block).
template <int DT>
__device__ double row_residual_mass(const VerifyArgs& A, int i, const RowRec& rr, double w,
                                    double Td, RowShared& sh) {
  const void* row = (const char*)A.logits + (size_t)i * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
  const float* qrow = A.draft_probs + (size_t)i * (size_t)A.ld_q;
  const int V = A.vocab;
  double a = 0.0;
  auto term = [&](float x, int v) {
    const double pv = exp(((double)x - (double)rr.m) / Td) / rr.zn;
    a += fmax(w * pv - (double)qrow[v], 0.0);
  };
  if (rr.mode == kModeRange && !(rr.flags & kRecTieCut)) {
    const uint32_t bkey = rr.bkey;
    const int nb = rr.nb;
    for_each_element_ranked<DT>(
        row, V, [&](float x) { return fkey(x) == bkey; },
        [&](float x, int v, int rank) {
          const uint32_t k = fkey(x);
          if (k > bkey || (k == bkey && rank < nb)) term(x, v);
        },
        sh);
  } else {
    const bool range = rr.mode == kModeRange;
    const uint32_t bkey = rr.bkey;
    const int cut = rr.tie_cut;
    for_each_element<DT>(row, V, [&](float x, int v) {
      if (range) {
        const uint32_t k = fkey(x);
        if (!(k > bkey || (k == bkey && v < cut))) return;
      }
      term(x, v);
    });
  }
  return a;
}

// Block verification of one sampled request (Sun, Mendlovic, Leviathan,
// Aharoni, Beirami, Ro, Suresh, "Block Verification Accelerates Speculative
// Decoding") over its G verified positions, rows s..s+G, every row resolved.
// Block weights p_0 = 1, p_i = min(p_{i-1} p(d)/q(d), 1) at row i - 1; the test
// of position i is u_{i-1} < h_i with h_i = A_i / (A_i + 1 - p_i), A_i the
// residual mass of row i at weight p_i (h_G = p_G); tau = the last position
// passed.  The token comes from row tau: the residual max(p_tau p - q, 0) (raced
// as max(p' - q, 0) with p' over Z_N / p_tau), or p when tau = G or row tau's
// draft is out of range.  p_i and h_i go to the workspace (block_w).
template <int DT>
__device__ void block_finalize(const VerifyArgs& A, RowShared& sh, int r, int s, int nr, int G) {
  const int tid = threadIdx.x;
  const int V = A.vocab;
  const float T = A.temperature[r];
  const double Td = T;
  const uint32_t rid = A.request_id ? A.request_id[r] : (uint32_t)r;
  const uint32_t pos0 = A.position0 ? A.position0[r] : 0u;
  double* bw = A.block_w;
  double* ratio = (double*)sh.buf;  // one chunk of ratios
  // weights: the ratios of a chunk of positions gathered in parallel, their
  // clamped running product by thread 0
  double p = 1.0;
  if (tid == 0) bw[2 * (size_t)s] = 1.0;
  for (int c0 = 0; c0 < G; c0 += kBlock) {
    const int j = c0 + tid;
    if (j < G) {
      const int d = A.draft_tokens[s + j];
      double rt = 0.0;
      if (d >= 0 && d < V) {
        const double pb = A.rec[s + j].pd;
        const double q = (double)A.draft_probs[(size_t)(s + j) * (size_t)A.ld_q + d];
        rt = q > 0.0 ? pb / q : (pb > 0.0 ? __builtin_inf() : 0.0);
      }
      ratio[tid] = rt;
    }
    __syncthreads();
    if (tid == 0) {
      const int n = G - c0 < kBlock ? G - c0 : kBlock;
      for (int t = 0; t < n; ++t) {
        p = p > 0.0 ? fmin(p * ratio[t], 1.0) : 0.0;
        bw[2 * (size_t)(s + c0 + t + 1)] = p;
      }
    }
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();
  // test bounds: listed rows one wave each, lanes over the kept entries
  for (int i = 1 + wave_id(); i < G; i += kWaves) {
    const RowRec rr = A.rec[s + i];
    if (rr.mode != kModeList) continue;
    const double w = bw[2 * (size_t)(s + i)];
    const ListEntry* Lst = A.list + (size_t)(s + i) * kListCap;
    const float* qrow = A.draft_probs + (size_t)(s + i) * (size_t)A.ld_q;
    double a = 0.0;
    for (int t = lane_id(); t < rr.nkeep; t += 64) {
      const ListEntry le = Lst[t];
      const double pv = exp(((double)le.x - (double)rr.m) / Td) / rr.zn;
      a += fmax(w * pv - (double)qrow[le.idx], 0.0);
    }
    a = wave_sum_d(a);
    if (lane_id() == 0) bw[2 * (size_t)(s + i) + 1] = block_bound(a, w);
  }
  // the other rows by the whole workgroup
  for (int i = 1; i < G; ++i) {
    const RowRec rr = A.rec[s + i];
    if (rr.mode == kModeList) continue;
    const double w = bw[2 * (size_t)(s + i)];
    const double a = block_sum_d(row_residual_mass<DT>(A, s + i, rr, w, Td, sh), sh.dscr);
    if (tid == 0) bw[2 * (size_t)(s + i) + 1] = block_bound(a, w);
    __syncthreads();
  }
  if (tid == 0 && G > 0) bw[2 * (size_t)(s + G) + 1] = bw[2 * (size_t)(s + G)];
  __threadfence_block();
  __syncthreads();
  // the last position passed
  int last = 0;
  for (int i = 1 + tid; i <= G; i += kBlock) {
    const double u = accept_uniform(A.seed, rid, pos0 + (uint32_t)(i - 1));
    if (u < bw[2 * (size_t)(s + i) + 1]) last = i;
  }
  const int tau = (int)block_max_u64((uint64_t)last, sh.uscr);
  // the emitted token of row tau
  const int is = s + tau;
  const RowRec rr = A.rec[is];
  const int dtau = tau < G ? A.draft_tokens[is] : -1;
  bool residual = tau < G && dtau >= 0 && dtau < V;
  bool resid_empty = false;
  const double wt = bw[2 * (size_t)is];
  if (residual && !(wt > 0.0)) {  // zero weight: the residual is empty
    residual = false;
    resid_empty = true;
  }
  RowRec rs = rr;
  if (residual) rs.zn = rr.zn / wt;
  const float* qrow = A.draft_probs + (size_t)is * (size_t)A.ld_q;
  const uint32_t pos = pos0 + (uint32_t)tau;
  int sample;
  int job = -1;
  if (rr.mode == kModeList) {
    const ListEntry* Lst = A.list + (size_t)is * kListCap;
    sample = list_race(Lst, rs, T, qrow, residual, A.seed, rid, pos, sh);
    if (residual && sample < 0) {
      resid_empty = true;
      sample = list_race(Lst, rr, T, qrow, false, A.seed, rid, pos, sh);
    }
  } else if (A.race_segs > 0 &&
             (rr.mode == kModeAll || (rr.mode == kModeRange && (rr.flags & kRecTieCut)))) {
    job = 2 * is + (residual ? 1 : 0);
    if (tid == 0) A.race_zn[r] = rs.zn;
    sample = -1;
  } else {
    const void* row = (const char*)A.logits + (size_t)is * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
    auto race = [&](const RowRec& rx, bool resid) {
      int smp = -2;
      if (rx.mode == kModeAll || (rx.mode == kModeRange && (rx.flags & kRecTieCut)))
        smp = stream_race_all<DT>(row, V, rx.m, rx.zn, rx.mode == kModeRange ? rx.bkey : 0u,
                                  rx.mode == kModeRange ? rx.tie_cut : 0x7FFFFFFF, T, qrow, resid,
                                  A.seed, rid, pos, sh);
      if (smp == -2) smp = stream_race<DT>(row, V, rx, T, qrow, resid, A.seed, rid, pos, sh);
      return smp;
    };
    sample = race(rs, residual);
    if (residual && sample < 0) {
      resid_empty = true;
      sample = race(rr, false);
    }
  }
  for (int j = tid; j < nr; j += kBlock) {
    const int i = s + j;
    A.out_tokens[i] = j < tau ? A.draft_tokens[i] : (j == tau ? sample : -1);
    if (A.row_flags) {
      uint8_t f = 0;
      if (j < G && accept_uniform(A.seed, rid, pos0 + (uint32_t)j) < bw[2 * (size_t)(i + 1) + 1])
        f |= 1;
      if (j == tau) f |= 2;
      if (j == tau && resid_empty) f |= 32;
      A.row_flags[i] = f;
    }
  }
  if (tid == 0) {
    A.accept_len[r] = tau;
    A.next_token[r] = sample;
    if (A.race_segs > 0) A.race_job[r] = job;
  }
}

// ------------------------------------------------------- finalize kernel
template <int DT, bool BLK>
__device__ __forceinline__ void finalize(const VerifyArgs& A, RowShared& sh) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  if (A.check && *A.check != 0) {
    // refused call: every request emits nothing; the rows are cleared in
    // even shares per workgroup (qo_indptr is not trusted)
    if (tid == 0) {
      A.accept_len[r] = 0;
      A.next_token[r] = -1;
      if (A.race_segs > 0) A.race_job[r] = -1;
    }
    const int R = A.num_requests;
    const int share = (A.num_rows + R - 1) / R;
    const int lo = r * share;
    const int hi = lo + share < A.num_rows ? lo + share : A.num_rows;
    for (int i = lo + tid; i < hi; i += kBlock) {
      A.out_tokens[i] = -1;
      if (A.row_flags) A.row_flags[i] = 0;
    }
    return;
  }
  const int s = A.qo[r], e = A.qo[r + 1];
  const int nr = e - s;
  if (nr <= 0) {
    if (tid == 0) {
      A.accept_len[r] = 0;
      A.next_token[r] = -1;
      if (A.race_segs > 0) A.race_job[r] = -1;
    }
    return;
  }
  const int gamma = nr - 1;
  int cap_eff = gamma;
  if (A.verify_cap) {
    int cv = A.verify_cap[r];
    cap_eff = cv < 0 ? 0 : (cv > gamma ? gamma : cv);
  }
  // block verification (its own kernel instantiation) for sampled requests
  const bool blk = BLK && A.temperature && A.temperature[r] > 0.0f;
  // fast path: every record read in one round by wave 0; taken when no row
  // is pending and the emit row's token is already known
  if (nr <= 64 && !blk) {
    if (wave_id() == 0) {
      const int j = lane_id();
      const bool in = j < nr;
      const RowRec rj = in ? A.rec[s + j] : RowRec{};
      const int dj = in ? A.draft_tokens[s + j] : -1;
      const bool pend = __ballot(in && j <= cap_eff && rj.mode == kModePending) != 0;
      const uint64_t mk = __ballot(j < cap_eff && !(rj.flags & kRecAccept));
      const int L = mk ? __ffsll((unsigned long long)mk) - 1 : cap_eff;
      const int fl = __shfl(rj.flags, L, 64);
      const int md = __shfl(rj.mode, L, 64);
      const int smp = __shfl((fl & kRecSampled) ? rj.sample : rj.a, L, 64);
      const bool fast = !pend && ((fl & kRecSampled) || md == kModeGreedy);
      if (fast) {
        const bool empty = (fl & kRecSampled) && (fl & kRecResidEmpty);
        if (in) {
          A.out_tokens[s + j] = j < L ? dj : (j == L ? smp : -1);
          if (A.row_flags) {
            uint8_t f = 0;
            if (j < cap_eff && (rj.flags & kRecAccept)) f |= 1;
            if (j == L) f |= 2;
            if (j == L && empty) f |= 32;
            A.row_flags[s + j] = f;
          }
        }
        if (j == 0) {
          A.accept_len[r] = L;
          A.next_token[r] = smp;
        }
      }
      if (j == 0) {
        sh.sel_exact = fast ? 1 : 0;
        if (fast && A.race_segs > 0) A.race_job[r] = -1;
      }
    }
    __syncthreads();
    if (sh.sel_exact) return;
  }
  // rows of this request the streaming pass left to the exact path
  for (int j = 0; j <= cap_eff; ++j) {
    if (A.rec[s + j].mode == kModePending)
      resolve_pending<DT>(A, s + j, r, j, j < cap_eff, j == cap_eff, sh);
  }
  if constexpr (BLK) {
    if (blk) {
      block_finalize<DT>(A, sh, r, s, nr, cap_eff);
      return;
    }
  }
  // accepted prefix: first row j < cap_eff whose test rejected (wave 0 ballots)
  if (wave_id() == 0) {
    int L = cap_eff;
    for (int j0 = 0; j0 < cap_eff; j0 += 64) {
      const int j = j0 + lane_id();
      const bool rej = j < cap_eff && !(A.rec[s + j].flags & kRecAccept);
      const uint64_t mk = __ballot(rej);
      if (mk) {
        L = j0 + __ffsll((unsigned long long)mk) - 1;
        break;
      }
    }
    if (lane_id() == 0) sh.found = L;
  }
  __syncthreads();
  const int L = sh.found;
  const int is = s + L;
  const RowRec rr = A.rec[is];
  const bool rejected = L < cap_eff;
  const bool bad = rejected && (rr.flags & kRecBadDraft);
  const float T = A.temperature ? A.temperature[r] : 0.0f;
  const uint32_t rid = A.request_id ? A.request_id[r] : (uint32_t)r;
  const uint32_t pos = (A.position0 ? A.position0[r] : 0u) + (uint32_t)L;
  int sample;
  bool resid_empty = false;
  int job = -1;  // a full-vocabulary race left to the split race kernels
  if (rr.mode == kModeGreedy) {
    sample = rr.a;
  } else {
    const void* row = (const char*)A.logits + (size_t)is * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
    const float* qrow = A.draft_probs ? A.draft_probs + (size_t)is * (size_t)A.ld_q : nullptr;
    const bool residual = rejected && !bad;
    if (rr.mode == kModeList) {
      const ListEntry* Lst = A.list + (size_t)is * kListCap;
      sample = list_race(Lst, rr, T, qrow, residual, A.seed, rid, pos, sh);
      if (residual && sample < 0) {
        resid_empty = true;
        sample = list_race(Lst, rr, T, qrow, false, A.seed, rid, pos, sh);
      }
    } else if (A.race_segs > 0 &&
               (rr.mode == kModeAll || (rr.mode == kModeRange && (rr.flags & kRecTieCut)))) {
      job = 2 * is + (residual ? 1 : 0);
      if (tid == 0) A.race_zn[r] = rr.zn;
      sample = -1;
    } else {
      auto race = [&](bool resid) {
        int smp = -2;
        if (rr.mode == kModeAll || (rr.mode == kModeRange && (rr.flags & kRecTieCut)))
          smp = stream_race_all<DT>(row, A.vocab, rr.m, rr.zn,
                                    rr.mode == kModeRange ? rr.bkey : 0u,
                                    rr.mode == kModeRange ? rr.tie_cut : 0x7FFFFFFF, T, qrow,
                                    resid, A.seed, rid, pos, sh);
        if (smp == -2)
          smp = stream_race<DT>(row, A.vocab, rr, T, qrow, resid, A.seed, rid, pos, sh);
        return smp;
      };
      sample = race(residual);
      if (residual && sample < 0) {
        resid_empty = true;
        sample = race(false);
      }
    }
  }
  for (int j = tid; j < nr; j += kBlock) {
    const int i = s + j;
    A.out_tokens[i] = j < L ? A.draft_tokens[i] : (j == L ? sample : -1);
    if (A.row_flags) {
      uint8_t f = 0;
      if (j < cap_eff && (A.rec[i].flags & kRecAccept)) f |= 1;
      if (j == L) f |= 2;
      if (j == L && resid_empty) f |= 32;
      A.row_flags[i] = f;
    }
  }
  if (tid == 0) {
    A.accept_len[r] = L;
    A.next_token[r] = sample;
    if (A.race_segs > 0) A.race_job[r] = job;
  }
}

__global__ __launch_bounds__(kBlock) void finalize_kernel(VerifyArgs A) {
  __shared__ RowShared sh;
  if (A.dtype == 1) finalize<1, false>(A, sh);
  else finalize<0, false>(A, sh);
}

__global__ __launch_bounds__(kBlock) void finalize_block_kernel(VerifyArgs A) {
  __shared__ RowShared sh;
  if (A.dtype == 1) finalize<1, true>(A, sh);
  else finalize<0, true>(A, sh);
}

// Grid-stride over the (request, segment) items of the requests that have a
// race: every workgroup first lists those requests in LDS (in request order),
// so the items spread evenly over the grid.  With more requests than the list
// holds it strides over every item instead, skipping those without a race.
constexpr int kRaceJobList = 2048;

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void race_segment_kernel(VerifyArgs A) {
  __shared__ RowShared sh;
  __shared__ int jobs[kRaceJobList];
  const int R = A.num_requests;
  const bool listed = R <= kRaceJobList;
  int nj = 0;
  if (listed) {
    for (int base = 0; base < R; base += kBlock) {
      const int r = base + (int)threadIdx.x;
      const int has = (r < R && A.race_job[r] >= 0) ? 1 : 0;
      int total;
      const int off = block_exclusive_sum(has, sh.iscr, &total);
      if (has) jobs[nj + off] = r;
      nj += total;
    }
    __syncthreads();
  }
  // segments per race: with the jobs counted, as many as keep every
  // workgroup at two items at most (segments of 1024 elements at least);
  // otherwise the size-based count
  int S = A.race_segs;
  if (listed && nj > 0) {
    const int by_grid = 2 * (int)gridDim.x / nj;
    const int by_size = (A.vocab + 1023) / 1024;
    const int hi = by_size < kMaxRaceSegs ? by_size : kMaxRaceSegs;
    S = by_grid < 2 ? 2 : (by_grid > hi ? hi : by_grid);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *A.race_nseg = S;
  const int items = (listed ? nj : R) * S;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int j = it / S;
    const int r = listed ? jobs[j] : j;
    if (!listed && A.race_job[r] < 0) continue;
    if (A.dtype == 1) race_segment<1>(A, r, it - j * S, S, sh);
    else race_segment<0>(A, r, it - j * S, S, sh);
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBlock) void race_finish_kernel(VerifyArgs A) {
  __shared__ RowShared sh;
  if (A.dtype == 1) race_finish<1>(A, sh);
  else race_finish<0>(A, sh);
}

// ---------------------------------------------------- build outputs kernel
template <int DT>
__device__ __forceinline__ void build_out(const VerifyArgs& A, const BuildOutArgs& B, RowShared& sh) {
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int V = A.vocab;
  if (A.check && *A.check != 0) {
    // refused call: per-row outputs marked invalid, probabilities untouched
    if (tid == 0) {
      if (B.row_max) B.row_max[i] = __builtin_nanf("");
      if (B.row_argmax) B.row_argmax[i] = -1;
      if (B.row_lse) B.row_lse[i] = __builtin_nanf("");
      if (B.kept_count) B.kept_count[i] = -1;
    }
    if (B.kept_idx)
      for (int t = tid; t < B.kmax; t += kBlock) B.kept_idx[(size_t)i * B.kmax + t] = -1;
    return;
  }
  const int r = row_to_request(A.qo, A.num_requests, A.num_rows, i);
  if (A.rec[i].mode == kModePending) resolve_pending<DT>(A, i, r, i - A.qo[r], false, false, sh);
  const RowRec rr = A.rec[i];
  const float T = A.temperature ? A.temperature[r] : 0.0f;
  const void* row = (const char*)A.logits + (size_t)i * (size_t)A.ld_logits * (DT == 1 ? 2 : 4);
  if (tid == 0) {
    if (B.row_max) B.row_max[i] = rr.m;
    if (B.row_argmax) B.row_argmax[i] = rr.a;
    if (B.row_lse) B.row_lse[i] = rr.lse;
    if (B.kept_count) B.kept_count[i] = rr.nkeep;
  }
  // kept ids in order
  if (B.kept_idx && B.kmax > 0) {
    int32_t* out = B.kept_idx + (size_t)i * B.kmax;
    const int nk = rr.nkeep < B.kmax ? rr.nkeep : B.kmax;
    if (rr.mode == kModeGreedy) {
      for (int t = tid; t < B.kmax; t += kBlock) out[t] = t == 0 ? rr.a : -1;
    } else if (rr.mode == kModeList) {
      const ListEntry* L = A.list + (size_t)i * kListCap;
      for (int t = tid; t < B.kmax; t += kBlock) out[t] = t < nk ? L[t].idx : -1;
    } else {
      // the first nk kept ids are the best nk of the row: find the count
      // boundary exactly, then collect the elements at or above it in id order
      uint32_t bkey = 0u;
      int nb = 0x7FFFFFFF;
      if (nk < V) {
        ExactOut eo;
        exact_kept_set<DT>(row, V, rr.m, T, nk, 1.0f, -1, 0.0f, sh, eo);
        bkey = eo.bkey;
        nb = eo.nb;
      }
      if (tid == 0) sh.count = 0;
      __syncthreads();
      for_each_element_ranked<DT>(
          row, V, [&](float x) { return fkey(x) == bkey; },
          [&](float x, int v, int rank) {
            const uint32_t key = fkey(x);
            if (key > bkey || (key == bkey && rank < nb)) {
              const int slot = atomicAdd(&sh.count, 1);
              if (slot < kCap) sh.buf[slot] = make_entry(x, v);
            }
          },
          sh);
      __syncthreads();
      int n = sh.count < kCap ? sh.count : kCap;
      __syncthreads();
      sort_desc(sh, n);
      for (int t = tid; t < B.kmax; t += kBlock) out[t] = t < nk && t < n ? entry_idx(sh.buf[t]) : -1;
      __syncthreads();
    }
  }
  // dense probabilities
  if (B.probs) {
    float* prow = B.probs + (size_t)i * (size_t)B.ld_probs;
    const double Td = T;
    if (rr.mode == kModeGreedy) {
      for (int v = tid; v < V; v += kBlock) prow[v] = v == rr.a ? 1.0f : 0.0f;
    } else if (rr.mode == kModeList) {
      for (int v = tid; v < V; v += kBlock) prow[v] = 0.0f;
      __syncthreads();
      const ListEntry* L = A.list + (size_t)i * kListCap;
      for (int t = tid; t < rr.nkeep; t += kBlock) {
        const ListEntry le = L[t];
        prow[le.idx] = (float)(exp(((double)le.x - (double)rr.m) / Td) / rr.zn);
      }
    } else if (rr.mode == kModeAll) {
      for_each_element<DT>(row, V, [&](float x, int v) {
        prow[v] = (float)(exp(((double)x - (double)rr.m) / Td) / rr.zn);
      });
    } else {
      const uint32_t bkey = rr.bkey;
      const int nb = rr.nb;
      for_each_element_ranked<DT>(
          row, V, [&](float x) { return fkey(x) == bkey; },
          [&](float x, int v, int rank) {
            const uint32_t key = fkey(x);
            const bool in = key > bkey || (key == bkey && rank < nb);
            prow[v] = in ? (float)(exp(((double)x - (double)rr.m) / Td) / rr.zn) : 0.0f;
          },
          sh);
    }
  }
}

__global__ __launch_bounds__(kBlock) void build_out_kernel(VerifyArgs A, BuildOutArgs B) {
  __shared__ RowShared sh;
  if (A.dtype == 1) build_out<1>(A, B, sh);
  else build_out<0>(A, B, sh);
}

// ------------------------------------------------------ layout check
// qo_indptr against the packing contract: qo[0] = 0 (bit 1), non-decreasing
// (bit 2), qo[R] = rows (bit 4).  One workgroup strides over the requests and
// reads qo[0..R] only, so any contents are safe to check.
__global__ __launch_bounds__(1024) void check_layout_kernel(const int32_t* qo, int32_t R,
                                                            int32_t rows, int32_t* word) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int mine = 0;
  for (int r = threadIdx.x; r < R; r += blockDim.x)
    if (qo[r + 1] < qo[r]) mine = 2;
  if (threadIdx.x == 0) {
    if (qo[0] != 0) mine |= 1;
    if (qo[R] != rows) mine |= 4;
  }
  if (mine) atomicOr(&bad, mine);
  __syncthreads();
  if (threadIdx.x == 0) *word = bad;
}

// ------------------------------------------------------ row diagnostics
// The decision quantities the last call recorded per row: Z_K, Z_N (masses
// relative to exp(m / T)), p(d) of a tested draft, and the row mode.
__global__ __launch_bounds__(256) void diagnostics_kernel(const RowRec* rec, int32_t rows,
                                                          double* zk, double* zn, double* pd,
                                                          int32_t* mode) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += gridDim.x * blockDim.x) {
    const RowRec r = rec[i];
    if (zk) zk[i] = r.zk;
    if (zn) zn[i] = r.zn;
    if (pd) pd[i] = r.pd;
    if (mode) mode[i] = r.mode;
  }
}

}  // namespace sv
