// sv_rowpass.hpp -- one workgroup per logits row: a single coalesced streaming
// pass over the row with per-wave candidate buffers, the block-level merge and
// selections that follow it, and row iterators for the later passes.
//
// Streaming pass.  Each thread loads 16-byte vectors (8 bf16 or 4 fp32).  For
// a fixed wave the element ids it sees increase from tile to tile, so every
// element a wave sees after one of its tile boundaries has a larger id than
// every element it saw before.  Per element the pass keeps a running max (and,
// when needed, the first index reaching it and an exp-sum at the row's
// temperature).  Rows that need a top-k or top-p set also keep, in the wave's
// own LDS segment, every element better in (value desc, id asc) order than the
// wave's threshold entry theta_w; when the segment passes a limit a wave-local
// radix select over the 64-bit entries keeps the best `keep` and raises
// theta_w.  An element equal in value to theta_w comes later and so never
// beats it: the filter is one strict float compare, done on the chunk max in
// the common case.  Nothing in the streaming loop synchronises the block.
// Each segment holds the best |segment| elements its wave has seen, so the
// union of the segments holds every element of the row that is at least as
// good as max_w theta_w (the certified prefix), and the top-k of the row for
// any k <= keep.
#pragma once

#include <type_traits>

#include "sv_device.hpp"

namespace sv {

constexpr int kWaveCap = kCap / kWaves;   // entries per wave segment
// Vector-candidate rows: per wave, kVecCap entries followed by their raw
// 16-byte vectors, in a region of kVecStride entries.
constexpr int kVecCap = 256;
constexpr int kVecDatOff = kVecCap;
constexpr int kVecStride = kVecCap + 2 * kVecCap;
static_assert(kWaves * kVecStride <= kCap, "vector segments fit the buffer");
static_assert(kThreshVec < kVecCap, "room for a tile of appends");

struct RowShared {
  uint64_t buf[kCap];               // wave segments while streaming; merged area after
  uint32_t whist[kWaves][256];      // per-wave radix histograms; whist[0] at block level
  uint64_t mhist[256];              // fixed-point masses of the block-level mass walk
  double dscr[kWaves];
  uint64_t uscr[kWaves];
  float fscr[kWaves];
  int iscr[kWaves];
  int wcount[kWaves];               // final entries per wave segment
  float wtau[kWaves];               // wave thresholds (published while streaming, final after)
  float endx[16];                   // vector-candidate rows: head (0..7) and tail (8..15) elements
  int woverflow;
  int count;
  int sel_digit, sel_need, sel_exact, found;
  uint64_t sel_entry;
  double zn_shared;
};

// -------------------------------------------------------------- wave sync
// Order the wave's LDS accesses: its lanes run in lockstep, so completing the
// outstanding LDS operations is all another lane of the same wave needs.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------ radix selections
// Digit of 256 bins (scanned from the top by one wave, lane l owning digits
// 255-4l .. 252-4l) where the running count reaches `need`.  Returns the
// digit, the entries still needed inside it and whether it holds exactly them.
__device__ __forceinline__ void wave_pick_digit(const uint32_t* hist, int need, int& digit,
                                                int& rem, bool& exact) {
  const int l = lane_id();
  const int h0 = (int)hist[255 - 4 * l], h1 = (int)hist[254 - 4 * l];
  const int h2 = (int)hist[253 - 4 * l], h3 = (int)hist[252 - 4 * l];
  const int local = h0 + h1 + h2 + h3;
  const int incl = wave_inclusive_sum(local);
  const int excl = incl - local;
  const uint64_t m = __ballot(excl < need && need <= incl);
  const int src = m ? __ffsll((unsigned long long)m) - 1 : 63;
  int c = excl, d, hd;
  if (c + h0 >= need) { d = 255 - 4 * l; hd = h0; }
  else if ((c += h0) + h1 >= need) { d = 254 - 4 * l; hd = h1; }
  else if ((c += h1) + h2 >= need) { d = 253 - 4 * l; hd = h2; }
  else { c += h2; d = 252 - 4 * l; hd = h3; }
  digit = __shfl(d, src, 64);
  rem = __shfl(need - c, src, 64);
  exact = __shfl(hd == need - c ? 1 : 0, src, 64) != 0;
}

// Wave-local: the `keep` best of seg[0, n) (n > keep), compacted in place to
// seg[0, keep), moving dat[] along when given.  Returns the worst kept entry.
// Only this wave takes part.
__device__ __forceinline__ uint64_t wave_compact(uint64_t* seg, uint32_t* hist, int n, int keep,
                                                 uint4* dat = nullptr) {
  const int l = lane_id();
  uint64_t prefix = 0, pmask = 0;
  int need = keep;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[l * 4 + b] = 0u;
    wave_lds_sync();
    for (int e = l; e < n; e += 64) {
      const uint64_t v = seg[e];
      if ((v & pmask) == prefix) atomicAdd(&hist[(uint32_t)(v >> shift) & 255u], 1u);
    }
    wave_lds_sync();
    int d, rem;
    bool exact;
    wave_pick_digit(hist, need, d, rem, exact);
    need = rem;
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)0xFF << shift;
    wave_lds_sync();
    if (exact) break;
  }
  // in place, 64 entries per round: round s writes below 64(s+1)
  uint64_t mn = ~0ull;
  int pos0 = 0;
  for (int b0 = 0; b0 < n; b0 += 64) {
    const int e = b0 + l;
    const uint64_t v = e < n ? seg[e] : 0ull;
    const bool k = e < n && (v & pmask) >= prefix;
    uint4 dv = make_uint4(0u, 0u, 0u, 0u);
    if (dat && k) dv = dat[e];
    const uint64_t km = __ballot(k);
    const int off = __popcll(km & ((1ull << l) - 1ull));
    wave_lds_sync();
    if (k) {
      seg[pos0 + off] = v;
      if (dat) dat[pos0 + off] = dv;
      mn = v < mn ? v : mn;
    }
    pos0 += __popcll(km);
    wave_lds_sync();
  }
  return wave_min_u64(mn);
}

// Block level: radix select over buf[0, n): (prefix, pmask) such that exactly
// `keep` entries satisfy (e & pmask) >= prefix.  keep < n.
__device__ __forceinline__ void radix_select_top(RowShared& sh, int n, int keep, uint64_t& prefix,
                                                 uint64_t& pmask) {
  prefix = 0;
  pmask = 0;
  int need = keep;
  uint32_t* hist = sh.whist[0];
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += kBlock) hist[b] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kBlock) {
      const uint64_t v = sh.buf[e];
      if ((v & pmask) == prefix) atomicAdd(&hist[(uint32_t)(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave_id() == 0) {
      int d, rem;
      bool exact;
      wave_pick_digit(hist, need, d, rem, exact);
      if (lane_id() == 0) {
        sh.sel_digit = d;
        sh.sel_need = rem;
        sh.sel_exact = exact ? 1 : 0;
      }
    }
    __syncthreads();
    const int d = sh.sel_digit;
    need = sh.sel_need;
    const int exact = sh.sel_exact;
    prefix |= (uint64_t)d << shift;
    pmask |= (uint64_t)0xFF << shift;
    if (exact) break;
  }
}

// Block level: keep the `keep` best of buf[0, n) (n > keep) in buf[0, keep).
__device__ __forceinline__ void compact_top(RowShared& sh, int n, int keep) {
  uint64_t prefix, pmask;
  radix_select_top(sh, n, keep, prefix, pmask);
  int pos0 = 0;
  for (int b0 = 0; b0 < n; b0 += kBlock) {
    const int e = b0 + threadIdx.x;
    const uint64_t v = e < n ? sh.buf[e] : 0ull;
    const bool k = e < n && (v & pmask) >= prefix;
    int total;
    const int pos = block_exclusive_sum(k ? 1 : 0, sh.iscr, &total);  // barriers: reads done
    if (k) sh.buf[pos0 + pos] = v;
    pos0 += total;
  }
  if (threadIdx.x == 0) sh.count = keep;
  __syncthreads();
}

// Sort buf[0, n) descending (n <= kCap): rank counting for n <= kBlock,
// bitonic network otherwise.
__device__ __forceinline__ void sort_desc(RowShared& sh, int n) {
  if (n <= 1) return;
  if (n <= kBlock) {
    const int t = threadIdx.x;
    const uint64_t v = t < n ? sh.buf[t] : 0ull;
    int rank = 0;
    if (t < n)
      for (int u = 0; u < n; ++u) rank += sh.buf[u] > v ? 1 : 0;
    __syncthreads();
    if (t < n) sh.buf[rank] = v;
    __syncthreads();
    return;
  }
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  for (int e = n + threadIdx.x; e < p2; e += kBlock) sh.buf[e] = 0ull;
  __syncthreads();
  for (int k = 2; k <= p2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (p2 >> 1); i += kBlock) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo | j;
        const uint64_t a = sh.buf[lo], b = sh.buf[hi];
        const bool desc = (lo & k) == 0;
        if (desc ? (a < b) : (a > b)) {
          sh.buf[lo] = b;
          sh.buf[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Merge the wave segments into buf[0, total) (block level).  Round s moves
// merged entries [256s, 256s+256); an entry only moves down and no later
// round reads an address a round writes, so one barrier per round suffices.
__device__ __forceinline__ int merge_segments(RowShared& sh) {
  int base[kWaves];
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    base[w] = total;
    total += sh.wcount[w];
  }
  for (int g0 = 0; g0 < total; g0 += kBlock) {
    const int g = g0 + threadIdx.x;
    uint64_t v = 0ull;
    if (g < total) {
      int w = 0;
#pragma unroll
      for (int q = 1; q < kWaves; ++q)
        if (g >= base[q]) w = q;
      v = sh.buf[w * kWaveCap + (g - base[w])];
    }
    __syncthreads();
    if (g < total) sh.buf[g] = v;
  }
  __syncthreads();
  return total;
}

// --------------------------------------------------------- streaming pass
struct StreamAcc {
  float mx;     // running max of this thread's elements (also the sum reference)
  int bi;       // first index reaching mx (ARG)
  float nmc;    // -(mx * c) rounded to fp32: exp2(fma(x, c, nmc)) are the weights
  double corr;  // exp2(-(mx * c + nmc)): corrects the rounding of nmc exactly
  double s;     // sum of weights relative to exp2(mx * c)  (SUM)
};

// Per-wave candidate state.  Invariant: every element the wave has seen and
// not kept has value <= tau, and (when it is finite and the wave kept at least
// `keep` finite entries) `keep` kept entries that are better in (value desc,
// id asc) order.
struct WaveBuf {
  int count;     // entries in the wave segment (may pass kWaveCap: overflow)
  float tau;     // own threshold: later elements must be strictly larger
  float tsh;     // best threshold published by any wave, non-strict (-inf: none)
  int keep, thresh;
  bool share;    // publish and read thresholds across the block's waves
};

template <int DT>
struct Vec;
template <>
struct Vec<1> {  // bf16
  static constexpr int kEpv = 8;
  static constexpr int kEsz = 2;
  __device__ static __forceinline__ void unpack(const uint4& v, float* x) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ float load1(const void* p, long i) {
    return __uint_as_float((uint32_t)__ldg((const unsigned short*)p + i) << 16);
  }
};
template <>
struct Vec<0> {  // fp32
  static constexpr int kEpv = 4;
  static constexpr int kEsz = 4;
  __device__ static __forceinline__ void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float load1(const void* p, long i) {
    return __ldg((const float*)p + i);
  }
};

// Split of a row into a scalar head (to 16-byte alignment), a body of 16-byte
// vectors and a scalar tail.
template <int DT>
struct RowSplit {
  const uint4* vbase;
  int head, nvec, tail0;
  __device__ RowSplit(const void* row, int V) {
    constexpr int E = Vec<DT>::kEsz, P = Vec<DT>::kEpv;
    const uintptr_t addr = (uintptr_t)row;
    int h = (int)(((16u - (uint32_t)(addr & 15u)) & 15u) / E);
    head = h < V ? h : V;
    nvec = (V - head) / P;
    tail0 = head + nvec * P;
    vbase = (const uint4*)((const char*)row + (size_t)head * E);
  }
};

__device__ __forceinline__ void set_reference(StreamAcc& a, float mx, float c) {
  a.mx = mx;
  a.nmc = -(mx * c);
  const float err = fmaf(mx, c, a.nmc);  // mx*c + nmc, exact
  a.corr = exp2(-(double)err);
}

// Maximum that propagates NaN (one v_maximum3 per two inputs, no operand
// canonicalisation).  Logits are finite or -inf; a NaN only blinds the
// vector it sits in.
__device__ __forceinline__ float maxm(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
template <int P>
__device__ __forceinline__ float vec_max(const float* x) {
  if constexpr (P == 1) return x[0];
  else if constexpr (P == 4) return maxm(maxm(maxm(x[0], x[1]), x[2]), x[3]);
  else {
    float m = maxm(maxm(x[0], x[1]), x[2]);
    m = maxm(maxm(m, x[3]), x[4]);
    m = maxm(maxm(m, x[5]), x[6]);
    return maxm(m, x[7]);
  }
}
template <int P>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (P == 1) return x[0];
  else if constexpr (P == 4) return (x[0] + x[1]) + (x[2] + x[3]);
  else return tree_sum<4>(x) + tree_sum<4>(x + 4);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// k-th largest of the keys a and b of every lane (absent keys are 0), or 0
// when fewer than k keys are nonzero: a radix select two bits at a time with
// three independent ballot counts per step, from the top bit down to bit
// `lo`.  Keys of bf16 values pass lo = 16: their low 16 bits follow from the
// sign bit (0 for a positive value, all ones for a negative one), so key
// order is the order of the high halves.
__device__ __forceinline__ uint32_t wave_kth_key(uint32_t a, uint32_t b, int k, int lo) {
  uint32_t t = 0u;
  for (int bit = 30; bit >= lo; bit -= 2) {
    const uint32_t c1 = t | (1u << bit), c2 = t | (2u << bit), c3 = t | (3u << bit);
    const int n3 = __popcll(__ballot(a >= c3)) + __popcll(__ballot(b >= c3));
    const int n2 = __popcll(__ballot(a >= c2)) + __popcll(__ballot(b >= c2));
    const int n1 = __popcll(__ballot(a >= c1)) + __popcll(__ballot(b >= c1));
    t = n3 >= k ? c3 : (n2 >= k ? c2 : (n1 >= k ? c1 : t));
  }
  if (lo == 16 && t != 0u && !(t & 0x80000000u)) t |= 0xFFFFu;
  return t;
}

// Largest lane key k such that at least `keep` lanes (keep <= 64) hold a key
// >= k: those lanes' entries are `keep` entries at least as good as k.
__device__ __forceinline__ uint32_t wave_kth_lane_key(uint32_t lk, int keep) {
  return wave_kth_key(lk, 0u, keep, 0);
}

// As wave_kth_lane_key over two keys per lane (best b1, second b2; 0 when
// absent), for keep <= 128.
__device__ __forceinline__ uint32_t wave_kth_lane_key2(uint32_t b1, uint32_t b2, int keep) {
  return wave_kth_key(b1, b2, keep, 0);
}

// Threshold key for `keep` <= 64 from per-lane best and second-best keys.
__device__ __forceinline__ uint32_t wave_threshold_key(uint32_t b1, uint32_t b2, int keep) {
  return keep <= 32 ? wave_kth_lane_key(b1, keep) : wave_kth_lane_key2(b1, b2, keep);
}

// k-th largest of one key per lane (lanes with ok == false hold none); 0
// when fewer than k keys are held.
__device__ __forceinline__ uint32_t wave_kth_key_ballot(uint32_t key, bool ok, int k) {
  return wave_kth_key(ok ? key : 0u, 0u, k, 0);
}

// A key t such that lo <= #(entries of seg[0, n) with key >= t) <= hi,
// estimated from a 64-entry sample and checked by one counting pass (a few
// attempts); 0 when none was found.  Wave-local, n >= hi.
__device__ __forceinline__ uint32_t wave_sample_threshold(const uint64_t* seg, int n, int lo,
                                                          int hi) {
  const int l = lane_id();
  const uint32_t smp = (uint32_t)(seg[(int)(((long long)l * n) >> 6)] >> 32);
  int target = (lo + hi) >> 1;
#pragma unroll 1
  for (int att = 0; att < 4; ++att) {
    int rnk = (int)(((long long)target * 64 + n - 1) / n);
    rnk = rnk < 1 ? 1 : (rnk > 64 ? 64 : rnk);
    const uint32_t t = wave_kth_key_ballot(smp, true, rnk);
    int cnt = 0;
    for (int e0 = 0; e0 < n; e0 += 64) {
      const int e = e0 + l;
      cnt += __popcll(__ballot(e < n && (uint32_t)(seg[e] >> 32) >= t));
    }
    if (cnt >= lo && cnt <= hi) return t;
    // move the target the other way by the observed miss
    target = cnt < lo ? target + (lo - cnt) + (hi - lo) / 4 : target - (cnt - hi) - (hi - lo) / 4;
    if (target < 1) target = 1;
  }
  return 0u;
}

// Keep the entries of seg[0, n) whose key is >= kmin, in place (wave-local),
// moving the companion array along when given; returns how many remain.
template <class D = uint4>
__device__ __forceinline__ int wave_keep_ge(uint64_t* seg, int n, uint32_t kmin,
                                            D* dat = nullptr) {
  const int l = lane_id();
  int pos0 = 0;
  for (int b0 = 0; b0 < n; b0 += 64) {
    const int e = b0 + l;
    const uint64_t v = e < n ? seg[e] : 0ull;
    const bool k = e < n && (uint32_t)(v >> 32) >= kmin;
    D dv{};
    if (dat && k) dv = dat[e];
    const uint64_t km = __ballot(k);
    wave_lds_sync();
    if (k) {  // never above e: reads of later rounds intact
      seg[pos0 + lanes_below(km)] = v;
      if (dat) dat[pos0 + lanes_below(km)] = dv;
    }
    pos0 += __popcll(km);
    wave_lds_sync();
  }
  return pos0;
}

// Append the elements of one vector that beat both thresholds (wave-uniform
// call).  Element e has id id0 + e; positions in the segment follow (e, lane)
// order, which nothing downstream relies on.
template <int P>
__device__ __forceinline__ void wave_append(const float* x, int id0, WaveBuf& wb, uint64_t* seg) {
  int base = wb.count;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const bool pass = x[e] > wb.tau && x[e] >= wb.tsh;
    const uint64_t m = __ballot(pass);
    if (pass) {
      const int slot = base + lanes_below(m);
      if (slot < kWaveCap) seg[slot] = make_entry(x[e], id0 + e);
    }
    base += __popcll(m);
  }
  wb.count = base;
}

// Wave tile boundary: shrink the segment once it passed its limit, raising
// tau.  For keep <= 64 the new tau is the largest key that `keep` lane
// maxima reach (cheap, keeps a few more than `keep`); otherwise, or when that
// leaves too many, a radix select keeps exactly `keep`.  Either way every
// dropped entry has `keep` better ones left.  An overflowed segment stops
// admitting (the row then takes the exact path).  With sharing on, a wave
// also filters by the best threshold any wave has published (non-strict: ids
// interleave across waves); stale reads only lower that filter.
__device__ __forceinline__ void wave_tile_end(WaveBuf& wb, uint64_t* seg, uint32_t* hist,
                                              RowShared& sh) {
  if (wb.count > kWaveCap) {
    wb.tau = __builtin_huge_valf();  // overflowed: admit nothing more
  } else if (wb.count > wb.thresh) {
    wave_lds_sync();
    int n = wb.count;
    if (wb.keep <= 64) {
      uint32_t b1 = 0u, b2 = 0u;  // this lane's best two keys of its column
      for (int e = lane_id(); e < n; e += 64) {
        const uint32_t k = (uint32_t)(seg[e] >> 32);
        if (k > b1) { b2 = b1; b1 = k; } else if (k > b2) { b2 = k; }
      }
      const uint32_t tk = wave_threshold_key(b1, b2, wb.keep);
      if (tk != 0u) {  // 0: fewer than `keep` entries (not reached while n > thresh >= keep)
        n = wave_keep_ge(seg, n, tk);
        wb.tau = key_to_float(tk);
      }
    }
    if (n > wb.thresh) {
      const uint64_t th = wave_compact(seg, hist, n, wb.keep);
      n = wb.keep;
      wb.tau = entry_val(th);
    }
    wb.count = n;
    if (wb.share && lane_id() == 0) sh.wtau[wave_id()] = wb.tau;
    wave_lds_sync();
  }
  if (wb.share) {
    float t = sh.wtau[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) t = fmaxf(t, sh.wtau[q]);
    wb.tsh = t;
  }
}

// Running max, first argmax and exp-sum over a tile of U vectors of P
// elements (masked elements are -inf).  The max and the sum reference move
// at most once per tile.
template <bool SUM, bool ARG, int U, int P>
__device__ __forceinline__ void tile_stats(const float* x, const int* ids, float cm, float c,
                                           StreamAcc& a) {
  if (cm > a.mx) {  // rare after the first tiles
    if (ARG) {
      int first = 0x7FFFFFFF;
#pragma unroll
      for (int u = U - 1; u >= 0; --u)
#pragma unroll
        for (int e = P - 1; e >= 0; --e)
          if (x[u * P + e] == cm) first = ids[u] + e;
      a.bi = first;
    }
    if (SUM) {
      a.s *= exp2((double)(a.mx - cm) * (double)c);  // rescale to the new max
      set_reference(a, cm, c);
    } else {
      a.mx = cm;
    }
  }
  if (SUM) {
    float cs = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float w[P];
#pragma unroll
      for (int e = 0; e < P; ++e) w[e] = __builtin_amdgcn_exp2f(fmaf(x[u * P + e], c, a.nmc));
      cs += tree_sum<P>(w);
    }
    a.s += (double)cs * a.corr;
  }
}

// Filter a tile into the wave segment and close the tile.
template <int U, int P>
__device__ __forceinline__ void tile_buffer(const float* x, const float* um, float cm,
                                            const int* ids, WaveBuf& wb, uint64_t* seg,
                                            uint32_t* hist, RowShared& sh) {
  if (__ballot(cm > wb.tau && cm >= wb.tsh)) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (__ballot(um[u] > wb.tau && um[u] >= wb.tsh)) wave_append<P>(x + u * P, ids[u], wb, seg);
    wave_tile_end(wb, seg, hist, sh);
  } else if (wb.share) {
    wave_tile_end(wb, seg, hist, sh);
  }
}

// Vector-candidate variant: entries are (vector max, vector index) with the
// raw vector beside them; a row's top-k elements all lie in its top-k vectors
// under that order, since every vector ahead of one holding a top-k element
// owns a distinct better element.  Same shrinking rule as wave_tile_end
// (keep <= 64), data moving with the entries; capacity kVecCap.
// dat == nullptr: entries only (capacity kWaveCap), for keeps beyond 64 with
// thresholds shared across the block's waves as in wave_tile_end.
__device__ __forceinline__ void wave_tile_end_vec(WaveBuf& wb, uint64_t* seg, uint4* dat,
                                                  uint32_t* hist, RowShared& sh) {
  const int cap = dat ? kVecCap : kWaveCap;
  if (wb.count > cap) {
    wb.tau = __builtin_huge_valf();  // overflowed: admit nothing more
  } else if (wb.count > wb.thresh) {
    wave_lds_sync();
    int n = wb.count;
    if (wb.keep <= 64) {
      uint32_t b1 = 0u, b2 = 0u;
      for (int e = lane_id(); e < n; e += 64) {
        const uint32_t k = (uint32_t)(seg[e] >> 32);
        if (k > b1) { b2 = b1; b1 = k; } else if (k > b2) { b2 = k; }
      }
      const uint32_t tk = wave_threshold_key(b1, b2, wb.keep);
      if (tk != 0u) {
        n = wave_keep_ge(seg, n, tk, dat);
        wb.tau = key_to_float(tk);
      }
    } else {
      // keep between `keep` and halfway to the limit, by a sampled threshold
      const uint32_t tk = wave_sample_threshold(seg, n, wb.keep, (wb.keep + wb.thresh) >> 1);
      if (tk != 0u) {
        n = wave_keep_ge(seg, n, tk, dat);
        wb.tau = key_to_float(tk);
      }
    }
    if (n > wb.thresh) {
      const uint64_t th = wave_compact(seg, hist, n, wb.keep, dat);
      n = wb.keep;
      wb.tau = entry_val(th);
    }
    wb.count = n;
    if (wb.share && lane_id() == 0) sh.wtau[wave_id()] = wb.tau;
    wave_lds_sync();
  }
  if (wb.share) {
    float t = sh.wtau[0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) t = fmaxf(t, sh.wtau[q]);
    wb.tsh = t;
  }
}

// raw(u) gives the u-th vector's 16 bytes (kept or rebuilt from its elements).
template <int U, bool DATA, class Raw>
__device__ __forceinline__ void tile_buffer_vec(Raw&& raw, const float* um, float cm, int vi0,
                                                WaveBuf& wb, uint64_t* seg, uint4* dat,
                                                uint32_t* hist, RowShared& sh) {
  constexpr int cap = DATA ? kVecCap : kWaveCap;
  if (__ballot(cm > wb.tau && cm >= wb.tsh)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool pass = um[u] > wb.tau && um[u] >= wb.tsh;
      const uint64_t m = __ballot(pass);
      if (pass) {
        const int slot = wb.count + lanes_below(m);
        if (slot < cap) {
          seg[slot] = make_entry(um[u], vi0 + u * kBlock);
          if (DATA) dat[slot] = raw(u);
        }
      }
      wb.count += __popcll(m);
    }
    wave_tile_end_vec(wb, seg, DATA ? dat : nullptr, hist, sh);
  } else if (wb.share) {
    wave_tile_end_vec(wb, seg, DATA ? dat : nullptr, hist, sh);
  }
}

// Wave priority from a row's progress.  Waves of older workgroups win the
// CU's instruction arbitration, so rows streamed side by side on one CU would
// finish far apart and leave the CU short of loads in flight at the end; a
// wave's priority instead falls from 3 to 0 as its row advances, which keeps
// the CU's rows level until they end together.
__device__ __forceinline__ void progress_priority(int t, int ntile, int& cur) {
  const int lvl = 3 - (4 * t) / (ntile + 1);
  if (lvl == cur) return;
  cur = lvl;
  switch (lvl) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// Full tiles of U vectors per thread from vector v0 on, two load buffers in
// turn so the next tile is in flight while one is consumed (the scheduling
// barrier keeps the compiler from sinking the loads below the consumer).
// Returns the first vector not consumed.
template <int DT, int U, class F>
__device__ __forceinline__ int stream_tiles(const RowSplit<DT>& sp, int v0, bool level,
                                            F&& consume) {
  const int ntile = (sp.nvec - v0) / (U * kBlock);
  int prio = level ? -1 : 0;
  uint4 A[U], B[U];
  auto ld = [&](uint4* v, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = load_stream(sp.vbase + v0 + (t * U + u) * kBlock + (int)threadIdx.x);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (ntile >= 1) ld(A, 0);
  int t = 0;
  for (; t + 3 <= ntile; t += 2) {
    if (level) progress_priority(t, ntile, prio);
    ld(B, t + 1);
    consume(A, v0 + t * U * kBlock);
    ld(A, t + 2);
    consume(B, v0 + (t + 1) * U * kBlock);
  }
  if (t + 2 == ntile) {
    ld(B, t + 1);
    consume(A, v0 + t * U * kBlock);
    consume(B, v0 + (t + 1) * U * kBlock);
  } else if (t + 1 == ntile) {
    consume(A, v0 + t * U * kBlock);
  }
  if (prio > 0) __builtin_amdgcn_s_setprio(0);
  return v0 + ntile * U * kBlock;
}

// Stream one row.  Element-buffered rows (BUF) keep, per wave, at least the
// best `keep` elements seen (shrinking the segment when it holds more than
// `thresh`), starting with `ramp` smaller tiles and sharing thresholds across
// waves.  Vector-buffered rows (VEC, keep <= 64) keep the best `keep` body
// vectors by their max instead; their first full tile admits only vectors
// that `keep` lanes' best vectors reach.  Head and tail elements are not
// buffered in VEC mode.
template <int DT, bool BUF, bool SUM, bool ARG, int VEC = 0>
__device__ __forceinline__ void stream_row(const void* row, int V, float c, int keep, int thresh,
                                           int ramp, RowShared& sh, StreamAcc& a,
                                           bool level = false) {
  constexpr int P = Vec<DT>::kEpv;
  constexpr int U = SV_UNROLL;
  constexpr float kNegInf = -__builtin_huge_valf();
  constexpr bool VD = VEC == 1;  // vector candidates with their raw bytes (small keep)
  static_assert(!(BUF && VEC), "one buffer kind per row");
  static_assert(!(VD && (SUM || ARG)), "vector candidates with data stream alone");
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  const int w = wave_id();
  uint64_t* seg = sh.buf + w * (VD ? kVecStride : kWaveCap);
  uint4* dat = (uint4*)(sh.buf + w * kVecStride + kVecDatOff);
  uint32_t* hist = sh.whist[w];
  a.bi = 0x7FFFFFFF;
  a.s = 0.0;
  a.mx = -3.402823466e38f;  // below every finite element: weights of -inf are 0
  a.nmc = 0.0f;
  a.corr = 1.0;
  WaveBuf wb;
  wb.count = 0;
  wb.tau = kNegInf;
  wb.tsh = kNegInf;
  wb.keep = keep;
  wb.thresh = thresh;
  wb.share = BUF || VEC == 2;

  // U vectors from vector vb (all in range) -> elements, vector maxima, tile max
  auto unpack = [&](const uint4* v, int vb, float* x, float* um, int* ids) {
    float cm = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Vec<DT>::unpack(v[u], x + u * P);
      um[u] = vec_max<P>(x + u * P);
      cm = maxm(cm, um[u]);
      ids[u] = sp.head + (vb + u * kBlock + tid) * P;
    }
    return cm;
  };
  // scalar pieces (head and tail): one element per thread, -inf when out of range
  auto scalar = [&](int i, bool in, int slot) {
    float x[1] = {in ? Vec<DT>::load1(row, i) : kNegInf};
    int ids[1] = {i};
    tile_stats<SUM, ARG, 1, 1>(x, ids, x[0], c, a);
    if (BUF) tile_buffer<1, 1>(x, x, x[0], ids, wb, seg, hist, sh);
    if (VD && in) sh.endx[slot] = x[0];  // kept aside for the finish
  };
  if (sp.head > 0) scalar(tid, tid < sp.head, tid);

  int v0 = 0;
  if (VD && sp.nvec >= U * kBlock) {
    // first tile: admit vectors whose max reaches the threshold key of the
    // lanes' best two vector maxima
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_stream(sp.vbase + u * kBlock + tid);
    float x[U * P], um[U];
    int ids[U];
    const float cm = unpack(v, 0, x, um, ids);
    tile_stats<SUM, ARG, U, P>(x, ids, cm, c, a);
    uint32_t b1 = 0u, b2 = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = fkey(um[u]);
      if (k > b1) { b2 = b1; b1 = k; } else if (k > b2) { b2 = k; }
    }
    const uint32_t tk = wave_threshold_key(b1, b2, keep);
    const float t0 = tk != 0u ? key_to_float(tk) : kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool pass = um[u] >= t0;
      const uint64_t m = __ballot(pass);
      if (pass) {
        const int slot = wb.count + lanes_below(m);
        if (slot < kVecCap) {
          seg[slot] = make_entry(um[u], u * kBlock + tid);
          dat[slot] = v[u];
        }
      }
      wb.count += __popcll(m);
    }
    wb.tau = t0;  // later vectors with max equal to t0 have larger ids: strict from here
    wave_tile_end_vec(wb, seg, dat, hist, sh);
    v0 = U * kBlock;
  }
  if (VEC == 2 && sp.nvec >= U * kBlock) {
    // first tile of a top-p row: the starting threshold is the key that
    // about 3/2 keep of the wave's vectors reach, estimated from this tile's
    // vector maxima (the wave's 64 U of them); the tile's vectors at or above
    // it are admitted.  A low estimate costs compactions later, a high one
    // only a smaller certified prefix.
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_stream(sp.vbase + u * kBlock + tid);
    float x[U * P], um[U];
    int ids[U];
    const float cm = unpack(v, 0, x, um, ids);
    tile_stats<SUM, ARG, U, P>(x, ids, cm, c, a);
    const long long vpw = sp.nvec / kWaves;  // vectors this wave sees
    long long kr = (64LL * U * (3 * keep / 2) + vpw - 1) / vpw;
    const int k = kr < 1 ? 1 : (kr > 64 * U ? 64 * U : (int)kr);
    uint32_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) key[u] = fkey(um[u]);
    uint32_t tk = 0u;  // k-th largest of the wave's keys, bit by bit
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = tk | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) cnt += __popcll(__ballot(key[u] >= cand));
      if (cnt >= k) tk = cand;
    }
    const float t0 = key_to_float(tk);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool pass = um[u] >= t0;
      const uint64_t m = __ballot(pass);
      if (pass) {
        const int slot = wb.count + lanes_below(m);
        if (slot < kWaveCap) seg[slot] = make_entry(um[u], u * kBlock + tid);
      }
      wb.count += __popcll(m);
    }
    wb.tau = t0;  // later vectors with max equal to t0 have larger ids: strict from here
    if (lane_id() == 0) sh.wtau[w] = t0;
    wave_tile_end_vec(wb, seg, nullptr, hist, sh);
    v0 = U * kBlock;
  }
  if (BUF) {
    // smaller tiles first, so the segment cannot overflow before tau settles
    auto small = [&](auto Ut) {
      constexpr int UU = decltype(Ut)::value;
      uint4 v[UU];
      float x[UU * P], um[UU];
      int ids[UU];
      float cm = kNegInf;
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        v[u] = load_stream(sp.vbase + v0 + u * kBlock + tid);
        Vec<DT>::unpack(v[u], x + u * P);
        um[u] = vec_max<P>(x + u * P);
        cm = maxm(cm, um[u]);
        ids[u] = sp.head + (v0 + u * kBlock + tid) * P;
      }
      tile_stats<SUM, ARG, UU, P>(x, ids, cm, c, a);
      tile_buffer<UU, P>(x, um, cm, ids, wb, seg, hist, sh);
      v0 += UU * kBlock;
    };
    if (v0 + kBlock <= sp.nvec) small(std::integral_constant<int, 1>{});
    if (v0 + kBlock <= sp.nvec) small(std::integral_constant<int, 1>{});
    for (int r = 0; r < ramp; ++r)
      if (v0 + 2 * kBlock <= sp.nvec) small(std::integral_constant<int, 2>{});
  }
  v0 = stream_tiles<DT, U>(sp, v0, level, [&](const uint4* v, int vb) {
    float x[U * P], um[U];
    int ids[U];
    const float cm = unpack(v, vb, x, um, ids);
    tile_stats<SUM, ARG, U, P>(x, ids, cm, c, a);
    if (BUF) tile_buffer<U, P>(x, um, cm, ids, wb, seg, hist, sh);
    if (VEC)
      tile_buffer_vec<U, VD>([&](int u) { return v[u]; }, um, cm, vb + tid, wb, seg, dat, hist,
                             sh);
  });
  // ragged last tiles of the body: vectors [v0, nvec), one per thread
  for (; v0 < sp.nvec; v0 += kBlock) {
    const int vi = v0 + tid;
    float x[P];
    uint4 rv = make_uint4(0u, 0u, 0u, 0u);
    if (vi < sp.nvec) {
      rv = load_stream(sp.vbase + vi);
      Vec<DT>::unpack(rv, x);
    } else {
#pragma unroll
      for (int e = 0; e < P; ++e) x[e] = kNegInf;
    }
    int ids[1] = {sp.head + vi * P};
    const float cm = vec_max<P>(x);
    tile_stats<SUM, ARG, 1, P>(x, ids, cm, c, a);
    if (BUF) tile_buffer<1, P>(x, &cm, cm, ids, wb, seg, hist, sh);
    if (VEC) tile_buffer_vec<1, VD>([&](int) { return rv; }, &cm, cm, vi, wb, seg, dat, hist, sh);
  }
  if (sp.tail0 < V) scalar(sp.tail0 + tid, sp.tail0 + tid < V, 8 + tid);
  if (VEC == 2 && wb.count > kTopPEnd && wb.count <= kWaveCap) {
    // at most kTopPEnd per wave at the end, so the block's certified vectors fit
    wave_lds_sync();
    int n = wb.count;
    const uint32_t tk = wave_sample_threshold(seg, n, keep, kTopPEnd);
    if (tk != 0u) {
      n = wave_keep_ge(seg, n, tk);
      wb.tau = key_to_float(tk);
    } else {
      wb.tau = entry_val(wave_compact(seg, hist, n, keep));
      n = keep;
    }
    wb.count = n;
    wave_lds_sync();
  }
  if ((BUF || VEC) && lane_id() == 0) {
    const int cap = VD ? kVecCap : kWaveCap;
    sh.wcount[w] = wb.count > cap ? cap : wb.count;
    sh.wtau[w] = wb.tau;
    if (wb.count > cap) atomicOr(&sh.woverflow, 1);
  }
}

// Visit every element once (no ordering across threads), 16-byte loads.
template <int DT, class F>
__device__ __forceinline__ void for_each_element(const void* row, int V, F&& f) {
  constexpr int P = Vec<DT>::kEpv;
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  if (tid < sp.head) f(Vec<DT>::load1(row, tid), tid);
  for (int vi = tid; vi < sp.nvec; vi += kBlock) {
    float x[P];
    Vec<DT>::unpack(__ldg(sp.vbase + vi), x);
    const int b = sp.head + vi * P;
#pragma unroll
    for (int e = 0; e < P; ++e) f(x[e], b + e);
  }
  if (sp.tail0 + tid < V) f(Vec<DT>::load1(row, sp.tail0 + tid), sp.tail0 + tid);
}

// As for_each_element with a small register footprint: one 32-bit word of a
// vector at a time (the exact path runs inside the streaming kernel).
template <int DT, class F>
__device__ __forceinline__ void for_each_element_lean(const void* row, int V, F&& f) {
  constexpr int P = Vec<DT>::kEpv;
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  if (tid < sp.head) f(Vec<DT>::load1(row, tid), tid);
  for (int vi = tid; vi < sp.nvec; vi += kBlock) {
    const uint4 v = __ldg(sp.vbase + vi);
    const int b = sp.head + vi * P;
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
      if (DT == 1) {
        f(bf16_lo(w), b + 2 * q);
        f(bf16_hi(w), b + 2 * q + 1);
      } else {
        f(__uint_as_float(w), b + q);
      }
    }
  }
  if (sp.tail0 + tid < V) f(Vec<DT>::load1(row, sp.tail0 + tid), sp.tail0 + tid);
}

// Every element of a row for a pass that one workgroup makes over the whole
// row: vec(x, id0) gets each 16-byte vector unpacked (P elements, ids id0..),
// elem(x, id) the scalar head and tail elements.  Up to 2U vectors are in
// flight per thread (the next group of U is loaded while the current one is
// visited): such a pass is bound by load latency otherwise.
template <int DT, int U, class FV, class FE>
__device__ __forceinline__ void for_each_vector_deep(const void* row, int V, FV&& vec, FE&& elem) {
  constexpr int P = Vec<DT>::kEpv;
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  if (tid < sp.head) elem(Vec<DT>::load1(row, tid), tid);
  // every load is issued (past the end: the last vector again, not used), so
  // the number of loads in flight is fixed and each wait covers only the
  // group being visited, not the one being fetched
  auto load = [&](int v0, uint4* w) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = v0 + u * kBlock;
      w[u] = __ldg(sp.vbase + (vi < sp.nvec ? vi : sp.nvec - 1));
    }
  };
  auto visit = [&](int v0, const uint4* w) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // the vector's registers are read on every path (an empty statement
      // that takes them as inputs), so its load is waited for here in every
      // lane, never left pending into the next iteration
      asm volatile("" ::"v"(w[u].x), "v"(w[u].y), "v"(w[u].z), "v"(w[u].w));
      const int vi = v0 + u * kBlock;
      if (vi < sp.nvec) {
        float x[P];
        Vec<DT>::unpack(w[u], x);
        vec(x, sp.head + vi * P);
      }
    }
  };
  constexpr int G = kBlock * U;  // vectors per group
  uint4 wa[U], wb[U];
  if (sp.nvec > 0) load(tid, wa);
  // the trip count is the same in every lane (groups, not this lane's
  // vectors), which keeps the waits partial
  for (int b0 = 0; b0 < sp.nvec; b0 += 2 * G) {
    load(b0 + G + tid, wb);
    visit(b0 + tid, wa);
    load(b0 + 2 * G + tid, wa);
    visit(b0 + G + tid, wb);  // (vectors past the end are skipped inside)
  }
  if (sp.tail0 + tid < V) elem(Vec<DT>::load1(row, sp.tail0 + tid), sp.tail0 + tid);
}

// Visit every element in tiles of increasing ids with a block-wide rank of the
// elements for which `tie(x)` holds: f(x, id, rank) where rank counts tie
// elements with a smaller id.  Every thread must call it.
template <int DT, class TieF, class F>
__device__ __forceinline__ void for_each_element_ranked(const void* row, int V, TieF&& tie, F&& f,
                                                        RowShared& sh) {
  constexpr int P = Vec<DT>::kEpv;
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  int run = 0;  // ties in earlier tiles
  auto scalar_tile = [&](int first, int n) {
    const int i = first + tid;
    const bool in = tid < n;
    const float x = in ? Vec<DT>::load1(row, i) : 0.0f;
    const bool t = in && tie(x);
    int total;
    const int r = block_exclusive_sum(t ? 1 : 0, sh.iscr, &total);
    if (in) f(x, i, run + r);
    run += total;
  };
  if (sp.head > 0) scalar_tile(0, sp.head);
  for (int v0 = 0; v0 < sp.nvec; v0 += kBlock) {
    const int vi = v0 + tid;
    const bool in = vi < sp.nvec;
    float x[P];
    Vec<DT>::unpack(in ? __ldg(sp.vbase + vi) : make_uint4(0u, 0u, 0u, 0u), x);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < P; ++e) cnt += (in && tie(x[e])) ? 1 : 0;
    int total;
    int r = block_exclusive_sum(cnt, sh.iscr, &total);
    if (in) {
      const int b = sp.head + vi * P;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const bool t = tie(x[e]);
        f(x[e], b + e, run + r);
        r += t ? 1 : 0;
      }
    }
    run += total;
  }
  if (sp.tail0 < V) scalar_tile(sp.tail0, V - sp.tail0);
}

}  // namespace sv
