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

struct RowShared {
  uint64_t buf[kCap];               // wave segments while streaming; merged area after
  uint32_t whist[kWaves][256];      // per-wave radix histograms; whist[0] at block level
  uint64_t mhist[256];              // fixed-point masses of the block-level mass walk
  double dscr[kWaves];
  uint64_t uscr[kWaves];
  float fscr[kWaves];
  int iscr[kWaves];
  int wcount[kWaves];               // final entries per wave segment
  uint64_t wtheta[kWaves];          // worst kept entry per wave (0: never compacted)
  float wtau[kWaves];               // published wave thresholds (-inf before any)
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
// seg[0, keep).  Returns the worst kept entry.  Only this wave takes part.
__device__ __forceinline__ uint64_t wave_compact(uint64_t* seg, uint32_t* hist, int n, int keep) {
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
    const uint64_t km = __ballot(k);
    const int off = __popcll(km & ((1ull << l) - 1ull));
    wave_lds_sync();
    if (k) {
      seg[pos0 + off] = v;
      mn = v < mn ? v : mn;
    }
    pos0 += __popcll(km);
    wave_lds_sync();
  }
  return wave_min_u64(mn);
}

// Wave-local exact selection for keep <= 64: every entry's rank is counted
// against the whole segment (broadcast LDS reads), four entries per lane at a
// time; the `keep` best go to `tmp` at their rank and then back to the front
// of the segment, sorted.  Returns the worst kept entry.
__device__ __forceinline__ uint64_t wave_select_small(uint64_t* seg, uint64_t* tmp, int n,
                                                      int keep) {
  const int l = lane_id();
  for (int j0 = 0; j0 < n; j0 += 256) {
    uint64_t mine[4];
    int rank[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = j0 + 64 * j + l;
      mine[j] = e < n ? seg[e] : 0ull;
      rank[j] = 0;
    }
    for (int u = 0; u < n; ++u) {
      const uint64_t v = seg[u];
#pragma unroll
      for (int j = 0; j < 4; ++j) rank[j] += v > mine[j] ? 1 : 0;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j0 + 64 * j + l < n && rank[j] < keep) tmp[rank[j]] = mine[j];
  }
  wave_lds_sync();
  if (l < keep) seg[l] = tmp[l];
  wave_lds_sync();
  return seg[keep - 1];
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

struct WaveBuf {
  int count;       // entries in the wave segment (may pass kWaveCap: overflow)
  float tau;       // own filter: value of theta_w (NaN admits everything), strict
  float tsh;       // shared filter: best published wave threshold, non-strict
  uint64_t theta;  // worst kept entry after a compaction (0 before any)
  int keep, thresh;
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

// Tree reductions over P = 1, 4 or 8 values.
template <int P>
__device__ __forceinline__ float tree_max(const float* x) {
  if constexpr (P == 1) return x[0];
  else if constexpr (P == 4) return fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  else return fmaxf(tree_max<4>(x), tree_max<4>(x + 4));
}
template <int P>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (P == 1) return x[0];
  else if constexpr (P == 4) return (x[0] + x[1]) + (x[2] + x[3]);
  else return tree_sum<4>(x) + tree_sum<4>(x + 4);
}

// Append the elements of one vector that pass both filters (wave-uniform
// call; rare once the thresholds have settled).  Element e has id id0 + e.
// Slots come from one ballot per element position: positions in the segment
// follow (e, lane) order, which the segment does not need to preserve.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <int P>
__device__ __forceinline__ void wave_append(const float* x, int id0, bool ok, WaveBuf& wb,
                                            uint64_t* seg) {
  int base = wb.count;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const bool pass = ok && !(x[e] <= wb.tau) && x[e] >= wb.tsh;
    const uint64_t m = __ballot(pass);
    if (pass) {
      const int slot = base + lanes_below(m);
      if (slot < kWaveCap) seg[slot] = make_entry(x[e], id0 + e);
    }
    base += __popcll(m);
  }
  wb.count = base;
}

// One tile of U vectors of P elements held by this thread.  Ids increase with
// (u, e).  The running max, argmax and sum reference move at most once per
// tile; the buffer append is one wave-uniform branch per tile.
template <bool BUF, bool SUM, bool ARG, int U, int P>
__device__ __forceinline__ void consume_tile(const float* x, const int* ids, const bool* ok,
                                             float c, StreamAcc& a, WaveBuf& wb, uint64_t* seg) {
  float um[U];
#pragma unroll
  for (int u = 0; u < U; ++u) um[u] = ok[u] ? tree_max<P>(x + u * P) : -3.402823466e38f;
  float cm = um[0];
#pragma unroll
  for (int u = 1; u < U; ++u) cm = fmaxf(cm, um[u]);
  if (cm > a.mx) {  // the running max moves: rare after the first tiles
    if (ARG) {
      int first = 0x7FFFFFFF;
#pragma unroll
      for (int u = U - 1; u >= 0; --u)
#pragma unroll
        for (int e = P - 1; e >= 0; --e)
          if (ok[u] && x[u * P + e] == cm) first = ids[u] + e;
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
    float part[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float w[P];
#pragma unroll
      for (int e = 0; e < P; ++e) w[e] = __builtin_amdgcn_exp2f(fmaf(x[u * P + e], c, a.nmc));
      part[u] = ok[u] ? tree_sum<P>(w) : 0.0f;
    }
    float cs = part[0];
#pragma unroll
    for (int u = 1; u < U; ++u) cs += part[u];
    a.s += (double)cs * a.corr;
  }
  if (BUF) {
    const bool any = !(cm <= wb.tau) && cm >= wb.tsh && cm > -3.402823466e38f;
    if (__ballot(any)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool pu = ok[u] && !(um[u] <= wb.tau) && um[u] >= wb.tsh;
        if (__ballot(pu)) wave_append<P>(x + u * P, ids[u], ok[u], wb, seg);
      }
    }
  }
}

// Wave tile boundary: compact the segment when it passed its limit; an
// overflowed segment stops admitting (the row then takes the exact path).
// Every wave filters by its own threshold (strict: its later elements have
// larger ids) and by the best threshold any wave has published (non-strict:
// ids interleave across waves).  An element below another wave's threshold
// value has `keep` better elements there, so it is in neither the row's top-k
// (k <= keep) nor the certified prefix; stale reads only lower the filter.
__device__ __forceinline__ void wave_tile_end(WaveBuf& wb, uint64_t* seg, uint32_t* hist,
                                              RowShared& sh) {
  if (wb.count > wb.thresh) {
    if (wb.count > kWaveCap) {
      wb.tau = __int_as_float(0x7F800000);  // +inf: overflowed, admit nothing more
      return;
    }
    wave_lds_sync();
    wb.theta = wb.keep <= 64 ? wave_select_small(seg, (uint64_t*)hist, wb.count, wb.keep)
                             : wave_compact(seg, hist, wb.count, wb.keep);
    wb.count = wb.keep;
    wb.tau = entry_val(wb.theta);
    if (lane_id() == 0) sh.wtau[wave_id()] = wb.tau;
  }
  float t = sh.wtau[0];
#pragma unroll
  for (int q = 1; q < kWaves; ++q) t = fmaxf(t, sh.wtau[q]);
  wb.tsh = t;
}

// Stream one row.  Buffered rows keep, per wave, the best `keep` elements
// (compacting when a segment holds more than `thresh`); `ramp` extra small
// tiles let a loose threshold settle before full tiles start.  Full tiles
// alternate between two load buffers so the next tile is always in flight.
template <int DT, bool BUF, bool SUM, bool ARG>
__device__ __forceinline__ void stream_row(const void* row, int V, float c, int keep, int thresh,
                                           int ramp, RowShared& sh, StreamAcc& a) {
  constexpr int P = Vec<DT>::kEpv;
  constexpr int U = SV_UNROLL;
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  const int w = wave_id();
  uint64_t* seg = sh.buf + w * kWaveCap;
  uint32_t* hist = sh.whist[w];
  a.bi = 0x7FFFFFFF;
  a.s = 0.0;
  a.mx = -3.402823466e38f;  // before any finite element: weights of -inf are 0
  a.nmc = 0.0f;
  a.corr = 1.0;
  WaveBuf wb;
  wb.count = 0;
  wb.tau = __int_as_float(0x7FC00000);  // NaN
  wb.tsh = -__int_as_float(0x7F800000);  // -inf
  wb.theta = 0ull;
  wb.keep = keep;
  wb.thresh = thresh;

  // scalar pieces (head and tail): one element per thread
  auto scalar = [&](int i, bool in) {
    float x[1] = {in ? Vec<DT>::load1(row, i) : 0.0f};
    int ids[1] = {i};
    bool ok[1] = {in};
    consume_tile<BUF, SUM, ARG, 1, 1>(x, ids, ok, c, a, wb, seg);
    if (BUF) wave_tile_end(wb, seg, hist, sh);
  };
  if (sp.head > 0) scalar(tid, tid < sp.head);

  int v0 = 0;
  auto small_tile = [&](auto Ut) {
    constexpr int UU = decltype(Ut)::value;
    uint4 v[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) v[u] = load_stream(sp.vbase + v0 + u * kBlock + tid);
    float x[UU * P];
    int ids[UU];
    bool ok[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      Vec<DT>::unpack(v[u], x + u * P);
      ids[u] = sp.head + (v0 + u * kBlock + tid) * P;
      ok[u] = true;
    }
    consume_tile<BUF, SUM, ARG, UU, P>(x, ids, ok, c, a, wb, seg);
    v0 += UU * kBlock;
    if (BUF) wave_tile_end(wb, seg, hist, sh);
  };
  if (BUF && keep <= 64 && v0 + kBlock <= sp.nvec) {
    // first tile: admit only entries at least as good as the keep-th best lane
    // maximum -- keep lanes hold an entry that good, so nothing better is lost
    const uint4 v = load_stream(sp.vbase + v0 + tid);
    float x[P];
    Vec<DT>::unpack(v, x);
    const int id0 = sp.head + (v0 + tid) * P;
    int ids[1] = {id0};
    bool ok[1] = {true};
    consume_tile<false, SUM, ARG, 1, P>(x, ids, ok, c, a, wb, seg);
    uint64_t best = 0ull;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const uint64_t en = make_entry(x[e], id0 + e);
      best = en > best ? en : best;
    }
    int rank = 0;
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((uint32_t)best, u);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(best >> 32), u);
      rank += (((uint64_t)hi << 32) | (uint64_t)lo) > best ? 1 : 0;
    }
    const uint64_t sel = __ballot(rank == keep - 1);
    uint64_t theta0 = 0ull;
    if (sel) {
      const int src = __ffsll((unsigned long long)sel) - 1;
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(best >> 32), src);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((uint32_t)best, src);
      theta0 = ((uint64_t)hi << 32) | (uint64_t)lo;
    }
    int base = 0;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const uint64_t en = make_entry(x[e], id0 + e);
      const bool pass = en >= theta0;
      const uint64_t m = __ballot(pass);
      if (pass) {
        const int slot = base + lanes_below(m);
        if (slot < kWaveCap) seg[slot] = en;
      }
      base += __popcll(m);
    }
    wb.count = base;
    if (theta0) {
      wb.theta = theta0;
      wb.tau = entry_val(theta0);
      if (lane_id() == 0) sh.wtau[w] = wb.tau;
    }
    v0 += kBlock;
    wave_tile_end(wb, seg, hist, sh);
  }
  if (BUF) {
    if (v0 + kBlock <= sp.nvec) small_tile(std::integral_constant<int, 1>{});
    if (v0 + kBlock <= sp.nvec) small_tile(std::integral_constant<int, 1>{});
    for (int r = 0; r < ramp; ++r)
      if (v0 + 2 * kBlock <= sp.nvec) small_tile(std::integral_constant<int, 2>{});
  }
  while (v0 + U * kBlock <= sp.nvec) small_tile(std::integral_constant<int, U>{});
  // ragged last tiles of the body: vectors [v0, nvec), one per thread
  for (; v0 < sp.nvec;) {
    const int vi = v0 + tid;
    const bool in = vi < sp.nvec;
    float x[P];
    Vec<DT>::unpack(in ? load_stream(sp.vbase + vi) : make_uint4(0u, 0u, 0u, 0u), x);
    int ids[1] = {sp.head + vi * P};
    bool ok[1] = {in};
    consume_tile<BUF, SUM, ARG, 1, P>(x, ids, ok, c, a, wb, seg);
    v0 += kBlock;
    if (BUF) wave_tile_end(wb, seg, hist, sh);
  }
  if (sp.tail0 < V) scalar(sp.tail0 + tid, sp.tail0 + tid < V);
  if (BUF && lane_id() == 0) {
    sh.wcount[w] = wb.count > kWaveCap ? kWaveCap : wb.count;
    sh.wtheta[w] = wb.theta;
    if (wb.count > kWaveCap) atomicOr(&sh.woverflow, 1);
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
