// sv_rowpass.hpp -- one workgroup per logits row: a single coalesced streaming
// pass over the row, and the exact multi-pass path for rows whose kept set does
// not fit the candidate buffer.
//
// Streaming pass.  Each thread loads 16-byte vectors (8 bf16 or 4 fp32); the
// row is walked in tiles whose index ranges increase, so every element seen
// after a tile boundary has a larger id than every element seen before it.
// Per element the pass keeps a running max (and, when needed, the first index
// reaching it and an online sum of exp2((x - max) * log2e / T)).  Rows that
// need a top-k or top-p set also keep, in an LDS buffer, every element that is
// better in (value desc, id asc) order than a threshold entry theta; whenever
// the buffer grows past a limit a radix select over the 64-bit entries keeps
// the best `keep` and raises theta to the worst of them.  Because later
// elements have larger ids, an element with the value of theta can never beat
// it, so the filter is a single strict float compare -- done once per chunk on
// the chunk max in the common case.  The buffer always holds the best |buffer|
// elements of the prefix streamed so far.
#pragma once

#include "sv_device.hpp"

namespace sv {

struct RowShared {
  uint64_t buf[kCap];      // candidate entries; reused as histogram space
  uint32_t hist[256];
  double dscr[kWaves];
  uint64_t uscr[kWaves];
  float fscr[kWaves];
  int iscr[kWaves];
  int count;
  int overflow;
  float tau;
  int sel_digit, sel_need, sel_exact;
  int found;               // position of the draft token in a sorted list
  double zn_shared;
};

// --------------------------------------------------------------- selection
// Radix select over buf[0, n): returns (prefix, pmask) such that exactly `keep`
// entries satisfy (e & pmask) >= prefix -- the `keep` largest.  keep < n.
__device__ __forceinline__ void radix_select_top(RowShared& sh, int n, int keep, uint64_t& prefix,
                                        uint64_t& pmask) {
  prefix = 0;
  pmask = 0;
  int need = keep;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += kBlock) sh.hist[b] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kBlock) {
      uint64_t v = sh.buf[e];
      if ((v & pmask) == prefix) atomicAdd(&sh.hist[(uint32_t)(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave_id() == 0) {
      const int l = lane_id();
      // lane l owns digits 255-4l .. 252-4l, scanned from the top
      const int h0 = (int)sh.hist[255 - 4 * l], h1 = (int)sh.hist[254 - 4 * l];
      const int h2 = (int)sh.hist[253 - 4 * l], h3 = (int)sh.hist[252 - 4 * l];
      const int local = h0 + h1 + h2 + h3;
      const int incl = wave_inclusive_sum(local);
      const int excl = incl - local;
      const bool here = excl < need && need <= incl;
      const uint64_t m = __ballot(here);
      const int src = __ffsll((unsigned long long)m) - 1;
      if (l == src) {
        int c = excl, d, hd;
        if (c + h0 >= need) { d = 255 - 4 * l; hd = h0; }
        else if ((c += h0) + h1 >= need) { d = 254 - 4 * l; hd = h1; }
        else if ((c += h1) + h2 >= need) { d = 253 - 4 * l; hd = h2; }
        else { c += h2; d = 252 - 4 * l; hd = h3; }
        sh.sel_digit = d;
        sh.sel_need = need - c;
        sh.sel_exact = (hd == need - c) ? 1 : 0;
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

// Keep the `keep` best of buf[0, n) (n > keep), moved to buf[0, keep);
// sh.tau becomes the value of the worst kept entry.  In place, one 256-entry
// round at a time: round s reads entries [256s, 256s+256) and writes its kept
// ones at positions below 256(s+1), so no unread entry is overwritten.
__device__ __forceinline__ void compact_top(RowShared& sh, int n, int keep) {
  uint64_t prefix, pmask;
  radix_select_top(sh, n, keep, prefix, pmask);
  uint64_t mn = ~0ull;
  int pos0 = 0;
  for (int b0 = 0; b0 < n; b0 += kBlock) {
    const int e = b0 + threadIdx.x;
    const uint64_t v = e < n ? sh.buf[e] : 0ull;
    const bool k = e < n && (v & pmask) >= prefix;
    if (k) mn = v < mn ? v : mn;
    int total;
    const int pos = block_exclusive_sum(k ? 1 : 0, sh.iscr, &total);  // barriers: reads done
    if (k) sh.buf[pos0 + pos] = v;
    pos0 += total;
  }
  mn = block_min_u64(mn, sh.uscr);
  if (threadIdx.x == 0) {
    sh.count = keep;
    sh.tau = entry_val(mn);
  }
  __syncthreads();
}

// Sort buf[0, n) descending (n <= kCap).
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

// --------------------------------------------------------- streaming pass
struct StreamAcc {
  float mx;    // running max of this thread's elements
  int bi;      // first index reaching mx (ARG)
  float sref;  // reference of the running sum (SUM)
  double s;    // sum of exp2((x - sref) * c) (SUM)
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

// One chunk of NE elements of this thread, ids increasing with e.  `valid`
// masks elements (head, tail and ragged last tiles); wave-level operations stay
// in uniform control flow.
template <bool BUF, bool SUM, bool ARG, int NE>
__device__ __forceinline__ void consume_chunk(const float* x, const int* idx, const bool* valid,
                                              float c, float tau, StreamAcc& a, RowShared& sh) {
  float cm = -3.402823466e38f;
#pragma unroll
  for (int e = 0; e < NE; ++e)
    if (valid[e]) cm = fmaxf(cm, x[e]);
  if (ARG) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if (valid[e] && x[e] > a.mx) { a.mx = x[e]; a.bi = idx[e]; }
  } else {
    a.mx = fmaxf(a.mx, cm);
  }
  if (SUM) {
    if (cm > a.sref) {
      a.s *= (double)exp2f((a.sref - cm) * c);
      a.sref = cm;
    }
    float cs = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if (valid[e]) cs += exp2f((x[e] - a.sref) * c);
    a.s += (double)cs;
  }
  if (BUF) {
    const bool any = !(cm <= tau) && cm > -3.402823466e38f;
    if (__ballot(any)) {
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < NE; ++e) cnt += (valid[e] && !(x[e] <= tau)) ? 1 : 0;
      const int incl = wave_inclusive_sum(cnt);
      const int total = __shfl(incl, 63, 64);
      int base = 0;
      if (lane_id() == 63 && total > 0) base = atomicAdd(&sh.count, total);
      base = __shfl(base, 63, 64);
      int slot = base + incl - cnt;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        if (valid[e] && !(x[e] <= tau)) {
          if (slot < kCap) sh.buf[slot] = make_entry(x[e], idx[e]);
          ++slot;
        }
      }
    }
  }
}

// Tile boundary of a buffered stream: compact when the buffer passed its
// limit, flag overflow when appends were lost.  Returns the new threshold.
__device__ __forceinline__ float tile_end(RowShared& sh, int keep, int thresh, float tau) {
  __syncthreads();
  const int cnt = sh.count;
  const int ovf = sh.overflow;
  __syncthreads();
  if (ovf) return tau;
  if (cnt > kCap) {
    if (threadIdx.x == 0) {
      sh.overflow = 1;
      sh.tau = __int_as_float(0x7F800000);  // +inf: nothing passes any more
    }
    __syncthreads();
    return sh.tau;
  }
  if (cnt > thresh) compact_top(sh, cnt, keep);  // ends with a barrier
  return sh.tau;
}

// Stream one row.  Buffered rows keep the best `keep` (>= 1) elements.
template <int DT, bool BUF, bool SUM, bool ARG>
__device__ __forceinline__ void stream_row(const void* row, int V, float c, int keep, RowShared& sh,
                           StreamAcc& a) {
  constexpr int P = Vec<DT>::kEpv;
  const RowSplit<DT> sp(row, V);
  const int tid = threadIdx.x;
  a.mx = -3.402823466e38f;
  a.bi = 0x7FFFFFFF;
  a.sref = -3.402823466e38f;
  a.s = 0.0;
  float tau = __int_as_float(0x7FC00000);  // NaN admits everything
  int thresh = 2 * keep;
  thresh = thresh < 512 ? 512 : thresh;
  thresh = thresh > kCap / 2 ? kCap / 2 : thresh;
  thresh = thresh < keep ? keep : thresh;
  if (BUF) {
    if (tid == 0) {
      sh.count = 0;
      sh.overflow = 0;
      sh.tau = tau;
    }
    __syncthreads();
  }
  // head
  if (sp.head > 0) {
    float x[1];
    int id[1] = {tid};
    bool ok[1] = {tid < sp.head};
    x[0] = ok[0] ? Vec<DT>::load1(row, tid) : 0.0f;
    consume_chunk<BUF, SUM, ARG, 1>(x, id, ok, c, tau, a, sh);
    if (BUF) tau = tile_end(sh, keep, thresh, tau);
  }
  // body: a short ramp of small tiles for buffered rows, then 4 vectors/thread
  int v0 = 0;
  auto tile = [&](auto Ut) {
    constexpr int U = decltype(Ut)::value;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_stream(sp.vbase + v0 + u * kBlock + tid);
    float x[U * P];
    int id[U * P];
    bool ok[U * P];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Vec<DT>::unpack(v[u], x + u * P);
      const int b = sp.head + (v0 + u * kBlock + tid) * P;
#pragma unroll
      for (int e = 0; e < P; ++e) { id[u * P + e] = b + e; ok[u * P + e] = true; }
    }
    consume_chunk<BUF, SUM, ARG, U * P>(x, id, ok, c, tau, a, sh);
    v0 += U * kBlock;
    if (BUF) tau = tile_end(sh, keep, thresh, tau);
  };
  if (BUF) {
    if (v0 + kBlock <= sp.nvec) tile(std::integral_constant<int, 1>{});
    if (v0 + kBlock <= sp.nvec) tile(std::integral_constant<int, 1>{});
    if (v0 + 2 * kBlock <= sp.nvec) tile(std::integral_constant<int, 2>{});
  }
  while (v0 + 4 * kBlock <= sp.nvec) tile(std::integral_constant<int, 4>{});
  // ragged last tile of the body: vectors [v0, nvec)
  if (v0 < sp.nvec) {
    constexpr int U = 4;
    float x[U * P];
    int id[U * P];
    bool ok[U * P];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = v0 + u * kBlock + tid;
      const bool in = vi < sp.nvec;
      uint4 v = in ? load_stream(sp.vbase + vi) : make_uint4(0u, 0u, 0u, 0u);
      Vec<DT>::unpack(v, x + u * P);
      const int b = sp.head + vi * P;
#pragma unroll
      for (int e = 0; e < P; ++e) { id[u * P + e] = b + e; ok[u * P + e] = in; }
    }
    consume_chunk<BUF, SUM, ARG, U * P>(x, id, ok, c, tau, a, sh);
    if (BUF) tau = tile_end(sh, keep, thresh, tau);
  }
  // tail
  if (sp.tail0 < V) {
    float x[1];
    const int i = sp.tail0 + tid;
    int id[1] = {i};
    bool ok[1] = {i < V};
    x[0] = ok[0] ? Vec<DT>::load1(row, i) : 0.0f;
    consume_chunk<BUF, SUM, ARG, 1>(x, id, ok, c, tau, a, sh);
    if (BUF) tau = tile_end(sh, keep, thresh, tau);
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
  // head + tail handled as tiles of one element per thread
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
