// sv_device.hpp -- device helpers for the verify kernels (gfx950, wave64).
//
// Philox4x32-10 follows Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3" (SC'11): two 32x32->64 multiplies per round with the
// paper's multipliers, Weyl key increments between rounds, ten rounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Tuning knobs of the streaming row pass (defaults are the tuned values).
#ifndef SV_BLOCK
#define SV_BLOCK 256        // threads per row workgroup
#endif
#ifndef SV_UNROLL
#define SV_UNROLL 4         // 16-byte vectors per thread per tile
#endif
#ifndef SV_PREFETCH
#define SV_PREFETCH 1       // issue the next tile's loads before consuming this one
#endif
#ifndef SV_NT_LOADS
#define SV_NT_LOADS 1       // non-temporal loads for the logits stream
#endif
#ifndef SV_CHECK_EVERY
#define SV_CHECK_EVERY 1    // tiles between candidate-buffer checks after the ramp
#endif

namespace sv {

constexpr int kBlock = SV_BLOCK;          // threads per row workgroup
constexpr int kWaves = kBlock / 64;
constexpr int kCap = 4096;                // LDS candidate buffer (64-bit entries)
constexpr int kKeepTopP = 384;            // candidates kept per wave for top-k-off rows
constexpr int kThreshTopP = 768;          // per-wave compaction limit for those rows
constexpr int kTopPEnd = 512;             // top-p vector candidates per wave after the stream
constexpr int kTopkFast = 256;            // largest k on the buffer path
constexpr int kTopkVec = 64;              // largest k on the vector-candidate path
constexpr int kThreshVec = 128;           // per-wave compaction limit there (>= 2 kTopkVec)
constexpr int kListCap = 4096;            // kept-set entries stored per row (workspace)
constexpr int kKmaxCap = 1024;            // largest kmax of the target-probs build
constexpr float kLog2e = 1.4426950408889634f;

// Row modes recorded by the row pass.
enum : int32_t {
  kModeSkip = 0,    // row never used (past the verify cap)
  kModeGreedy = 1,  // one-hot at the argmax
  kModeList = 2,    // kept set stored as an explicit list
  kModeAll = 3,     // kept set is the whole row (top-k and top-p off)
  kModeRange = 4,   // kept set = {key > bkey} + first nb ties at bkey
  kModePending = 5  // kept set needs the exact multi-pass path (resolved later)
};

// Row record flag bits.
enum : int32_t {
  kRecAccept = 1,
  kRecTested = 2,
  kRecExact = 4,      // kept set came from the multi-pass exact path
  kRecBadDraft = 8,
  kRecSampled = 16,   // `sample` holds this row's emitted token if it is the emit row
  kRecResidEmpty = 32, // that sample came from p: the residual was zero on the kept set
  kRecTieCut = 64      // kModeRange: tie_cut holds the id past the last kept element at bkey
};

struct RowRec {
  float m;        // row max
  int32_t a;      // argmax (lowest id)
  int32_t mode;
  int32_t nkeep;  // |N|
  double zn;      // mass of N relative to exp(m/T)
  double zk;      // mass of K (or of the whole row) relative to exp(m/T)
  uint32_t bkey;  // kModeRange: order key of the boundary value
  int32_t nb;     // kModeRange: ties at bkey that are kept (lowest ids)
  int32_t flags;
  float lse;      // log sum exp(x / T_eff) over the row (build path)
  double pd;      // p(d) of the tested draft, as the ratio test used it
  int32_t sample;  // kRecSampled: token emitted when this row is the request's emit row
  int32_t tie_cut; // kRecTieCut: elements at bkey with a smaller id are the kept ties
};
static_assert(sizeof(RowRec) == 64, "RowRec layout");

struct ListEntry {
  int32_t idx;
  float x;
};

// ---------------------------------------------------------------- Philox
__device__ __forceinline__ uint4 philox4x32_10(uint32_t k0, uint32_t k1, uint4 c) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    // one 32 x 32 -> 64-bit product per multiplier (both halves at once)
    const uint64_t p0 = (uint64_t)M0 * c.x, p1 = (uint64_t)M1 * c.z;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Acceptance uniform: 53 bits of words 0-1, in [0, 1).  Counter (position,
// request id, tag 0, 0).
__device__ __forceinline__ double accept_uniform(uint64_t seed, uint32_t rid, uint32_t pos) {
  uint4 o = philox4x32_10((uint32_t)seed, (uint32_t)(seed >> 32), make_uint4(pos, rid, 0u, 0u));
  uint64_t bits = ((uint64_t)o.y << 32) | (uint64_t)o.x;
  return (double)(bits >> 11) * 0x1.0p-53;
}

// Race uniform for token v: word (v & 3) of counter (position, request id,
// tag, v >> 2), mapped to an odd multiple of 2^-24 in (0, 1).
__device__ __forceinline__ uint32_t race_word(uint64_t seed, uint32_t rid, uint32_t pos,
                                              uint32_t tag, uint32_t v) {
  uint4 o = philox4x32_10((uint32_t)seed, (uint32_t)(seed >> 32), make_uint4(pos, rid, tag, v >> 2));
  uint32_t lane = v & 3u;
  return lane == 0 ? o.x : lane == 1 ? o.y : lane == 2 ? o.z : o.w;
}
__device__ __forceinline__ double race_uniform(uint64_t seed, uint32_t rid, uint32_t pos,
                                               uint32_t tag, uint32_t v) {
  uint32_t w = race_word(seed, rid, pos, tag, v);
  return (double)(2u * (w >> 9) + 1u) * 0x1.0p-24;
}

// ------------------------------------------------------------- keys
// Order key of a float: unsigned order equals numeric order; -0 maps to +0.
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  u = (f == 0.0f) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// Candidate entry: larger entry = better = (value desc, id asc).
__device__ __forceinline__ uint64_t make_entry(float x, int32_t idx) {
  return ((uint64_t)fkey(x) << 32) | (uint64_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int32_t entry_idx(uint64_t e) { return (int32_t)(~(uint32_t)e); }
__device__ __forceinline__ float entry_val(uint64_t e) { return key_to_float((uint32_t)(e >> 32)); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Streaming 16-byte load (non-temporal: the logits are read once).
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
#if SV_NT_LOADS
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// --------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

template <class T>
__device__ __forceinline__ T wave_inclusive_sum(T v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    T y = __shfl_up(v, d, 64);
    if (lane_id() >= d) v += y;
  }
  return v;
}
// Inclusive sum over the lanes of a fully active wave by DPP row shifts and
// row broadcasts (register moves, no LDS round trips).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_from(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_from_d(double v) {
  const int lo = dpp_from<CTRL, ROWS>(__double2loint(v));
  const int hi = dpp_from<CTRL, ROWS>(__double2hiint(v));
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += dpp_from<0x111, 0xF>(v);  // row_shr:1
  v += dpp_from<0x112, 0xF>(v);  // row_shr:2
  v += dpp_from<0x114, 0xF>(v);  // row_shr:4
  v += dpp_from<0x118, 0xF>(v);  // row_shr:8
  v += dpp_from<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_from<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ double wave_scan_dpp(double v) {
  v += dpp_from_d<0x111, 0xF>(v);
  v += dpp_from_d<0x112, 0xF>(v);
  v += dpp_from_d<0x114, 0xF>(v);
  v += dpp_from_d<0x118, 0xF>(v);
  v += dpp_from_d<0x142, 0xA>(v);
  v += dpp_from_d<0x143, 0xC>(v);
  return v;
}
// Value of lane l - 1 (0 in lane 0): DPP wave_shr:1.
__device__ __forceinline__ double wave_prev_d(double v) { return dpp_from_d<0x138, 0xF>(v); }
__device__ __forceinline__ double readlane_d(double v, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int d) {
  uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    uint64_t o = shfl_xor_u64(v, d);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    uint64_t o = shfl_xor_u64(v, d);
    v = o < v ? o : v;
  }
  return v;
}

// Block-wide reductions through a small LDS scratch (kWaves slots).  Every
// thread of the block must call them; they end with the result visible to all.
__device__ __forceinline__ double block_sum_d(double v, double* scratch) {
  v = wave_sum_d(v);
  __syncthreads();
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += scratch[w];  // fixed order: deterministic
  return t;
}
__device__ __forceinline__ int block_sum_i(int v, int* scratch) {
  v = wave_sum_i(v);
  __syncthreads();
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += scratch[w];
  return t;
}
__device__ __forceinline__ float block_max_f(float v, float* scratch) {
  v = wave_max_f(v);
  __syncthreads();
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  float t = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = fmaxf(t, scratch[w]);
  return t;
}
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* scratch) {
  v = wave_max_u64(v);
  __syncthreads();
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  uint64_t t = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = scratch[w] > t ? scratch[w] : t;
  return t;
}
__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t* scratch) {
  v = wave_min_u64(v);
  __syncthreads();
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  uint64_t t = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = scratch[w] < t ? scratch[w] : t;
  return t;
}
// Exclusive prefix sum over the block in thread order; returns the total.
__device__ __forceinline__ int block_exclusive_sum(int v, int* scratch, int* total) {
  int incl = wave_inclusive_sum(v);
  __syncthreads();
  if (lane_id() == 63) scratch[wave_id()] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave_id()) base += scratch[w];
    tot += scratch[w];
  }
  *total = tot;
  return base + incl - v;
}
__device__ __forceinline__ double block_exclusive_sum_d(double v, double* scratch, double* total) {
  double incl = wave_inclusive_sum(v);
  __syncthreads();
  if (lane_id() == 63) scratch[wave_id()] = incl;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave_id()) base += scratch[w];
    tot += scratch[w];
  }
  *total = tot;
  return base + (incl - v);
}

// Request of packed row i: the r with qo[r] <= i < qo[r + 1] (qo
// non-decreasing, qo[0] = 0, qo[R] = rows).  Evenly packed windows resolve
// from the proportional guess in one load round; otherwise an upper-bound
// search.
__device__ __forceinline__ int row_to_request(const int32_t* qo, int R, int rows, int i) {
  if (rows > 0) {
    const int g = (int)(((long long)i * R) / rows);
    if (g < R && __ldg(qo + g) <= i && i < __ldg(qo + g + 1)) return g;
  }
  int lo = 0, hi = R;  // find last r with qo[r] <= i, among requests with rows
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (__ldg(qo + mid) <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace sv
