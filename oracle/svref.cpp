/*
 * svref.cpp -- CPU oracle for the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY (see svref.h).  Plain single-threaded C++17, fp64
 * arithmetic, one full std::sort per row.  Nothing here is blocked, fused or
 * reordered beyond what the definitions below state, so each step can be read
 * against the pages.  Built with g++ -O2 -ffp-contract=off and no fast-math.
 *
 * Readings taken where the pages are silent:
 *  - logits are converted exactly to fp64; a bf16 value is its bit pattern
 *    shifted into the high half of an fp32.
 *  - ties: the order of a row is (value descending, index ascending); the
 *    argmax, the top-k set and the top-p walk all use it.
 *  - filter order: top-k on the raw logits, then temperature, then top-p on the
 *    top-k renormalised distribution (standard nucleus: keep pi_t while the
 *    mass before it is below P * Z_K; pi_0 is always kept).
 *  - greedy rows (T <= 0 or NaN) use the argmax; their lse is taken at T = 1.
 *  - a draft id outside [0, V) is rejected and the row then samples from p,
 *    since nothing was proposed there.
 *  - q(d) = 0 gives ratio 1 when p(d) > 0 and 0 otherwise.
 *  - a residual that is zero on the whole kept set falls back to p.
 *  - confidences are clamped to [0,1] with NaN -> 0; survival products are fp32,
 *    left to right; the rank key is (S desc, j asc, r asc).
 */
#include "svref.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

namespace {

/* ---------------- Philox4x32-10 (Salmon et al., SC'11) ---------------- */
/* Round multipliers and Weyl key increments as published in the paper. */
const uint32_t kPhiloxM0 = 0xD2511F53u;
const uint32_t kPhiloxM1 = 0xCD9E8D57u;
const uint32_t kPhiloxW0 = 0x9E3779B9u;
const uint32_t kPhiloxW1 = 0xBB67AE85u;

void philox_round(uint32_t c[4], const uint32_t k[2]) {
  /* Two 32x32 -> 64 products; the high halves are mixed with the other two
   * counter words and the key, the low halves are moved across. */
  uint64_t prod0 = (uint64_t)kPhiloxM0 * (uint64_t)c[0];
  uint64_t prod1 = (uint64_t)kPhiloxM1 * (uint64_t)c[2];
  uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
  uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n1 = lo1;
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  uint32_t n3 = lo0;
  c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void philox10(const uint32_t key[2], const uint32_t ctr[4], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k[0] += kPhiloxW0; k[1] += kPhiloxW1; }
    philox_round(c, k);
  }
  out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* Counter layout: (absolute position, request id, stream tag, block). */
double uniform_accept(uint64_t seed, uint32_t rid, uint32_t pos) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {pos, rid, 0u, 0u};
  uint32_t o[4];
  philox10(key, ctr, o);
  uint64_t bits = ((uint64_t)o[1] << 32) | (uint64_t)o[0];
  return (double)(bits >> 11) * 0x1.0p-53;  /* 53 random bits -> [0, 1) */
}

double uniform_race(uint64_t seed, uint32_t rid, uint32_t pos, uint32_t tag, uint32_t token) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {pos, rid, tag, token >> 2};
  uint32_t o[4];
  philox10(key, ctr, o);
  uint32_t word = o[token & 3u];
  /* 23 random bits placed at odd multiples of 2^-24: never 0, never 1. */
  return (double)(2u * (word >> 9) + 1u) * 0x1.0p-24;
}

/* ---------------- per-row target distribution ---------------- */

double load_logit(const void* logits, int32_t dtype, int64_t ld, int64_t row, int64_t v) {
  if (dtype == SVREF_F32) {
    return (double)((const float*)logits)[row * ld + v];
  }
  uint16_t h = ((const uint16_t*)logits)[row * ld + v];
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

struct Params {
  bool greedy;
  double T;      /* request temperature (meaningful when !greedy) */
  int32_t k;     /* raw top-k value */
  float P;       /* raw top-p value */
};

struct RowDist {
  double m = 0;          /* row max                                  */
  int32_t a = -1;        /* argmax, lowest index among ties          */
  double lse = 0;        /* log sum exp(x / T_eff)                   */
  std::vector<int32_t> kept;  /* N in order (value desc, index asc)  */
  std::vector<int32_t> order; /* the row order pi (sampled rows)     */
  std::vector<double> p;      /* dense p_v over the vocabulary       */
  double zk = 0, zn = 0;      /* masses of K and N relative to max   */
  int32_t n_lo = 0, n_hi = 0; /* kept counts over the near-tie band  */
  bool near_topp = false;
};

/* Kept count of the nucleus walk for a mass target: positions t < kc whose
 * prefix mass before them is below the target (pi_0 is counted whenever the
 * target is positive). */
int32_t nucleus_count(const std::vector<double>& w, int32_t kc, double target) {
  double c = 0.0;
  int32_t n = 0;
  for (int32_t t = 0; t < kc; ++t) {
    if (c < target) { ++n; c += w[t]; } else { break; }
  }
  return n;
}

void build_row(const void* logits, int32_t dtype, int64_t ld, int64_t row, int32_t V,
               const Params& prm, RowDist& out) {
  std::vector<double> x(V);
  for (int32_t v = 0; v < V; ++v) x[v] = load_logit(logits, dtype, ld, row, v);

  /* O1: max and lowest-index argmax. */
  double m = x[0];
  int32_t a = 0;
  for (int32_t v = 1; v < V; ++v) {
    if (x[v] > m) { m = x[v]; a = v; }
  }
  out.m = m;
  out.a = a;

  /* lse at T_eff over the whole vocabulary. */
  double teff = prm.greedy ? 1.0 : prm.T;
  double s = 0.0;
  for (int32_t v = 0; v < V; ++v) s += std::exp((x[v] - m) / teff);
  out.lse = m / teff + std::log(s);

  out.p.assign(V, 0.0);
  out.kept.clear();
  out.near_topp = false;

  if (prm.greedy) {
    /* O2: one-hot at the argmax. */
    out.kept.push_back(a);
    out.order.assign(1, a);
    out.p[a] = 1.0;
    out.zk = out.zn = 1.0;
    out.n_lo = out.n_hi = 1;
    return;
  }

  /* O3: the row order pi. */
  std::vector<int32_t> pi(V);
  std::iota(pi.begin(), pi.end(), 0);
  std::sort(pi.begin(), pi.end(), [&](int32_t i, int32_t j) {
    if (x[i] != x[j]) return x[i] > x[j];
    return i < j;
  });

  /* O4: top-k on the raw logits. */
  int32_t kc = (prm.k > 0 && prm.k < V) ? prm.k : V;

  /* O5: temperature applied to the selected values only; mass in pi order. */
  std::vector<double> w(kc);
  double zk = 0.0;
  for (int32_t t = 0; t < kc; ++t) {
    w[t] = std::exp((x[pi[t]] - m) / prm.T);
    zk += w[t];
  }
  out.zk = zk;

  /* O6: top-p nucleus over K. */
  int32_t n = kc;
  if (!(prm.P < 1.0f)) {
    n = kc;                        /* off (P >= 1 or NaN) */
    out.n_lo = out.n_hi = n;
  } else if (!(prm.P > 0.0f)) {
    n = 1;                         /* P <= 0 keeps the top token */
    out.n_lo = out.n_hi = n;
  } else {
    const double target = (double)prm.P * zk;
    n = nucleus_count(w, kc, target);
    /* Near-tie band: the kept counts a target anywhere within 1e-6 * Z_K of
     * P * Z_K would give.  The row is a top-p near tie when they differ. */
    const double band = 1e-6 * zk;
    out.n_lo = std::max(1, nucleus_count(w, kc, target - band));
    out.n_hi = nucleus_count(w, kc, target + band);
    out.near_topp = out.n_lo != out.n_hi;
  }

  /* O7: probabilities on N. */
  double zn = 0.0;
  for (int32_t t = 0; t < n; ++t) zn += w[t];
  out.zn = zn;
  out.kept.assign(pi.begin(), pi.begin() + n);
  out.order.swap(pi);
  for (int32_t t = 0; t < n; ++t) out.p[out.order[t]] = w[t] / zn;
}

Params request_params(const svref_sampling* sp, int32_t r) {
  Params prm;
  float T = sp->temperature ? sp->temperature[r] : 0.0f;
  prm.greedy = !(T > 0.0f);
  prm.T = (double)T;
  prm.k = sp->top_k ? sp->top_k[r] : 0;
  prm.P = sp->top_p ? sp->top_p[r] : 1.0f;
  return prm;
}

/* O9: exponential race.  Winner = argmax over weight_v / E_v with
 * E_v = -ln U_v, over weights > 0; ties go to the lower token id. */
struct RaceResult {
  int32_t token = -1;
  bool near = false;
};

template <class WeightFn>
RaceResult race(const std::vector<int32_t>& cand, WeightFn weight, uint64_t seed, uint32_t rid,
                uint32_t pos, uint32_t tag) {
  RaceResult res;
  double best = -1.0, second = -1.0;
  int32_t best_v = -1;
  for (int32_t v : cand) {
    double wv = weight(v);
    if (!(wv > 0.0)) continue;
    double e = -std::log(uniform_race(seed, rid, pos, tag, (uint32_t)v));
    double key = wv / e;
    if (key > best || (key == best && v < best_v)) {
      second = best;
      best = key;
      best_v = v;
    } else if (key > second) {
      second = key;
    }
  }
  res.token = best_v;
  if (best_v >= 0 && second > 0.0 && (best - second) / best < 1e-6) res.near = true;
  return res;
}

/* Block verification of one sampled request (Sun, Mendlovic, Leviathan,
 * Aharoni, Beirami, Ro, Suresh, "Block Verification Accelerates Speculative
 * Decoding": the block is accepted jointly, not token by token, and the
 * correction token comes from a residual reweighted by the block's weight).
 * Rows s..s+G verify drafts 0..G-1 (G = the verified positions) and row s+G is
 * the row after them.  In the paper's notation, with M_b the target and M_s
 * the draft distribution of each row:
 *   p_0 = 1; p_i = min(p_{i-1} M_b(X_i) / M_s(X_i), 1)        (row i-1, i = 1..G)
 *   h_i = A_i / (A_i + 1 - p_i), A_i = sum_x max(p_i M_b(x) - M_s(x), 0) over
 *         row i, for i < G;  h_G = p_G
 *   tau = the largest i with eta_i < h_i (0 if none)
 *   emitted: X_1..X_tau, then Y from row tau: M_b when tau = G, otherwise
 *         the residual max(p_tau M_b - M_s, 0) (normalised).
 * Readings: eta_i is the acceptance uniform of row i - 1 (so G = 1 is the
 * token rule with the same uniform, a strict '<' as there); a draft id
 * outside [0, V) has ratio 0, and when it is the draft of row tau, Y comes
 * from M_b (nothing was proposed there); q = 0 at the draft gives ratio 1
 * when M_b(X) > 0 (0 otherwise), p_i = 0 once any ratio was 0; h_i = 1 when
 * its denominator is 0 (then p_i = 1 and row i's distributions agree, and a
 * later position is always accepted); an all-zero residual falls back to M_b
 * (flagged, as in the token rule).  Row flags: ACCEPT on row i - 1 when
 * eta_i < h_i; NEAR_RATIO when |eta_i - h_i| < 1e-5; ratio / u diagnostics
 * hold h_i and eta_i. */
void block_verify_request(const void* logits, int32_t dtype, int64_t ld, int32_t V, int32_t s,
                          int32_t G, const int32_t* draft_tokens, const float* draft_probs,
                          int64_t ld_q, const Params& prm, uint64_t seed, uint32_t rid,
                          uint32_t pos0, int32_t& accept_len, int32_t& next_token,
                          int32_t* out_tokens, uint8_t* row_flags, double* row_ratio,
                          double* row_u, double* row_zk, double* row_zn) {
  std::vector<RowDist> rows((size_t)G + 1);
  for (int32_t j = 0; j <= G; ++j) {
    build_row(logits, dtype, ld, s + j, V, prm, rows[j]);
    if (row_zk) row_zk[s + j] = rows[j].zk;
    if (row_zn) row_zn[s + j] = rows[j].zn;
  }
  auto q_of = [&](int32_t j, int32_t v) { return (double)draft_probs[(int64_t)(s + j) * ld_q + v]; };
  auto bad = [&](int32_t j) { return draft_tokens[s + j] < 0 || draft_tokens[s + j] >= V; };

  /* the block weights p_0..p_G */
  std::vector<double> p((size_t)G + 1);
  p[0] = 1.0;
  for (int32_t i = 1; i <= G; ++i) {
    const int32_t j = i - 1;
    double ratio = 0.0;
    if (!bad(j)) {
      const int32_t x = draft_tokens[s + j];
      const double pb = rows[j].p[x], qs = q_of(j, x);
      ratio = qs > 0.0 ? pb / qs : (pb > 0.0 ? HUGE_VAL : 0.0);
    }
    p[i] = p[i - 1] > 0.0 ? std::min(p[i - 1] * ratio, 1.0) : 0.0;
  }

  /* the acceptance test of every position; tau is the last one passed */
  int32_t tau = 0;
  for (int32_t i = 1; i <= G; ++i) {
    double h;
    if (i < G) {
      double A = 0.0;  /* M_b is zero off the kept set, so only it contributes */
      for (int32_t x : rows[i].kept) A += std::max(p[i] * rows[i].p[x] - q_of(i, x), 0.0);
      const double den = A + 1.0 - p[i];
      h = den > 0.0 ? A / den : 1.0;
    } else {
      h = p[G];
    }
    const int32_t j = i - 1;
    const double eta = uniform_accept(seed, rid, pos0 + (uint32_t)j);
    uint8_t fl = bad(j) ? SVREF_ROW_BAD_DRAFT : 0;
    if (eta < h) {
      tau = i;
      fl |= SVREF_ROW_ACCEPT;
    }
    if (std::fabs(eta - h) < 1e-5) fl |= SVREF_ROW_NEAR_RATIO;
    if (rows[j].near_topp) fl |= SVREF_ROW_NEAR_TOPP;
    if (row_flags) row_flags[s + j] = fl;
    if (row_ratio) row_ratio[s + j] = h;
    if (row_u) row_u[s + j] = eta;
  }

  /* the emitted token from row tau */
  const RowDist& dt = rows[tau];
  const uint32_t pos = pos0 + (uint32_t)tau;
  uint8_t sfl = SVREF_ROW_SAMPLED | (dt.near_topp ? SVREF_ROW_NEAR_TOPP : 0);
  RaceResult rr;
  bool use_p = tau == G || bad(tau);
  if (!use_p) {
    const double w = p[tau];
    auto resid = [&](int32_t v) { return std::max(w * dt.p[v] - q_of(tau, v), 0.0); };
    rr = race(dt.kept, resid, seed, rid, pos, 1u);
    if (rr.token < 0) {
      use_p = true;
      sfl |= SVREF_ROW_RESID_EMPTY;
    }
  }
  if (use_p) {
    auto pw = [&](int32_t v) { return dt.p[v]; };
    rr = race(dt.kept, pw, seed, rid, pos, 1u);
  }
  if (rr.near) sfl |= SVREF_ROW_NEAR_RACE;
  if (row_flags) row_flags[s + tau] |= sfl;
  for (int32_t j = 0; j < tau; ++j) out_tokens[s + j] = draft_tokens[s + j];
  out_tokens[s + tau] = rr.token;
  accept_len = tau;
  next_token = rr.token;
}

bool check_layout(const int32_t* qo, int32_t R, int32_t rows) {
  if (R < 0 || rows < 0 || qo == nullptr) return false;
  if (qo[0] != 0 || qo[R] != rows) return false;
  for (int32_t r = 0; r < R; ++r)
    if (qo[r + 1] < qo[r]) return false;
  return true;
}

}  // namespace

extern "C" {

void svref_philox4x32_10(const uint32_t key[2], const uint32_t ctr[4], uint32_t out[4]) {
  philox10(key, ctr, out);
}

double svref_uniform_accept(uint64_t seed, uint32_t request_id, uint32_t position) {
  return uniform_accept(seed, request_id, position);
}

double svref_uniform_race(uint64_t seed, uint32_t request_id, uint32_t position, uint32_t tag,
                          uint32_t token) {
  return uniform_race(seed, request_id, position, tag, token);
}

int32_t svref_build_target_probs(const void* logits, int32_t dtype, int64_t ld_logits,
                                 int32_t num_rows, int32_t vocab, const int32_t* qo_indptr,
                                 int32_t num_requests, const svref_sampling* sp, double* probs,
                                 int64_t ld_probs, double* row_max, int32_t* row_argmax,
                                 double* row_lse, int32_t* kept_count, int32_t* kept_idx,
                                 int32_t kmax, double* row_zn, uint8_t* row_flags,
                                 double* row_zk, int32_t* kept_lo, int32_t* kept_hi,
                                 int32_t* order_idx) {
  if (!logits || !sp || vocab <= 0 || ld_logits < vocab) return -1;
  if (dtype != SVREF_F32 && dtype != SVREF_BF16) return -3;
  if (!check_layout(qo_indptr, num_requests, num_rows)) return -2;
  if (probs && ld_probs < vocab) return -2;
  RowDist d;
  for (int32_t r = 0; r < num_requests; ++r) {
    Params prm = request_params(sp, r);
    for (int32_t i = qo_indptr[r]; i < qo_indptr[r + 1]; ++i) {
      build_row(logits, dtype, ld_logits, i, vocab, prm, d);
      if (row_max) row_max[i] = d.m;
      if (row_argmax) row_argmax[i] = d.a;
      if (row_lse) row_lse[i] = d.lse;
      if (row_zn) row_zn[i] = d.zn;
      if (row_zk) row_zk[i] = d.zk;
      if (row_flags) row_flags[i] = d.near_topp ? SVREF_ROW_NEAR_TOPP : 0;
      if (kept_count) kept_count[i] = (int32_t)d.kept.size();
      if (kept_lo) kept_lo[i] = d.n_lo;
      if (kept_hi) kept_hi[i] = d.n_hi;
      if (kept_idx) {
        for (int32_t t = 0; t < kmax; ++t)
          kept_idx[(int64_t)i * kmax + t] = t < (int32_t)d.kept.size() ? d.kept[t] : -1;
      }
      if (order_idx) {
        for (int32_t t = 0; t < kmax; ++t)
          order_idx[(int64_t)i * kmax + t] = t < (int32_t)d.order.size() ? d.order[t] : -1;
      }
      if (probs) {
        for (int32_t v = 0; v < vocab; ++v) probs[(int64_t)i * ld_probs + v] = d.p[v];
      }
    }
  }
  return 0;
}

int32_t svref_rejection_sample(const void* logits, int32_t dtype, int64_t ld_logits,
                               int32_t vocab, const int32_t* qo_indptr, int32_t num_requests,
                               int32_t num_rows, const int32_t* draft_tokens,
                               const float* draft_probs, int64_t ld_q, const int32_t* verify_cap,
                               const svref_sampling* sp, int32_t* accept_len, int32_t* out_tokens,
                               int32_t* next_token, uint8_t* row_flags, double* row_ratio,
                               double* row_u, double* row_zk, double* row_zn) {
  if (!logits || !sp || !draft_tokens || !accept_len || !out_tokens || !next_token) return -1;
  if (vocab <= 0 || ld_logits < vocab) return -2;
  if (dtype != SVREF_F32 && dtype != SVREF_BF16) return -3;
  if (!check_layout(qo_indptr, num_requests, num_rows)) return -2;
  if (draft_probs && ld_q < vocab) return -2;

  for (int32_t r = 0; r < num_requests; ++r) {
    Params prm = request_params(sp, r);
    if (!prm.greedy && !draft_probs) return -1;
  }

  const double nan = std::nan("");
  for (int32_t i = 0; i < num_rows; ++i) {
    out_tokens[i] = -1;
    if (row_flags) row_flags[i] = 0;
    if (row_ratio) row_ratio[i] = nan;
    if (row_u) row_u[i] = nan;
    if (row_zk) row_zk[i] = nan;
    if (row_zn) row_zn[i] = nan;
  }

  RowDist d;
  for (int32_t r = 0; r < num_requests; ++r) {
    const int32_t s = qo_indptr[r], e = qo_indptr[r + 1];
    if (e - s <= 0) {            /* a request with no rows emits nothing */
      accept_len[r] = 0;
      next_token[r] = -1;
      continue;
    }
    const Params prm = request_params(sp, r);
    const int32_t gamma = e - s - 1;
    int32_t cap = gamma;
    if (verify_cap) cap = std::max(0, std::min(verify_cap[r], gamma));
    const uint32_t rid = sp->request_id ? sp->request_id[r] : (uint32_t)r;
    const uint32_t pos0 = sp->position0 ? sp->position0[r] : 0u;

    if ((sp->flags & SVREF_BLOCK_VERIFY) && !prm.greedy) {
      block_verify_request(logits, dtype, ld_logits, vocab, s, cap, draft_tokens, draft_probs,
                           ld_q, prm, sp->seed, rid, pos0, accept_len[r], next_token[r],
                           out_tokens, row_flags, row_ratio, row_u, row_zk, row_zn);
      continue;
    }

    /* O10/O11: test every draft row inside the cap; the first failure ends
     * the accepted prefix. */
    int32_t L = cap;
    bool rejected = false;
    bool bad_draft_at_L = false;
    for (int32_t j = 0; j < cap; ++j) {
      const int32_t i = s + j;
      const int32_t dtok = draft_tokens[i];
      const bool bad = dtok < 0 || dtok >= vocab;
      bool acc = false;
      uint8_t fl = 0;
      if (bad) {
        fl |= SVREF_ROW_BAD_DRAFT;
      } else if (prm.greedy) {
        build_row(logits, dtype, ld_logits, i, vocab, prm, d);
        acc = (dtok == d.a);
      } else {
        build_row(logits, dtype, ld_logits, i, vocab, prm, d);
        if (row_zk) row_zk[i] = d.zk;
        if (row_zn) row_zn[i] = d.zn;
        if (d.near_topp) fl |= SVREF_ROW_NEAR_TOPP;
        double pd = d.p[dtok];
        double q = (double)draft_probs[(int64_t)i * ld_q + dtok];
        double ratio = q > 0.0 ? std::min(1.0, pd / q) : (pd > 0.0 ? 1.0 : 0.0);
        double u = uniform_accept(sp->seed, rid, pos0 + (uint32_t)j);
        acc = u < ratio;
        if (std::fabs(u - ratio) < 1e-5) fl |= SVREF_ROW_NEAR_RATIO;
        if (row_ratio) row_ratio[i] = ratio;
        if (row_u) row_u[i] = u;
      }
      if (acc) fl |= SVREF_ROW_ACCEPT;
      if (row_flags) row_flags[i] = fl;
      if (!acc && !rejected) {
        rejected = true;
        L = j;
        bad_draft_at_L = bad;
      }
    }

    /* The emitted token comes from row s + L: the residual there after a
     * rejection, the target distribution after a full (or capped) accept. */
    const int32_t is = s + L;
    build_row(logits, dtype, ld_logits, is, vocab, prm, d);
    if (!prm.greedy) {
      if (row_zk) row_zk[is] = d.zk;
      if (row_zn) row_zn[is] = d.zn;
    }
    int32_t sample;
    uint8_t sfl = SVREF_ROW_SAMPLED;
    if (prm.greedy) {
      sample = d.a;
    } else {
      const uint32_t pos = pos0 + (uint32_t)L;
      if (d.near_topp) sfl |= SVREF_ROW_NEAR_TOPP;
      RaceResult rr;
      bool use_p = !rejected || bad_draft_at_L;
      if (!use_p) {
        const float* qrow = draft_probs + (int64_t)is * ld_q;
        auto resid = [&](int32_t v) { return std::max(0.0, d.p[v] - (double)qrow[v]); };
        rr = race(d.kept, resid, sp->seed, rid, pos, 1u);
        if (rr.token < 0) {
          use_p = true;
          sfl |= SVREF_ROW_RESID_EMPTY;
        }
      }
      if (use_p) {
        auto pw = [&](int32_t v) { return d.p[v]; };
        rr = race(d.kept, pw, sp->seed, rid, pos, 1u);
      }
      if (rr.near) sfl |= SVREF_ROW_NEAR_RACE;
      sample = rr.token;
    }
    if (row_flags) row_flags[is] |= sfl;

    for (int32_t j = 0; j < L; ++j) out_tokens[s + j] = draft_tokens[s + j];
    out_tokens[is] = sample;
    accept_len[r] = L;
    next_token[r] = sample;
  }
  return 0;
}

int32_t svref_plan_windows(const float* confidence, int64_t ld_conf, int32_t num_requests,
                           int32_t block, int32_t budget, int32_t* verify_len,
                           int32_t* qo_indptr, float* survival) {
  if (!confidence || !verify_len || !qo_indptr) return -1;
  if (num_requests < 0 || block < 0 || (num_requests > 0 && ld_conf < block)) return -2;
  const int32_t R = num_requests, B = block;

  /* Survival: clamp each confidence to [0,1] (NaN -> 0), then a left-to-right
   * fp32 cumulative product per request. */
  std::vector<float> S((size_t)R * B);
  for (int32_t r = 0; r < R; ++r) {
    float acc = 1.0f;
    for (int32_t j = 0; j < B; ++j) {
      float c = confidence[(int64_t)r * ld_conf + j];
      c = (c > 0.0f) ? (c < 1.0f ? c : 1.0f) : 0.0f;
      acc = (j == 0) ? c : acc * c;
      S[(size_t)r * B + j] = acc;
    }
  }
  if (survival)
    for (size_t t = 0; t < S.size(); ++t) survival[t] = S[t];

  /* Global rank by (S desc, j asc, r asc); the first min(budget, R*B) win. */
  struct Item { float s; int32_t j, r; };
  std::vector<Item> items;
  items.reserve(S.size());
  for (int32_t r = 0; r < R; ++r)
    for (int32_t j = 0; j < B; ++j) items.push_back({S[(size_t)r * B + j], j, r});
  std::sort(items.begin(), items.end(), [](const Item& x, const Item& y) {
    if (x.s != y.s) return x.s > y.s;
    if (x.j != y.j) return x.j < y.j;
    return x.r < y.r;
  });
  int64_t take = std::max<int64_t>(0, std::min<int64_t>(budget, (int64_t)R * B));
  for (int32_t r = 0; r < R; ++r) verify_len[r] = 0;
  for (int64_t t = 0; t < take; ++t) verify_len[items[t].r] += 1;

  /* Packed layout: each request submits verify_len + 1 rows (one bonus row). */
  qo_indptr[0] = 0;
  for (int32_t r = 0; r < R; ++r) qo_indptr[r + 1] = qo_indptr[r] + verify_len[r] + 1;
  return 0;
}

int32_t svref_budget_from_costs(const float* confidence, int64_t ld_conf, int32_t num_requests,
                                int32_t block, const float* cost, int32_t ncost,
                                int32_t* budget, double* theta) {
  if (!budget || (num_requests > 0 && block > 0 && !confidence)) return -1;
  if (num_requests < 0 || block < 0 || (num_requests > 0 && ld_conf < block)) return -2;
  const int32_t R = num_requests, B = block;
  const int64_t n = (int64_t)R * B;

  /* The survivals and their rank order, as the planner computes them. */
  std::vector<float> S((size_t)n);
  std::vector<int32_t> vl((size_t)R), qo((size_t)R + 1);
  if (n > 0 && svref_plan_windows(confidence, ld_conf, R, B, 0, vl.data(), qo.data(), S.data()))
    return -2;
  std::vector<std::pair<int32_t, int32_t>> order;  /* (j, r) of each survival */
  order.reserve((size_t)n);
  for (int32_t r = 0; r < R; ++r)
    for (int32_t j = 0; j < B; ++j) order.push_back({j, r});
  std::sort(order.begin(), order.end(), [&](const std::pair<int32_t, int32_t>& x,
                                            const std::pair<int32_t, int32_t>& y) {
    const float sx = S[(size_t)x.second * B + x.first], sy = S[(size_t)y.second * B + y.first];
    if (sx != sy) return sx > sy;
    if (x.first != y.first) return x.first < y.first;
    return x.second < y.second;
  });

  /* No table, or a flat one: no trim. */
  bool flat = true;
  if (cost && ncost > 0) {
    if ((int64_t)ncost < n + R + 1) return -3;
    for (int64_t t = R; t <= n + R; ++t) {
      if (!(cost[t] > 0.0f) || !std::isfinite(cost[t])) return -3;
      if (cost[t] != cost[R]) flat = false;
    }
  }
  if (flat) {
    *budget = (int32_t)n;
    if (theta) {
      double tau = (double)R;
      for (const auto& o : order) tau += (double)S[(size_t)o.second * B + o.first];
      *theta = (cost && ncost > 0) ? tau / (double)cost[n + R] : 0.0;
    }
    return 0;
  }

  /* Global argmax of Theta over every budget; ties to the smaller budget. */
  double tau = (double)R;
  int64_t best_b = 0;
  double best = tau / (double)cost[R];
  for (int64_t b = 1; b <= n; ++b) {
    const auto& o = order[(size_t)(b - 1)];
    tau += (double)S[(size_t)o.second * B + o.first];
    const double th = tau / (double)cost[b + R];
    if (th > best) {
      best = th;
      best_b = b;
    }
  }
  *budget = (int32_t)best_b;
  if (theta) *theta = best;
  return 0;
}

int32_t svref_accept_prefix(const uint8_t* accepted, const int32_t* qo_indptr,
                            int32_t num_requests, const int32_t* verify_cap, int32_t* accept_len) {
  if (!accepted || !qo_indptr || !accept_len || num_requests < 0) return -1;
  for (int32_t r = 0; r < num_requests; ++r) {
    int32_t s = qo_indptr[r], e = qo_indptr[r + 1];
    int32_t gamma = std::max(0, e - s - 1);
    int32_t cap = gamma;
    if (verify_cap) cap = std::max(0, std::min(verify_cap[r], gamma));
    int32_t L = 0;
    while (L < cap && accepted[s + L] != 0) ++L;
    accept_len[r] = L;
  }
  return 0;
}

// Acceptance and trim statistics: each request counted once, each position
// j of its window offered once and accepted when its accepted prefix is
// longer than j.
int32_t svref_acceptance_stats(const int32_t* accept_len, const int32_t* verify_len,
                               int32_t num_requests, int32_t block, int64_t* stats) {
  if (num_requests < 0 || block < 0 || !stats) return -1;
  if (num_requests > 0 && (!accept_len || !verify_len)) return -1;
  const int64_t n = 5 + 2 * (int64_t)block;
  for (int64_t t = 0; t < n; ++t) stats[t] = 0;
  stats[0] = num_requests;
  for (int32_t r = 0; r < num_requests; ++r) {
    const int32_t w = std::min(std::max(verify_len[r], 0), block);
    const int32_t L = std::min(std::max(accept_len[r], 0), w);
    const bool trimmed = w < block;
    if (trimmed) stats[1] += 1;
    if (trimmed && L == w) stats[2] += 1;
    stats[3] += L;
    stats[4] += w;
    for (int32_t j = 0; j < block; ++j) {
      if (w > j) stats[5 + j] += 1;
      if (L > j) stats[5 + block + j] += 1;
    }
  }
  return 0;
}

// ------------------------------------------------------------ estimator
int32_t svref_est_init(svref_estimator* est, int32_t block) {
  if (!est || block < 1 || block > SVREF_EST_MAXB) return -1;
  std::memset(est, 0, sizeof(*est));
  est->block = block;
  est->slope = 0.5;
  for (int32_t k = 0; k < block; ++k) est->bias[k] = -0.2;
  return 0;
}

int32_t svref_est_feature(const float* row_max, const float* row_lse, const float* t_eff,
                          int32_t num_rows, double* x) {
  if (num_rows < 0 || (num_rows > 0 && (!row_max || !row_lse || !t_eff || !x))) return -1;
  for (int32_t i = 0; i < num_rows; ++i) {
    const double T = t_eff[i] > 0.0f ? (double)t_eff[i] : 1.0;
    const double lq = (double)row_max[i] / T - (double)row_lse[i];  // log q_max <= 0
    // logit(q) = log q - log(1 - q)
    double v = lq - std::log1p(-std::exp(lq));
    if (!(v <= 40.0)) v = 40.0;  // q_max = 1 (or NaN) saturates
    if (v < -40.0) v = -40.0;
    x[i] = v;
  }
  return 0;
}

static double sigmoid(double z) { return 1.0 / (1.0 + std::exp(-z)); }

int32_t svref_est_predict(const svref_estimator* est, const double* x, const int32_t* pos,
                          int32_t n, double* p) {
  if (!est || n < 0 || (n > 0 && (!x || !pos || !p))) return -1;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t k = std::min(std::max(pos[i], 0), est->block - 1);
    p[i] = sigmoid(est->slope * x[i] + est->bias[k]);
  }
  return 0;
}

// Newton step of the logistic log-likelihood in (slope, bias_0..bias_{B-1}).
// The Hessian is an arrowhead: a dense slope row and column, a diagonal over
// the intercepts (an observation touches one intercept); with the ridge on the
// diagonal the slope direction is the Schur complement's solution and each
// intercept's direction follows from it.
static void est_refit(svref_estimator* e) {
  const double ridge = 1e-3;
  const int32_t B = e->block;
  double a = e->h_ss + ridge, g = e->g_s;
  for (int32_t k = 0; k < B; ++k) {
    const double d = e->h_kk[k] + ridge;
    a -= e->h_sk[k] * e->h_sk[k] / d;
    g -= e->h_sk[k] * e->g_k[k] / d;
  }
  const double ds = g / a;
  e->last_ds = ds;
  // slope: damped, non-finite dropped, halved while it would turn negative
  double step = ds * (e->n_s / (e->n_s + 50.0));
  if (!std::isfinite(step)) step = 0.0;
  int32_t halvings = 0;
  while (e->slope + step < 0.0 && halvings < 8) {
    step *= 0.5;
    ++halvings;
  }
  if (e->slope + step < 0.0) step = 0.0;
  // intercepts: their Newton step given the slope step taken, damped alike
  for (int32_t k = 0; k < B; ++k) {
    const double d = e->h_kk[k] + ridge;
    const double db = (e->g_k[k] - e->h_sk[k] * step) / d;
    e->last_db[k] = db;
    double sb = db * (e->n_k[k] / (e->n_k[k] + 50.0));
    if (!std::isfinite(sb)) sb = 0.0;
    e->bias[k] += sb;
  }
  e->slope += step;
  e->h_ss = e->g_s = e->n_s = 0.0;
  for (int32_t k = 0; k < B; ++k) e->h_sk[k] = e->h_kk[k] = e->g_k[k] = e->n_k[k] = 0.0;
  e->refits += 1;
}

int32_t svref_est_observe(svref_estimator* est, const double* x, const int32_t* accept_len,
                          const int32_t* verify_len, int32_t num_requests) {
  if (!est || num_requests < 0 || (num_requests > 0 && (!x || !accept_len || !verify_len)))
    return -1;
  const int32_t B = est->block;
  for (int32_t r = 0; r < num_requests; ++r) {
    const int32_t w = std::min(std::max(verify_len[r], 0), B);
    const int32_t L = std::min(std::max(accept_len[r], 0), w);
    const int32_t last = L < w ? L : L - 1;  // the accepted drafts, then the first rejected one
    for (int32_t k = 0; k <= last; ++k) {
      const double xv = x[(size_t)r * B + k];
      const double y = k < L ? 1.0 : 0.0;
      const double p = sigmoid(est->slope * xv + est->bias[k]);
      const double wt = p * (1.0 - p);
      est->h_ss += wt * xv * xv;
      est->h_sk[k] += wt * xv;
      est->h_kk[k] += wt;
      est->g_s += (y - p) * xv;
      est->g_k[k] += y - p;
      est->n_s += 1.0;
      est->n_k[k] += 1.0;
    }
  }
  est->calls += 1;
  if (est->calls >= SVREF_EST_REFIT) {
    est_refit(est);
    est->calls = 0;
  }
  return 0;
}

int32_t svref_sample_probs(const float* probs, int64_t ld_probs, int32_t num_rows, int32_t vocab,
                           const int32_t* qo_indptr, int32_t num_requests,
                           const uint32_t* request_id, const uint32_t* position0, uint64_t seed,
                           uint32_t tag, int32_t* out) {
  if (!probs || !out || vocab <= 0 || ld_probs < vocab) return -1;
  if (!check_layout(qo_indptr, num_requests, num_rows)) return -2;
  std::vector<int32_t> all(vocab);
  std::iota(all.begin(), all.end(), 0);
  for (int32_t r = 0; r < num_requests; ++r) {
    uint32_t rid = request_id ? request_id[r] : (uint32_t)r;
    uint32_t pos0 = position0 ? position0[r] : 0u;
    for (int32_t i = qo_indptr[r]; i < qo_indptr[r + 1]; ++i) {
      const float* row = probs + (int64_t)i * ld_probs;
      auto wfn = [&](int32_t v) { return (double)row[v]; };
      RaceResult rr = race(all, wfn, seed, rid, pos0 + (uint32_t)(i - qo_indptr[r]), tag);
      out[i] = rr.token;
    }
  }
  return 0;
}

}  // extern "C"
