// Host driver that runs every entry point of the CPU oracle on small seeded
// inputs, edge cases included (empty requests, a bonus-only request, -inf
// logits, out-of-range drafts, verify caps below zero and past the window,
// V = 1, P <= 0, NaN confidences, invalid cost tables).  It is built together
// with oracle/svref.cpp under AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_oracle_sanitize.py; any memory error or undefined operation
// aborts the process.  It checks no values: the pin tests do that.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "svref.h"

namespace {

std::mt19937_64 rng(12345);

float normal(float s) {
  std::normal_distribution<float> d(0.0f, s);
  return d(rng);
}

int uniform_int(int lo, int hi) {
  std::uniform_int_distribution<int> d(lo, hi);
  return d(rng);
}

uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int run_case(int V, int R, bool bf16, bool with_inf) {
  std::vector<int32_t> rows_per(R);
  for (int r = 0; r < R; ++r) rows_per[r] = uniform_int(0, 5);  // 0: no rows at all
  std::vector<int32_t> qo(R + 1, 0);
  for (int r = 0; r < R; ++r) qo[r + 1] = qo[r] + rows_per[r];
  const int rows = qo[R];
  // buffers hold at least one element so an empty batch still passes non-NULL
  // pointers (the oracle rejects NULL inputs)
  const size_t n1 = rows > 0 ? (size_t)rows : 1;
  std::vector<float> xf(n1 * V);
  for (auto& v : xf) v = normal(3.0f);
  if (with_inf)
    for (size_t t = 0; t < xf.size(); t += 5) xf[t] = -std::numeric_limits<float>::infinity();
  std::vector<uint16_t> xb(xf.size());
  for (size_t t = 0; t < xf.size(); ++t) xb[t] = to_bf16(xf[t]);
  const void* logits = bf16 ? (const void*)xb.data() : (const void*)xf.data();
  const int dt = bf16 ? SVREF_BF16 : SVREF_F32;

  std::vector<float> T(R), P(R);
  std::vector<int32_t> k(R), cap(R);
  std::vector<uint32_t> rid(R), pos0(R);
  const float Ps[] = {1.0f, 0.9f, 0.5f, 0.0f, -1.0f, 2.0f};
  for (int r = 0; r < R; ++r) {
    T[r] = uniform_int(0, 3) == 0 ? 0.0f : 0.3f + 0.1f * (float)uniform_int(0, 10);
    k[r] = uniform_int(-1, V + 1);
    P[r] = Ps[uniform_int(0, 5)];
    cap[r] = uniform_int(-2, 7);
    rid[r] = (uint32_t)r * 7u;
    pos0[r] = (uint32_t)uniform_int(0, 4096);
  }
  svref_sampling sp = {T.data(), k.data(), P.data(), rid.data(), pos0.data(), 99u, 0u};

  const int kmax = V < 16 ? V : 16;
  std::vector<double> probs(n1 * V), rmax(n1), rlse(n1), zn(n1), zk(n1);
  std::vector<int32_t> am(n1), kc(n1), kidx(n1 * kmax), lo(n1), hi(n1), oidx(n1 * kmax);
  std::vector<uint8_t> fl(n1);
  int rc = svref_build_target_probs(logits, dt, V, rows, V, qo.data(), R, &sp, probs.data(), V,
                                    rmax.data(), am.data(), rlse.data(), kc.data(), kidx.data(),
                                    kmax, zn.data(), fl.data(), zk.data(), lo.data(), hi.data(),
                                    oidx.data());
  if (rc) return rc;

  // draft distributions from draft logits, then drafts sampled from them
  std::vector<float> xd(xf.size());
  for (size_t t = 0; t < xd.size(); ++t) xd[t] = xf[t] + normal(1.0f);
  std::vector<double> qd(n1 * V);
  rc = svref_build_target_probs(xd.data(), SVREF_F32, V, rows, V, qo.data(), R, &sp, qd.data(), V,
                                nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr);
  if (rc) return rc;
  std::vector<float> q(qd.size());
  for (size_t t = 0; t < q.size(); ++t) q[t] = (float)qd[t];
  std::vector<int32_t> drafts(n1);
  rc = svref_sample_probs(q.data(), V, rows, V, qo.data(), R, rid.data(), pos0.data(), 99u, 2u,
                          drafts.data());
  if (rc) return rc;
  for (int i = 0; i < rows; i += 4) drafts[i] = (i % 8 == 0) ? -1 : V + 3;  // out of range

  std::vector<int32_t> L(R), out(n1), next(R);
  std::vector<double> ratio(n1), u(n1), vzk(n1), vzn(n1);
  for (int with_cap = 0; with_cap < 2; ++with_cap) {
    rc = svref_rejection_sample(logits, dt, V, V, qo.data(), R, rows, drafts.data(), q.data(), V,
                                with_cap ? cap.data() : nullptr, &sp, L.data(), out.data(),
                                next.data(), fl.data(), ratio.data(), u.data(), vzk.data(),
                                vzn.data());
    if (rc) return rc;
  }
  std::vector<uint8_t> acc(n1);
  for (int i = 0; i < rows; ++i) acc[i] = (uint8_t)(fl[i] & SVREF_ROW_ACCEPT);
  rc = svref_accept_prefix(acc.data(), qo.data(), R, cap.data(), L.data());
  return rc;
}

int run_planner(int R, int B) {
  const size_t n1 = R * B > 0 ? (size_t)R * B : 1;  // non-NULL buffers for empty sizes
  std::vector<float> conf(n1);
  for (auto& c : conf) c = 0.1f * (float)uniform_int(-2, 12);
  conf[0] = std::numeric_limits<float>::quiet_NaN();
  std::vector<int32_t> vl(R > 0 ? R : 1), qo(R + 1);
  std::vector<float> surv(n1);
  const int budgets[] = {-3, 0, 1, R * B / 2, R * B, R * B + 4};
  for (int b : budgets) {
    int rc = svref_plan_windows(conf.data(), B, R, B, b, vl.data(), qo.data(), surv.data());
    if (rc) return rc;
  }
  std::vector<float> cost((size_t)R * B + R + 1);
  for (size_t t = 0; t < cost.size(); ++t) cost[t] = 1.0f + (float)(t / 5);
  int32_t budget = 0;
  double theta = 0.0;
  int rc = svref_budget_from_costs(conf.data(), B, R, B, cost.data(), (int32_t)cost.size(), &budget,
                                   &theta);
  if (rc) return rc;
  rc = svref_budget_from_costs(conf.data(), B, R, B, nullptr, 0, &budget, &theta);
  if (rc) return rc;
  if (!cost.empty()) {  // an invalid table is reported, not read past
    cost.back() = -1.0f;
    if (svref_budget_from_costs(conf.data(), B, R, B, cost.data(), (int32_t)cost.size(), &budget,
                                &theta) != -3)
      return -100;
    if (svref_budget_from_costs(conf.data(), B, R, B, cost.data(), 1, &budget, &theta) != -3 &&
        R * B + R + 1 > 1)
      return -101;
  }
  std::vector<int32_t> L(R > 0 ? R : 1);
  for (int r = 0; r < R; ++r) L[r] = uniform_int(-2, B + 2);
  std::vector<int64_t> stats(5 + 2 * (size_t)B);
  rc = svref_acceptance_stats(L.data(), vl.data(), R, B, stats.data());
  if (rc) return rc;
  if (B >= 1 && B <= SVREF_EST_MAXB) {
    svref_estimator est;
    rc = svref_est_init(&est, B);
    if (rc) return rc;
    std::vector<float> m(n1), lse(n1), t(n1);
    for (size_t i = 0; i < m.size(); ++i) {
      m[i] = normal(4.0f);
      lse[i] = m[i] + 0.5f * (float)uniform_int(0, 6);
      t[i] = (float)uniform_int(0, 2) * 0.5f;
    }
    std::vector<double> x(n1), p(n1);
    std::vector<int32_t> pos(n1);
    for (size_t i = 0; i < pos.size(); ++i) pos[i] = (int32_t)(i % (size_t)B);
    rc = svref_est_feature(m.data(), lse.data(), t.data(), R * B, x.data());
    if (rc) return rc;
    for (int c = 0; c < SVREF_EST_REFIT + 3; ++c) {
      rc = svref_est_predict(&est, x.data(), pos.data(), R * B, p.data());
      if (rc) return rc;
      rc = svref_est_observe(&est, x.data(), L.data(), vl.data(), R);
      if (rc) return rc;
    }
  }
  return 0;
}

}  // namespace

int main() {
  const int Vs[] = {1, 2, 3, 17, 64, 301};
  for (int V : Vs)
    for (int R : {1, 3, 9})
      for (int bf16 = 0; bf16 < 2; ++bf16)
        for (int inf = 0; inf < 2; ++inf) {
          const int rc = run_case(V, R, bf16 != 0, inf != 0);
          if (rc) {
            std::printf("case V=%d R=%d bf16=%d inf=%d failed: %d\n", V, R, bf16, inf, rc);
            return 1;
          }
        }
  for (int R : {0, 1, 5, 40})
    for (int B : {0, 1, 4, 16}) {
      const int rc = run_planner(R, B);
      if (rc) {
        std::printf("planner R=%d B=%d failed: %d\n", R, B, rc);
        return 1;
      }
    }
  std::printf("sanitized oracle run: ok\n");
  return 0;
}
