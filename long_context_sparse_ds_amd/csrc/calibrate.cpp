// Offline label-channel calibration (CPU).
//
// Double Sparsity page, method details and abstract: the channel-sparsity
// pattern is close to static, so it is fixed once, offline, from a small
// calibration set, and reused at every decode step.  The page does not state
// the rule.  Here channel c of KV head g is scored by
//   mean over calibration queries n and the group's query heads h of |q[n,h,c]|
//   times mean over calibration keys n of |k[g,n,c]|,
// which is the mean of |q_c| * |k_c| over every query/key pair.  The r best
// channels are kept (the lower id wins a tie) and written in ascending order.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <string>
#include <vector>

#include "ds.h"

namespace ds {
void set_error(const char* msg);
}

extern "C" ds_status ds_calibrate_channels(const float* q_cal, int64_t n_q, const float* k_cal, int64_t n_k,
                                           int32_t Hq, int32_t Hkv, int32_t d, int32_t r, int32_t* channels_out) {
  if (!q_cal || !k_cal || !channels_out) {
    ds::set_error("null pointer argument");
    return DS_ERR_INVALID_ARGUMENT;
  }
  if (n_q < 1 || n_k < 1 || Hq < 1 || Hkv < 1 || d < 1) {
    ds::set_error("n_q, n_k, Hq, Hkv, d must be >= 1");
    return DS_ERR_INVALID_ARGUMENT;
  }
  if (Hq % Hkv != 0) {
    ds::set_error("Hq must be a multiple of Hkv");
    return DS_ERR_INVALID_ARGUMENT;
  }
  if (r < 1 || r > d) {
    ds::set_error("need 1 <= r <= d");
    return DS_ERR_INVALID_ARGUMENT;
  }
  ds::set_error("");
  const int G = Hq / Hkv;
  std::vector<double> a(d), b(d), s(d);
  std::vector<int32_t> order(d), result(size_t(Hkv) * r);
  for (int g = 0; g < Hkv; ++g) {
    std::fill(a.begin(), a.end(), 0.0);
    std::fill(b.begin(), b.end(), 0.0);
    for (int64_t n = 0; n < n_q; ++n)
      for (int h = g * G; h < (g + 1) * G; ++h) {
        const float* row = q_cal + (n * Hq + h) * int64_t(d);
        for (int c = 0; c < d; ++c) a[c] += std::fabs(double(row[c]));
      }
    for (int64_t n = 0; n < n_k; ++n) {
      const float* row = k_cal + (int64_t(g) * n_k + n) * d;
      for (int c = 0; c < d; ++c) b[c] += std::fabs(double(row[c]));
    }
    const double inv_q = 1.0 / double(n_q * G), inv_k = 1.0 / double(n_k);
    for (int c = 0; c < d; ++c) s[c] = (a[c] * inv_q) * (b[c] * inv_k);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return s[x] > s[y]; });
    std::sort(order.begin(), order.begin() + r);
    std::copy(order.begin(), order.begin() + r, result.begin() + size_t(g) * r);
  }
  std::copy(result.begin(), result.end(), channels_out);
  return DS_OK;
}
