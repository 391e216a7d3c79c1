#include "cg.hpp"

#include <cmath>
#include <complex>
#include <cstdlib>
#include <map>
#include <mutex>
#include <tuple>

namespace segpoly {

namespace {

using ld = long double;
using cld = std::complex<long double>;

ld factorial(int n) {
  static ld table[64];
  static bool init = false;
  if (!init) {
    table[0] = 1.0L;
    for (int i = 1; i < 64; ++i) table[i] = table[i - 1] * i;
    init = true;
  }
  return table[n];
}

// <l1 m1 l2 m2 | l3 m3>, Racah's closed formula.
ld cg_complex(int l1, int m1, int l2, int m2, int l3, int m3) {
  if (m1 + m2 != m3) return 0.0L;
  if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return 0.0L;
  if (std::abs(m1) > l1 || std::abs(m2) > l2 || std::abs(m3) > l3) return 0.0L;
  ld pre = (2 * l3 + 1) * factorial(l3 + l1 - l2) * factorial(l3 - l1 + l2) *
           factorial(l1 + l2 - l3) / factorial(l1 + l2 + l3 + 1);
  pre *= factorial(l3 + m3) * factorial(l3 - m3) * factorial(l1 - m1) * factorial(l1 + m1) *
         factorial(l2 - m2) * factorial(l2 + m2);
  ld sum = 0.0L;
  for (int k = 0; k <= l1 + l2 - l3; ++k) {
    int d[6] = {k, l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k};
    bool ok = true;
    ld den = 1.0L;
    for (int t : d) {
      if (t < 0) { ok = false; break; }
      den *= factorial(t);
    }
    if (!ok) continue;
    sum += ((k % 2) ? -1.0L : 1.0L) / den;
  }
  return std::sqrt(pre) * sum;
}

// Q[m, mu] of the complex -> real change of basis.
cld q_entry(int m, int mu) {
  const ld s = 1.0L / std::sqrt(2.0L);
  const ld sgn = (std::abs(m) % 2) ? -1.0L : 1.0L;  // (-1)^m
  if (m == 0) return mu == 0 ? cld(1.0L, 0.0L) : cld(0.0L, 0.0L);
  if (m < 0) {
    if (mu == m) return cld(0.0L, s);
    if (mu == -m) return cld(0.0L, -s * sgn);
    return cld(0.0L, 0.0L);
  }
  if (mu == -m) return cld(s, 0.0L);
  if (mu == m) return cld(s * sgn, 0.0L);
  return cld(0.0L, 0.0L);
}

std::vector<double> build(int l1, int l2, int l3) {
  const int d1 = 2 * l1 + 1, d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
  std::vector<double> out(static_cast<size_t>(d1) * d2 * d3, 0.0);
  if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return out;
  std::vector<cld> t(out.size());
  for (int m1 = -l1; m1 <= l1; ++m1)
    for (int m2 = -l2; m2 <= l2; ++m2)
      for (int m3 = -l3; m3 <= l3; ++m3) {
        cld acc(0.0L, 0.0L);
        int mu1s[2] = {m1, -m1}, mu2s[2] = {m2, -m2};
        for (int a = 0; a < (m1 == 0 ? 1 : 2); ++a)
          for (int b = 0; b < (m2 == 0 ? 1 : 2); ++b) {
            int mu1 = mu1s[a], mu2 = mu2s[b], mu3 = mu1 + mu2;
            if (std::abs(mu3) != std::abs(m3)) continue;
            ld c = cg_complex(l1, mu1, l2, mu2, l3, mu3);
            if (c == 0.0L) continue;
            acc += std::conj(q_entry(m1, mu1)) * std::conj(q_entry(m2, mu2)) * q_entry(m3, mu3) * c;
          }
        t[(static_cast<size_t>(m1 + l1) * d2 + (m2 + l2)) * d3 + (m3 + l3)] = acc;
      }
  ld max_re = 0.0L, max_im = 0.0L;
  for (const auto& v : t) {
    max_re = std::max(max_re, std::fabs(v.real()));
    max_im = std::max(max_im, std::fabs(v.imag()));
  }
  const bool use_re = max_re >= max_im;
  double amax = 0.0;
  for (size_t i = 0; i < t.size(); ++i) {
    ld v = use_re ? t[i].real() : t[i].imag();
    // residues of cancelled long-double sums are ~1e-19: exactly zero
    out[i] = (std::fabs(v) < 1e-14L) ? 0.0 : static_cast<double>(v);
    amax = std::max(amax, std::fabs(out[i]));
  }
  double ref = 0.0;
  if ((l1 + l2 + l3) % 2 == 0) {
    ref = out[(static_cast<size_t>(l1) * d2 + l2) * d3 + l3];
  } else {
    for (double v : out)
      if (std::fabs(v) > 1e-9 * amax) { ref = v; break; }
  }
  if (ref < 0)
    for (double& v : out) v = -v;
  return out;
}

}  // namespace

const std::vector<double>& real_cg(int l1, int l2, int l3) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, std::vector<double>> cache;
  std::lock_guard<std::mutex> g(mu);
  auto key = std::make_tuple(l1, l2, l3);
  auto it = cache.find(key);
  if (it == cache.end()) it = cache.emplace(key, build(l1, l2, l3)).first;
  return it->second;
}

}  // namespace segpoly
