#include "symcon_descriptor.hpp"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <numeric>
#include <set>
#include <tuple>
#include <stdexcept>

#include "cg.hpp"

namespace segpoly {

int64_t SymconDescriptor::num_terms() const {
  int64_t t = 0;
  for (const auto& c : couplings) t += static_cast<int64_t>(c.terms.size());
  return t;
}

int64_t SymconDescriptor::num_monomial_products() const {
  std::set<std::pair<int, int>> pairs;
  std::set<std::tuple<int, int, int>> triples;
  for (const auto& c : couplings)
    for (const auto& t : c.terms) {
      if (t.m[1] >= 0) pairs.insert({t.m[0], t.m[1]});
      if (t.m[2] >= 0) triples.insert({t.m[0], t.m[1], t.m[2]});
    }
  return static_cast<int64_t>(pairs.size() + triples.size());
}

namespace {

constexpr int kSymconMaxL = 6;

double cg_at(int l1, int l2, int l3, int i, int j, int k) {
  const auto& t = real_cg(l1, l2, l3);
  return t[(static_cast<size_t>(i) * (2 * l2 + 1) + j) * (2 * l3 + 1) + k];
}

// Symmetrise a tensor [n]^nu x [dL] over the nu input slots.
std::vector<double> symmetrize(const std::vector<double>& t, int n, int nu, int dL) {
  std::vector<double> s(t.size(), 0.0);
  std::vector<int> perm(nu);
  std::iota(perm.begin(), perm.end(), 0);
  int nperm = 0;
  std::vector<int> idx(nu), pidx(nu);
  const size_t slots = t.size() / dL;
  do {
    ++nperm;
    for (size_t flat = 0; flat < slots; ++flat) {
      size_t r = flat;
      for (int a = nu - 1; a >= 0; --a) {
        idx[a] = static_cast<int>(r % n);
        r /= n;
      }
      // s[idx] += t[idx permuted]: result(i_0..i_{nu-1}) = t(i_perm(0) ...)
      size_t src = 0;
      for (int a = 0; a < nu; ++a) src = src * n + idx[perm[a]];
      for (int M = 0; M < dL; ++M) s[flat * dL + M] += t[src * dL + M];
    }
  } while (std::next_permutation(perm.begin(), perm.end()));
  for (double& v : s) v /= nperm;
  return s;
}

double dot(const std::vector<double>& a, const std::vector<double>& b) {
  long double s = 0.0L;
  for (size_t i = 0; i < a.size(); ++i) s += static_cast<long double>(a[i]) * b[i];
  return static_cast<double>(s);
}

int distinct_orderings(const int* m, int nu) {
  if (nu == 1) return 1;
  if (nu == 2) return m[0] == m[1] ? 1 : 2;
  if (m[0] == m[1] && m[1] == m[2]) return 1;
  if (m[0] == m[1] || m[1] == m[2]) return 3;
  return 6;
}

}  // namespace

SymconDescriptor build_symcon(const std::string& s_in, const std::string& s_out,
                              const std::vector<int>& degrees) {
  SymconDescriptor d;
  d.in = parse_irreps(s_in);
  d.out = parse_irreps(s_out);
  d.degrees = degrees;
  if (d.in.empty() || d.out.empty()) throw std::invalid_argument("empty irreps");
  d.mul = d.in[0].mul;
  for (const auto& r : d.in)
    if (r.mul != d.mul) throw std::invalid_argument("symmetric contraction needs uniform multiplicities");
  for (const auto& r : d.out)
    if (r.mul != d.mul) throw std::invalid_argument("symmetric contraction needs uniform multiplicities");
  for (const auto& r : d.in)
    if (r.l > kSymconMaxL) throw std::invalid_argument("input l above the supported maximum");
  for (const auto& r : d.out)
    if (r.l > kSymconMaxL) throw std::invalid_argument("output l above the supported maximum");
  for (int nu : degrees)
    if (nu < 1 || nu > 3) throw std::invalid_argument("degrees must be within 1..3");

  int c = 0;
  for (const auto& r : d.in) {
    d.in_comp.push_back(c);
    c += 2 * r.l + 1;
  }
  d.n = c;
  c = 0;
  for (const auto& r : d.out) {
    d.out_comp.push_back(c);
    c += 2 * r.l + 1;
  }
  d.nout = c;
  d.dim_in = irreps_dim(d.in);
  d.dim_out = irreps_dim(d.out);
  const int n = d.n, nb = static_cast<int>(d.in.size());

  for (int nu : degrees) {
    size_t slots = 1;
    for (int a = 0; a < nu; ++a) slots *= n;
    for (size_t ob = 0; ob < d.out.size(); ++ob) {
      const int L = d.out[ob].l, pL = d.out[ob].p, dL = 2 * L + 1;
      std::vector<std::vector<double>> ortho;
      int k = 0;
      auto consider = [&](std::vector<double>& t) {
        std::vector<double> s = symmetrize(t, n, nu, dL);
        double ns = std::sqrt(dot(s, s));
        if (ns < 1e-12) return;
        std::vector<double> r = s;
        for (const auto& q : ortho) {
          double a = dot(q, r);
          for (size_t i = 0; i < r.size(); ++i) r[i] -= a * q[i];
        }
        double nr = std::sqrt(dot(r, r));
        if (nr <= 1e-8 * ns) return;
        for (double& v : r) v /= nr;
        ortho.push_back(std::move(r));
        SymconCoupling cp;
        cp.nu = nu;
        cp.ob = static_cast<int>(ob);
        cp.k = k++;
        cp.L = L;
        const double scale = std::sqrt(static_cast<double>(dL)) / ns;
        cp.dense.resize(s.size());
        for (size_t i = 0; i < s.size(); ++i) cp.dense[i] = s[i] * scale;
        d.couplings.push_back(std::move(cp));
      };
      std::vector<int> tup(nu, 0);
      while (true) {
        int par = 1;
        for (int b : tup) par *= d.in[b].p;
        if (par == pL) {
          if (nu == 1) {
            if (d.in[tup[0]].l == L) {
              std::vector<double> t(slots * dL, 0.0);
              for (int M = 0; M < dL; ++M) t[static_cast<size_t>(d.in_comp[tup[0]] + M) * dL + M] = 1.0;
              consider(t);
            }
          } else if (nu == 2) {
            const int l1 = d.in[tup[0]].l, l2 = d.in[tup[1]].l;
            if (std::abs(l1 - l2) <= L && L <= l1 + l2) {
              std::vector<double> t(slots * dL, 0.0);
              for (int i = 0; i < 2 * l1 + 1; ++i)
                for (int j = 0; j < 2 * l2 + 1; ++j)
                  for (int M = 0; M < dL; ++M)
                    t[(static_cast<size_t>(d.in_comp[tup[0]] + i) * n + d.in_comp[tup[1]] + j) * dL + M] =
                        cg_at(l1, l2, L, i, j, M);
              consider(t);
            }
          } else {
            const int l1 = d.in[tup[0]].l, l2 = d.in[tup[1]].l, l3 = d.in[tup[2]].l;
            for (int l12 = std::abs(l1 - l2); l12 <= l1 + l2; ++l12) {
              if (!(std::abs(l12 - l3) <= L && L <= l12 + l3)) continue;
              std::vector<double> t(slots * dL, 0.0);
              for (int i = 0; i < 2 * l1 + 1; ++i)
                for (int j = 0; j < 2 * l2 + 1; ++j)
                  for (int kk = 0; kk < 2 * l3 + 1; ++kk)
                    for (int M = 0; M < dL; ++M) {
                      long double v = 0.0L;
                      for (int a = 0; a < 2 * l12 + 1; ++a)
                        v += static_cast<long double>(cg_at(l1, l2, l12, i, j, a)) * cg_at(l12, l3, L, a, kk, M);
                      t[((static_cast<size_t>(d.in_comp[tup[0]] + i) * n + d.in_comp[tup[1]] + j) * n +
                         d.in_comp[tup[2]] + kk) * dL + M] = static_cast<double>(v);
                    }
              consider(t);
            }
          }
        }
        // next tuple in lexicographic order
        int a = nu - 1;
        while (a >= 0 && tup[a] == nb - 1) tup[a--] = 0;
        if (a < 0) break;
        ++tup[a];
      }
    }
  }
  // weight-segment order is nu, then output block, then k: the loops above
  // already produce it
  d.numel = static_cast<int64_t>(d.couplings.size()) * d.mul;

  for (auto& cp : d.couplings) {
    const int nu = cp.nu, dL = 2 * cp.L + 1;
    auto emit = [&](int m0, int m1, int m2) {
      int m[3] = {m0, m1, m2};
      size_t flat = 0;
      for (int a = 0; a < nu; ++a) flat = flat * n + m[a];
      for (int M = 0; M < dL; ++M) {
        double v = cp.dense[flat * dL + M];
        if (std::fabs(v) <= 1e-12) continue;
        cp.terms.push_back({{m0, m1, m2}, M, v * distinct_orderings(m, nu)});
      }
    };
    for (int m0 = 0; m0 < n; ++m0) {
      if (nu == 1) {
        emit(m0, -1, -1);
        continue;
      }
      for (int m1 = m0; m1 < n; ++m1) {
        if (nu == 2) {
          emit(m0, m1, -1);
          continue;
        }
        for (int m2 = m1; m2 < n; ++m2) emit(m0, m1, m2);
      }
    }
  }

  std::string key = "symcon:";
  for (const auto& r : d.in) key += type_str(r.l, r.p) + ",";
  key += "|";
  for (const auto& r : d.out) key += type_str(r.l, r.p) + ",";
  key += "|";
  for (int nu : degrees) key += std::to_string(nu) + ",";
  d.key = key;
  return d;
}

}  // namespace segpoly
