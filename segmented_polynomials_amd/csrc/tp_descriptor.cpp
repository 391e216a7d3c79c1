#include "tp_descriptor.hpp"

#include <algorithm>
#include <cstdlib>
#include <set>
#include <stdexcept>

#include "cg.hpp"

namespace segpoly {

int64_t TPDescriptor::cg_nnz() const {
  int64_t n = 0;
  for (const auto& p : paths) n += static_cast<int64_t>(p.nz.size());
  return n;
}

TPDescriptor build_tp(const std::string& s1, const std::string& s2, const std::string& so, bool merge) {
  TPDescriptor d;
  d.merged = merge;
  d.in1 = parse_irreps(s1);
  d.in2 = parse_irreps(s2);
  std::vector<Irrep> filt = parse_irreps(so);
  for (const auto& r : filt)
    if (r.l > kMaxL) throw std::invalid_argument("output filter has l above the supported maximum");
  for (const auto& r : d.in2)
    if (r.mul != 1) throw std::invalid_argument("input 2 must have multiplicity 1 per block");
  for (const auto& r : d.in1)
    if (r.l > kMaxL) throw std::invalid_argument("input 1 has l above the supported maximum");
  for (const auto& r : d.in2)
    if (r.l > kMaxL) throw std::invalid_argument("input 2 has l above the supported maximum");
  std::set<std::pair<int, int>> keep;
  for (const auto& r : filt) keep.insert({r.l, r.p});

  std::vector<int64_t> off1(d.in1.size()), off2(d.in2.size());
  std::vector<int> xcomp(d.in1.size());
  int64_t o = 0;
  int c = 0;
  for (size_t i = 0; i < d.in1.size(); ++i) {
    off1[i] = o;
    xcomp[i] = c;
    o += d.in1[i].mul * (2 * d.in1[i].l + 1);
    c += 2 * d.in1[i].l + 1;
  }
  d.dim1 = o;
  d.nx = c;
  o = 0;
  for (size_t j = 0; j < d.in2.size(); ++j) {
    off2[j] = o;
    o += 2 * d.in2[j].l + 1;
  }
  d.dim2 = o;

  std::vector<TPPath> paths;
  for (size_t i = 0; i < d.in1.size(); ++i)
    for (size_t j = 0; j < d.in2.size(); ++j) {
      const int l1 = d.in1[i].l, l2 = d.in2[j].l;
      for (int lo = std::abs(l1 - l2); lo <= l1 + l2; ++lo) {
        const int po = d.in1[i].p * d.in2[j].p;
        if (!keep.count({lo, po})) continue;
        TPPath p{};
        p.b1 = static_cast<int>(i);
        p.b2 = static_cast<int>(j);
        p.l1 = l1;
        p.l2 = l2;
        p.lo = lo;
        p.po = po;
        p.mul = d.in1[i].mul;
        p.off1 = off1[i];
        p.off2 = off2[j];
        p.xcomp = xcomp[i];
        paths.push_back(p);
      }
    }
  std::stable_sort(paths.begin(), paths.end(), [](const TPPath& a, const TPPath& b) {
    return type_rank(a.lo, a.po) < type_rank(b.lo, b.po);
  });
  int64_t oo = 0, wo = 0;
  int kc = 0;
  std::vector<int> type_first;  // merged: the first path of each output type
  for (size_t pi = 0; pi < paths.size(); ++pi) {
    TPPath& p = paths[pi];
    p.woff = wo;
    wo += p.mul;
    int same = -1;
    if (merge)
      for (int f : type_first)
        if (paths[f].lo == p.lo && paths[f].po == p.po) same = f;
    if (same >= 0) {  // one block per type: share the first path's block
      if (paths[same].mul != p.mul)
        throw std::invalid_argument("merged paths of one output type need one multiplicity");
      p.offo = paths[same].offo;
      p.kcomp = paths[same].kcomp;
    } else {
      p.offo = oo;
      p.kcomp = kc;
      oo += static_cast<int64_t>(p.mul) * (2 * p.lo + 1);
      kc += 2 * p.lo + 1;
      type_first.push_back(static_cast<int>(pi));
      d.out.push_back({p.mul, p.lo, p.po});
    }
    const auto& cg = real_cg(p.l1, p.l2, p.lo);
    const int d1 = 2 * p.l1 + 1, d2 = 2 * p.l2 + 1, d3 = 2 * p.lo + 1;
    for (int k = 0; k < d3; ++k)
      for (int i = 0; i < d1; ++i)
        for (int j = 0; j < d2; ++j) {
          double v = cg[(static_cast<size_t>(i) * d2 + j) * d3 + k];
          if (v != 0.0) p.nz.push_back({i, j, k, v});
        }
  }
  d.dimo = oo;
  d.numel = wo;
  d.nk = kc;
  d.paths = std::move(paths);

  d.uniform_mul = !d.in1.empty();
  d.mul = d.in1.empty() ? 0 : d.in1[0].mul;
  for (const auto& r : d.in1)
    if (r.mul != d.mul) d.uniform_mul = false;

  // structure key: input types and the realised path list
  std::string key = "tp:";
  for (const auto& r : d.in1) key += type_str(r.l, r.p) + ",";
  key += "|";
  for (const auto& r : d.in2) key += type_str(r.l, r.p) + ",";
  key += "|";
  for (const auto& p : d.paths)
    key += std::to_string(p.b1) + "." + std::to_string(p.b2) + "." + std::to_string(p.lo) + ",";
  if (merge) key += "|merged";
  d.key = key;
  return d;
}

}  // namespace segpoly
