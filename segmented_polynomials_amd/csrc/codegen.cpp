// Build-time generator of the specialised kernels.
//
// Reads a list of descriptors (specs.txt) and, for each, writes one HIP
// translation unit with a struct whose device functions carry the coupling
// coefficients of that descriptor as literal constants ("known at compile
// time and mostly zero", e3nn-course Lesson 12a, section 21.1), plus a
// registry mapping each descriptor's structure key to its launcher.  The
// kernel skeletons themselves are hand-written (kernels/*.hpp); only the
// per-descriptor arithmetic is emitted here.
//
// Spec lines:
//   tp     NAME DTYPES | IRREPS_IN1 | IRREPS_IN2 | IRREPS_OUT_FILTER
//   symcon NAME DTYPES | IRREPS_IN | IRREPS_OUT | DEGREES
// DTYPES is f32, f64 or f32,f64.  Multiplicities in the strings only fix the
// structure; the kernels take the multiplicity at run time.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <iostream>
#include <map>
#include <set>
#include <sstream>
#include <string>
#include <tuple>
#include <vector>

#include "symcon_descriptor.hpp"
#include "tp_descriptor.hpp"

using namespace segpoly;

namespace {

std::string lit(double v) {
  char buf[64];
  std::snprintf(buf, sizeof buf, "T(%.17g)", v);
  return buf;
}

std::string trim(const std::string& s) {
  size_t a = s.find_first_not_of(" \t\r\n");
  size_t b = s.find_last_not_of(" \t\r\n");
  return a == std::string::npos ? "" : s.substr(a, b - a + 1);
}

std::vector<std::string> split(const std::string& s, char c) {
  std::vector<std::string> out;
  std::stringstream ss(s);
  std::string item;
  while (std::getline(ss, item, c)) out.push_back(trim(item));
  return out;
}

unsigned dtype_mask(const std::string& s) {
  unsigned m = 0;
  for (const auto& t : split(s, ',')) {
    if (t == "f32") m |= 1u;
    else if (t == "f64") m |= 2u;
    else throw std::runtime_error("bad dtype list " + s);
  }
  return m;
}

// ---------------------------------------------------------------- TP

struct QTable {
  // uniform coefficient products q[n] = |c| * sh[j]; |c| == 1 -> raw sh
  std::map<std::pair<uint64_t, int>, int> index;
  std::vector<std::pair<double, int>> entries;
  int get(double absc, int j) {
    uint64_t bits;
    std::memcpy(&bits, &absc, sizeof bits);
    auto key = std::make_pair(bits, j);
    auto it = index.find(key);
    if (it != index.end()) return it->second;
    int id = static_cast<int>(entries.size());
    index[key] = id;
    entries.push_back({absc, j});
    return id;
  }
};

bool is_identity_l2_zero(const TPPath& p) {
  if (p.l2 != 0 || p.l1 != p.lo) return false;
  for (const auto& e : p.nz)
    if (e.c != 1.0 || e.i != e.k || e.j != 0) return false;
  return static_cast<int>(p.nz.size()) == 2 * p.l1 + 1;
}

bool is_identity_l1_zero(const TPPath& p) {
  if (p.l1 != 0 || p.l2 != p.lo) return false;
  for (const auto& e : p.nz)
    if (e.c != 1.0 || e.j != e.k || e.i != 0) return false;
  return static_cast<int>(p.nz.size()) == 2 * p.l2 + 1;
}

// Per-path body: `qn(absc, j)` names the uniform product |c| * sh_j, `X(i)`,
// `W()`, `A(k)` name input-1 component i of the path's block, the path's
// weight and output component k of the path's block.
template <class QN, class XN, class WN, class AN>
void emit_path_body(const TPPath& p, QN qn, XN X, WN W, AN A, const std::string& ind, std::ostream& e) {
  if (is_identity_l2_zero(p)) {
    e << ind << "const T ws = " << W() << " * " << qn(1.0, 0) << ";\n";
    for (int k = 0; k < 2 * p.lo + 1; ++k) e << ind << A(k) << " = fmadd(ws, " << X(k) << ", " << A(k) << ");\n";
  } else if (is_identity_l1_zero(p)) {
    e << ind << "const T xw = " << W() << " * " << X(0) << ";\n";
    for (int k = 0; k < 2 * p.lo + 1; ++k) e << ind << A(k) << " = fmadd(xw, " << qn(1.0, k) << ", " << A(k) << ");\n";
  } else if (2 * p.l1 + 1 < 2 * p.lo + 1) {
    // fold the weight into the inputs: (2l1+1) products, then nnz FMAs
    for (int i = 0; i < 2 * p.l1 + 1; ++i) e << ind << "const T xw" << i << " = " << W() << " * " << X(i) << ";\n";
    for (const auto& z : p.nz)
      e << ind << A(z.k) << " = fmadd(" << (z.c < 0 ? "-" : "") << qn(std::fabs(z.c), z.j) << ", xw" << z.i << ", "
        << A(z.k) << ");\n";
  } else {
    // per output component: t = sum (c sh_j) x_i, then acc += w t
    int cur = -1;
    for (size_t n = 0; n < p.nz.size(); ++n) {
      const auto& z = p.nz[n];
      std::string term = std::string(z.c < 0 ? "-" : "") + qn(std::fabs(z.c), z.j);
      if (z.k != cur) {
        cur = z.k;
        e << ind << "T t" << z.k << " = " << term << " * " << X(z.i) << ";\n";
      } else {
        e << ind << "t" << z.k << " = fmadd(" << term << ", " << X(z.i) << ", t" << z.k << ");\n";
      }
      bool last = (n + 1 == p.nz.size()) || p.nz[n + 1].k != z.k;
      if (last) e << ind << A(z.k) << " = fmadd(" << W() << ", t" << z.k << ", " << A(z.k) << ");\n";
    }
  }
}

// Row load/store of a per-channel component array in either layout, with
// CPL (1 or 2) adjacent channels ub, ub+1 per lane.  `blocks` lists
// (component offset, 2l+1) of the row's blocks; `n` is the array width
// constant (NX or NK).  With CPL = 2 every load is one aligned pair; ir_mul
// stores stay two plain stores (a pair store assembled from two slots of the
// register array keeps part of it out of registers on this compiler).
void emit_row_io(std::ostream& os, const std::string& fname, const std::string& n,
                 const std::vector<std::pair<int, int>>& blocks, int nc, bool load) {
  const std::string arr = "v";
  if (load)
    os << "  template <typename T, int LAYOUT, int CPL, bool NT = false>\n  __device__ __forceinline__ static void "
       << fname << "(const T* __restrict__ row, int mul, int ub, T (&v)[CPL][" << n << "]) {\n";
  else
    os << "  template <typename T, int LAYOUT, int CPL, bool NT = false>\n  __device__ __forceinline__ static void "
       << fname << "(T* __restrict__ row, int mul, int ub, const T (&v)[CPL][" << n << "]) {\n";
  os << "    static_assert(CPL == 1 || CPL == 2, \"one or two channels per lane\");\n";
  auto at = [](int s, int c) { return "v[" + std::to_string(s) + "][" + std::to_string(c) + "]"; };
  os << "    if constexpr (LAYOUT == kIrMul) {\n      if constexpr (CPL == 2) {\n";
  for (int m = 0; m < nc; ++m) {
    const std::string a0 = "row + " + std::to_string(m) + " * mul + ub";
    if (load)
      os << "        { const auto t = ld2<T, NT>(" << a0 << "); " << at(0, m) << " = t.x; " << at(1, m) << " = t.y; }\n";
    else
      os << "        st1<T, NT>(" << a0 << ", " << at(0, m) << "); st1<T, NT>(" << a0 << " + 1, " << at(1, m) << ");\n";
  }
  os << "      } else {\n";
  for (int m = 0; m < nc; ++m) {
    const std::string a0 = "row + " + std::to_string(m) + " * mul + ub";
    if (load)
      os << "        " << at(0, m) << " = ld1<T, NT>(" << a0 << ");\n";
    else
      os << "        st1<T, NT>(" << a0 << ", " << at(0, m) << ");\n";
  }
  os << "      }\n    } else {\n      if constexpr (CPL == 2) {\n";
  for (const auto& [comp, dl] : blocks) {
    // channels ub, ub+1 hold 2*dl consecutive values: element q -> slot q / dl, component q % dl
    for (int pq = 0; pq < dl; ++pq) {
      const int q0 = 2 * pq, q1 = 2 * pq + 1;
      const std::string a = "row + " + std::to_string(comp) + " * mul + ub * " + std::to_string(dl) + " + " + std::to_string(q0);
      if (load)
        os << "        { const auto t = ld2<T, NT>(" << a << "); " << at(q0 / dl, comp + q0 % dl) << " = t.x; "
           << at(q1 / dl, comp + q1 % dl) << " = t.y; }\n";
      else
        os << "        st2<T, NT>(" << a << ", " << at(q0 / dl, comp + q0 % dl) << ", " << at(q1 / dl, comp + q1 % dl)
           << ");\n";
    }
  }
  os << "      } else {\n";
  for (const auto& [comp, dl] : blocks)
    for (int i = 0; i < dl; ++i) {
      const std::string a = "row + " + std::to_string(comp) + " * mul + ub * " + std::to_string(dl) + " + " + std::to_string(i);
      if (load)
        os << "        " << at(0, comp + i) << " = ld1<T, NT>(" << a << ");\n";
      else
        os << "        st1<T, NT>(" << a << ", " << at(0, comp + i) << ");\n";
    }
  os << "      }\n    }\n  }\n\n";
}

// Backward per path: r_k = w g_k; dw = sum_k g_k t_k with t_k the forward
// contraction; the source message m_i += sum_{j,k} c sh_j r_k; the harmonics
// gradient h_j += sum_{i,k} c x_i r_k (summed over the lane's channels).
void emit_path_bwd(const TPPath& p, int pi, std::ostream& e) {
  const int X = p.xcomp, K = p.kcomp, J = static_cast<int>(p.off2), dl = 2 * p.lo + 1;
  QTable lq;
  std::ostringstream body;
  const std::string ind = "        ";
  auto x = [&](int i) { return "xv[s][" + std::to_string(X + i) + "]"; };
  auto gk = [&](int k) { return "gv[s][" + std::to_string(K + k) + "]"; };
  for (int k = 0; k < dl; ++k) body << ind << "const T r" << k << " = wv[s][" << pi << "] * " << gk(k) << ";\n";
  // t_k and dw
  int cur = -1;
  for (size_t n = 0; n < p.nz.size(); ++n) {
    const auto& z = p.nz[n];
    std::string q = std::string(z.c < 0 ? "-" : "") + "q" + std::to_string(lq.get(std::fabs(z.c), J + z.j));
    if (z.k != cur) {
      cur = z.k;
      body << ind << "T t" << z.k << " = " << q << " * " << x(z.i) << ";\n";
    } else {
      body << ind << "t" << z.k << " = fmadd(" << q << ", " << x(z.i) << ", t" << z.k << ");\n";
    }
  }
  body << ind << "T dw = T(0);\n";
  for (int k = 0; k < dl; ++k) {
    bool has = false;
    for (const auto& z : p.nz) has = has || z.k == k;
    if (has) body << ind << "dw = fmadd(" << gk(k) << ", t" << k << ", dw);\n";
  }
  body << ind << "dwv[s][" << pi << "] = dw;\n";
  // source message
  for (const auto& z : p.nz) {
    std::string q = std::string(z.c < 0 ? "-" : "") + "q" + std::to_string(lq.get(std::fabs(z.c), J + z.j));
    body << ind << "mxv[s][" << X + z.i << "] = fmadd(" << q << ", r" << z.k << ", mxv[s][" << X + z.i << "]);\n";
  }
  // harmonics gradient, one product x_i r_k per (i, k)
  int ck = -1, ci = -1;
  for (const auto& z : p.nz) {
    if (z.k != ck || z.i != ci) {
      ck = z.k;
      ci = z.i;
      body << ind << "const T xr" << z.i << "_" << z.k << " = " << x(z.i) << " * r" << z.k << ";\n";
    }
    body << ind << "hsh[" << J + z.j << "] = fmadd(" << lit(z.c) << ", xr" << z.i << "_" << z.k << ", hsh[" << J + z.j
         << "]);\n";
  }
  for (size_t n = 0; n < lq.entries.size(); ++n) {
    const auto& [c, j] = lq.entries[n];
    if (c == 1.0)
      e << "      const T q" << n << " = sh[" << j << "];\n";
    else
      e << "      const T q" << n << " = " << lit(c) << " * sh[" << j << "];\n";
  }
  e << "#pragma unroll\n      for (int s = 0; s < CPL; ++s) {\n" << body.str() << "      }\n";
}

void emit_tp(const std::string& name, unsigned dtypes, const TPDescriptor& d, std::ostream& os) {
  if (!d.uniform_mul) throw std::runtime_error("spec " + name + ": input-1 multiplicities must be uniform");
  const std::string S = "TPSpec_" + name;
  // edge<CPL>(): per path, its uniform products |c| * sh_j (formed right
  // before use from the raw sh row), then the channel slots
  std::ostringstream edge;
  for (size_t pi = 0; pi < d.paths.size(); ++pi) {
    const TPPath& p = d.paths[pi];
    const int X = p.xcomp, K = p.kcomp, J = static_cast<int>(p.off2);
    edge << "    // path " << pi << ": " << p.l1 << " x " << p.l2 << " -> " << p.lo << " (" << p.nz.size()
         << " non-zero)\n    {\n";
    QTable lq;
    std::ostringstream body;
    emit_path_body(
        p, [&](double c, int j) { return "q" + std::to_string(lq.get(c, J + j)); },
        [&](int i) { return "xv[s][" + std::to_string(X + i) + "]"; },
        [&]() { return "wv[s][" + std::to_string(pi) + "]"; },
        [&](int k) { return "acc[s][" + std::to_string(K + k) + "]"; }, "        ", body);
    for (size_t n = 0; n < lq.entries.size(); ++n) {
      const auto& [c, j] = lq.entries[n];
      if (c == 1.0)
        edge << "      const T q" << n << " = sh[" << j << "];\n";
      else
        edge << "      const T q" << n << " = " << lit(c) << " * sh[" << j << "];\n";
    }
    edge << "#pragma unroll\n      for (int s = 0; s < CPL; ++s) {\n" << body.str() << "      }\n    }\n";
  }

  os << "// Generated by codegen.cpp from the descriptor: " << irreps_str(d.in1) << " x " << irreps_str(d.in2)
     << " -> " << irreps_str(d.out) << "\n// key " << d.key << "\n";
  os << "#include \"kernels/tp_conv_spec.hpp\"\n#include \"kernels/tp_conv_bwd.hpp\"\n\nnamespace segpoly {\nnamespace kern {\n\n";
  os << "struct " << S << " {\n";
  os << "  static constexpr int NX = " << d.nx << ";\n";
  os << "  static constexpr int NK = " << d.nk << ";\n";
  os << "  static constexpr int NP = " << d.paths.size() << ";\n";
  os << "  static constexpr int D2 = " << d.dim2 << ";\n\n";
  std::vector<std::pair<int, int>> in_blocks, out_blocks;
  {
    int comp = 0;
    for (const auto& r : d.in1) {
      in_blocks.push_back({comp, 2 * r.l + 1});
      comp += 2 * r.l + 1;
    }
    for (const auto& p : d.paths) {  // one block per distinct output slot (merged paths share one)
      bool seen = false;
      for (const auto& b : out_blocks) seen = seen || b.first == p.kcomp;
      if (!seen) out_blocks.push_back({p.kcomp, 2 * p.lo + 1});
    }
  }
  // input-1 blocks (2l + 1 components each, in row order): the backward
  // stages mul_ir message rows block by block
  os << "  static constexpr int NXB = " << in_blocks.size() << ";\n";
  os << "  __host__ __device__ static constexpr int xblock_dim(int b) {\n    constexpr int d[NXB] = {";
  for (size_t b = 0; b < in_blocks.size(); ++b) os << (b ? ", " : "") << in_blocks[b].second;
  os << "};\n    return d[b];\n  }\n\n";
  emit_row_io(os, "load_xs", "NX", in_blocks, d.nx, true);
  emit_row_io(os, "store_xs", "NX", in_blocks, d.nx, false);
  emit_row_io(os, "load_gs", "NK", out_blocks, d.nk, true);
  emit_row_io(os, "store_s", "NK", out_blocks, d.nk, false);
  os << "  template <typename T, int CPL>\n  __device__ __forceinline__ static void bwd(const T (&xv)[CPL][NX], const T* __restrict__ sh,\n"
        "      const T (&wv)[CPL][NP], const T (&gv)[CPL][NK], T (&dwv)[CPL][NP], T (&mxv)[CPL][NX], T (&hsh)[D2]) {\n";
  os << "#pragma unroll\n    for (int s = 0; s < CPL; ++s)\n#pragma unroll\n      for (int i = 0; i < NX; ++i) mxv[s][i] = T(0);\n";
  os << "#pragma unroll\n    for (int j = 0; j < D2; ++j) hsh[j] = T(0);\n";
  for (size_t pi = 0; pi < d.paths.size(); ++pi) {
    const TPPath& p = d.paths[pi];
    os << "    // path " << pi << ": " << p.l1 << " x " << p.l2 << " -> " << p.lo << "\n    {\n";
    emit_path_bwd(p, static_cast<int>(pi), os);
    os << "    }\n";
  }
  os << "  }\n\n";
  os << "  template <typename T, int CPL>\n  __device__ __forceinline__ static void edge(const T (&xv)[CPL][NX], const T* __restrict__ sh,\n"
        "                                                   const T (&wv)[CPL][NP], T (&acc)[CPL][NK]) {\n";
  os << edge.str();
  os << "  }\n};\n\n}  // namespace kern\n\n";
  os << "int launch_tp_" << name << "(const TPArgs& a) {\n";
  if (dtypes & 1u) os << "  if (a.dtype == kF32) return kern::tp_conv_dispatch<kern::" << S << ", float>(a);\n";
  if (dtypes & 2u) os << "  if (a.dtype == kF64) return kern::tp_conv_dispatch<kern::" << S << ", double>(a);\n";
  os << "  return -1;\n}\n\n";
  os << "int launch_tp_bwd_" << name << "(const TPBwdArgs& a) {\n";
  if (dtypes & 1u) os << "  if (a.dtype == kF32) return kern::tp_bwd_dispatch<kern::" << S << ", float>(a);\n";
  if (dtypes & 2u) os << "  if (a.dtype == kF64) return kern::tp_bwd_dispatch<kern::" << S << ", double>(a);\n";
  os << "  return -1;\n}\n\n}  // namespace segpoly\n";
}

// ---------------------------------------------------------------- symcon

void emit_symcon(const std::string& name, unsigned dtypes, const SymconDescriptor& d, std::ostream& os) {
  const std::string S = "SymconSpec_" + name;
  const int n = d.n;
  const int ns = static_cast<int>(d.couplings.size());
  // monomial -> [(segment, M, c)]
  std::map<std::tuple<int, int, int>, std::vector<std::tuple<int, int, double>>> mono;
  for (int s = 0; s < ns; ++s)
    for (const auto& t : d.couplings[s].terms) mono[{t.m[0], t.m[1], t.m[2]}].push_back({s, t.M, t.c});
  // Forward, per atom and channel, with the degree-3 terms factored by
  // their first (smallest) component index a:
  //   o[og] += v[a] * sum over segments s into og of wv[s] * T_{s,M,a},
  //   T_{s,M,a} = sum over the terms (a, b, c) of (s, M) of c * q_bc,
  // q_bc = v[b] v[c] formed once, before its first use (a ascending).  Per
  // atom-channel this takes one multiply per distinct pair, one operation per
  // term and one per (s, M, a) and per (og, a) group, against one multiply
  // per distinct monomial plus one operation per term plus one per segment
  // when every monomial is formed and each segment's sum is weighted at the
  // end (the l <= 3 -> l <= 1 contraction: 854 against 1,089 operations).
  // Degrees 1 and 2: o[og] += wv[s] * (sum of c * v[a] or c * q_ab).
  std::ostringstream body;
  {
    std::set<std::pair<int, int>> have_q;
    std::set<int> started;
    auto q = [&](int b, int c) {
      const std::string nm = "q" + std::to_string(b) + "_" + std::to_string(c);
      if (!have_q.count({b, c})) {
        have_q.insert({b, c});
        body << "    const T " << nm << " = v[" << b << "] * v[" << c << "];\n";
      }
      return nm;
    };
    auto acc_o = [&](int og, const std::string& f, const std::string& t) {
      if (started.count(og)) {
        body << "    o[" << og << "] = fmadd(" << f << ", " << t << ", o[" << og << "]);\n";
      } else {
        started.insert(og);
        body << "    o[" << og << "] = " << f << " * " << t << ";\n";
      }
    };
    auto og_of = [&](int sg, int M) { return d.out_comp[d.couplings[sg].ob] + M; };
    // degrees 1 and 2, per (segment, component)
    std::map<std::pair<int, int>, std::vector<std::tuple<double, int, int>>> low;
    // degree 3: a -> (og, segment) -> [(c, b, cc)]
    std::map<int, std::map<std::pair<int, int>, std::vector<std::tuple<double, int, int>>>> hi3;
    for (int sg = 0; sg < ns; ++sg)
      for (const auto& t : d.couplings[sg].terms) {
        if (t.m[2] >= 0)
          hi3[t.m[0]][{og_of(sg, t.M), sg}].push_back({t.c, t.m[1], t.m[2]});
        else
          low[{sg, t.M}].push_back({t.c, t.m[0], t.m[1]});
      }
    for (const auto& [key, lst] : low) {
      const std::string tn = "t" + std::to_string(key.first) + "_" + std::to_string(key.second);
      bool first = true;
      for (const auto& [c, a, b] : lst) {
        const std::string x = b < 0 ? "v[" + std::to_string(a) + "]" : q(a, b);
        if (first)
          body << "    T " << tn << " = " << lit(c) << " * " << x << ";\n";
        else
          body << "    " << tn << " = fmadd(" << lit(c) << ", " << x << ", " << tn << ");\n";
        first = false;
      }
      acc_o(og_of(key.first, key.second), "wv[" + std::to_string(key.first) + "]", tn);
    }
    for (const auto& [a, groups] : hi3) {
      std::map<int, std::vector<int>> segs_of_og;  // og -> segments, in order
      for (const auto& [key, lst] : groups) segs_of_og[key.first].push_back(key.second);
      for (const auto& [og, segs] : segs_of_og) {
        const std::string un = "u" + std::to_string(a) + "_" + std::to_string(og);
        bool first_u = true;
        for (int sg : segs) {
          const auto& lst = groups.at({og, sg});
          const std::string tn = "r" + std::to_string(a) + "_" + std::to_string(og) + "_" + std::to_string(sg);
          bool first = true;
          for (const auto& [c, b, cc] : lst) {
            const std::string x = q(b, cc);
            if (first)
              body << "    T " << tn << " = " << lit(c) << " * " << x << ";\n";
            else
              body << "    " << tn << " = fmadd(" << lit(c) << ", " << x << ", " << tn << ");\n";
            first = false;
          }
          if (first_u)
            body << "    T " << un << " = wv[" << sg << "] * " << tn << ";\n";
          else
            body << "    " << un << " = fmadd(wv[" << sg << "], " << tn << ", " << un << ");\n";
          first_u = false;
        }
        acc_o(og, "v[" + std::to_string(a) + "]", un);
      }
    }
    for (int og = 0; og < d.nout; ++og)
      if (!started.count(og)) body << "    o[" << og << "] = T(0);\n";
  }

  // backward, per atom and channel, in two functions (fewer live registers):
  // bwd_w: dw[s] += sum over M of g[M] a_{s,M}, a_{s,M} the segment sums of
  //    the forward, evaluated in the forward's factored form (as above);
  // bwd_x: gw_{s,M} = w[s] g[M]; per monomial B = sum of c gw over its terms;
  //    dx by the product rule, grouped by the sorted prefix (a, b):
  //    S_ab = B_ab + sum_c B_abc v[c], dx[c] += B_abc v[a] v[b],
  //    dx[a] += v[b] S_ab, dx[b] += v[a] S_ab; degree 1: dx[a] += B_a.
  std::ostringstream bwd;
  std::string bwd_w, bwd_x;
  {
    std::set<std::pair<int, int>> used1;  // (segment, component) pairs with terms
    for (int sg = 0; sg < ns; ++sg)
      for (const auto& t : d.couplings[sg].terms) used1.insert({sg, t.M});
    auto og_of = [&](int sg, int M) { return d.out_comp[d.couplings[sg].ob] + M; };
    // bwd_w, factored like the forward, with the output gradient in the
    // place of the weights: dw[s] += g[og] * (degree-1 and -2 sums), and
    // per first index a, dw[s] += v[a] * sum over M of g[og] * T_{s,M,a}
    std::set<std::pair<int, int>> have_q;
    auto q = [&](int b, int c) {
      const std::string nm = "q" + std::to_string(b) + "_" + std::to_string(c);
      if (!have_q.count({b, c})) {
        have_q.insert({b, c});
        bwd << "      const T " << nm << " = v[" << b << "] * v[" << c << "];\n";
      }
      return nm;
    };
    std::map<std::pair<int, int>, std::vector<std::tuple<double, int, int>>> low;
    // a -> (segment, M) -> [(c, b, cc)]
    std::map<int, std::map<std::pair<int, int>, std::vector<std::tuple<double, int, int>>>> hi3;
    for (int sg = 0; sg < ns; ++sg)
      for (const auto& t : d.couplings[sg].terms) {
        if (t.m[2] >= 0)
          hi3[t.m[0]][{sg, t.M}].push_back({t.c, t.m[1], t.m[2]});
        else
          low[{sg, t.M}].push_back({t.c, t.m[0], t.m[1]});
      }
    bwd << "    {\n";
    for (const auto& [key, lst] : low) {
      const std::string tn = "t" + std::to_string(key.first) + "_" + std::to_string(key.second);
      bool first = true;
      for (const auto& [c, a, b] : lst) {
        const std::string x = b < 0 ? "v[" + std::to_string(a) + "]" : q(a, b);
        if (first)
          bwd << "      T " << tn << " = " << lit(c) << " * " << x << ";\n";
        else
          bwd << "      " << tn << " = fmadd(" << lit(c) << ", " << x << ", " << tn << ");\n";
        first = false;
      }
      bwd << "      dw[" << key.first << "] = fmadd(g[" << og_of(key.first, key.second) << "], " << tn << ", dw["
          << key.first << "]);\n";
    }
    for (const auto& [a, groups] : hi3) {
      std::map<int, std::vector<int>> comps_of_seg;  // segment -> components, in order
      for (const auto& [key, lst] : groups) comps_of_seg[key.first].push_back(key.second);
      for (const auto& [sg, comps] : comps_of_seg) {
        const std::string un = "u" + std::to_string(a) + "_" + std::to_string(sg);
        bool first_u = true;
        for (int M : comps) {
          const auto& lst = groups.at({sg, M});
          const std::string tn = "r" + std::to_string(a) + "_" + std::to_string(sg) + "_" + std::to_string(M);
          bool first = true;
          for (const auto& [c, b, cc] : lst) {
            const std::string x = q(b, cc);
            if (first)
              bwd << "      T " << tn << " = " << lit(c) << " * " << x << ";\n";
            else
              bwd << "      " << tn << " = fmadd(" << lit(c) << ", " << x << ", " << tn << ");\n";
            first = false;
          }
          const std::string gg = "g[" + std::to_string(og_of(sg, M)) + "]";
          if (first_u)
            bwd << "      T " << un << " = " << gg << " * " << tn << ";\n";
          else
            bwd << "      " << un << " = fmadd(" << gg << ", " << tn << ", " << un << ");\n";
          first_u = false;
        }
        bwd << "      dw[" << sg << "] = fmadd(v[" << a << "], " << un << ", dw[" << sg << "]);\n";
      }
    }
    bwd << "    }\n";
    bwd_w = bwd.str();
    bwd.str("");
    bwd << "    {\n";
    for (const auto& [sg, M] : used1) {
      const int og = d.out_comp[d.couplings[sg].ob] + M;
      bwd << "      const T gw" << sg << "_" << M << " = wv[" << sg << "] * g[" << og << "];\n";
    }
    for (int i = 0; i < n; ++i) bwd << "      dx[" << i << "] = T(0);\n";
    auto adj = [&](const std::string& B, const std::vector<std::tuple<int, int, double>>& terms) {
      bool first = true;
      for (const auto& [sg, M, c] : terms) {
        const std::string gw = "gw" + std::to_string(sg) + "_" + std::to_string(M);
        if (first)
          bwd << "      T " << B << " = " << lit(c) << " * " << gw << ";\n";
        else
          bwd << "      " << B << " = fmadd(" << lit(c) << ", " << gw << ", " << B << ");\n";
        first = false;
      }
    };
    for (int a = 0; a < n; ++a) {
      auto it = mono.find({a, -1, -1});
      if (it == mono.end()) continue;
      const std::string B = "b" + std::to_string(a);
      bwd << "      {\n";
      adj(B, it->second);
      bwd << "      dx[" << a << "] += " << B << ";\n      }\n";
    }
    for (int a = 0; a < n; ++a)
      for (int b = a; b < n; ++b) {
        const bool has2 = mono.count({a, b, -1}) > 0;
        bool has3 = false;
        for (int c = b; c < n && !has3; ++c) has3 = mono.count({a, b, c}) > 0;
        if (!has2 && !has3) continue;
        bwd << "      {\n";
        if (has2) {
          adj("S", mono.at({a, b, -1}));
        } else {
          bwd << "      T S = T(0);\n";
        }
        if (has3) bwd << "      const T p = v[" << a << "] * v[" << b << "];\n";
        for (int c = b; c < n; ++c) {
          auto jt = mono.find({a, b, c});
          if (jt == mono.end()) continue;
          const std::string B = "b" + std::to_string(c);
          bwd << "      {\n";
          adj(B, jt->second);
          bwd << "      S = fmadd(" << B << ", v[" << c << "], S);\n";
          bwd << "      dx[" << c << "] = fmadd(" << B << ", p, dx[" << c << "]);\n      }\n";
        }
        bwd << "      dx[" << a << "] = fmadd(v[" << b << "], S, dx[" << a << "]);\n";
        bwd << "      dx[" << b << "] = fmadd(v[" << a << "], S, dx[" << b << "]);\n      }\n";
      }
    bwd << "    }\n";
    bwd_x = bwd.str();
  }

  os << "// Generated by codegen.cpp from the descriptor: symmetric contraction " << irreps_str(d.in) << " -> "
     << irreps_str(d.out) << "\n// key " << d.key << "\n// " << d.num_terms() << " sorted-monomial terms\n";
  os << "#include \"kernels/symcon_spec.hpp\"\n#include \"kernels/symcon_bwd.hpp\"\n\nnamespace segpoly {\nnamespace kern {\n\n";
  os << "struct " << S << " {\n";
  os << "  static constexpr int NV = " << n << ";\n";
  os << "  static constexpr int NO = " << d.nout << ";\n";
  os << "  static constexpr int NS = " << ns << ";\n\n";
  os << "  template <typename T, int LAYOUT>\n  __device__ __forceinline__ static void load_v(const T* __restrict__ row, int mul, int u, T* v) {\n";
  os << "    if constexpr (LAYOUT == kIrMul) {\n";
  for (int m = 0; m < n; ++m) os << "      v[" << m << "] = row[" << m << " * mul + u];\n";
  os << "    } else {\n";
  for (size_t b = 0; b < d.in.size(); ++b) {
    const int dl = 2 * d.in[b].l + 1, comp = d.in_comp[b];
    os << "      {\n        const T* p = row + " << comp << " * mul + u * " << dl << ";\n";
    for (int i = 0; i < dl; ++i) os << "        v[" << comp + i << "] = p[" << i << "];\n";
    os << "      }\n";
  }
  os << "    }\n  }\n\n";
  // buffer-resource forms of the row accesses: load_v_b (input row),
  // load_o_b (output-gradient row), store_v_b (input-gradient row), store_b
  // (output row)
  auto emit_buf = [&](const char* fname, bool store, const char* arr, const std::vector<Irrep>& blocks,
                      const std::vector<int>& comps, int count) {
    os << "  template <typename T, int LAYOUT>\n  __device__ __forceinline__ static void " << fname
       << "(__amdgpu_buffer_rsrc_t r, int mul, int u, " << (store ? "const T* " : "T* ") << arr << ") {\n";
    os << "    constexpr uint32_t E = sizeof(T);\n    const uint32_t m = static_cast<uint32_t>(mul);\n";
    os << "    if constexpr (LAYOUT == kIrMul) {\n      const uint32_t vo = static_cast<uint32_t>(u) * E;\n";
    for (int k = 0; k < count; ++k) {
      if (store)
        os << "      buf_store_s<T>(r, vo, " << k << "u * m * E, " << arr << "[" << k << "]);\n";
      else
        os << "      " << arr << "[" << k << "] = buf_load_s<T>(r, vo, " << k << "u * m * E);\n";
    }
    os << "    } else {\n";
    for (size_t b = 0; b < blocks.size(); ++b) {
      const int dl = 2 * blocks[b].l + 1, comp = comps[b];
      os << "      {\n        const uint32_t vo = static_cast<uint32_t>(u) * " << dl << "u * E;\n";
      for (int i = 0; i < dl; ++i) {
        if (store)
          os << "        buf_store_s<T>(r, vo, (" << comp << "u * m + " << i << "u) * E, " << arr << "[" << comp + i
             << "]);\n";
        else
          os << "        " << arr << "[" << comp + i << "] = buf_load_s<T>(r, vo, (" << comp << "u * m + " << i
             << "u) * E);\n";
      }
      os << "      }\n";
    }
    os << "    }\n  }\n\n";
  };
  emit_buf("load_o_b", false, "o", d.out, d.out_comp, d.nout);
  emit_buf("store_v_b", true, "v", d.in, d.in_comp, n);
  // the same load through a buffer resource based at the row: the lane's
  // offset is one register per block width, the component offsets are
  // wave-uniform (scalar) operands, so no per-load address arithmetic
  os << "  template <typename T, int LAYOUT>\n  __device__ __forceinline__ static void load_v_b(__amdgpu_buffer_rsrc_t r, int mul, int u, T* v) {\n";
  os << "    constexpr uint32_t E = sizeof(T);\n    const uint32_t m = static_cast<uint32_t>(mul);\n";
  os << "    if constexpr (LAYOUT == kIrMul) {\n      const uint32_t vo = static_cast<uint32_t>(u) * E;\n";
  for (int m = 0; m < n; ++m) os << "      v[" << m << "] = buf_load_s<T>(r, vo, " << m << "u * m * E);\n";
  os << "    } else {\n";
  for (size_t b = 0; b < d.in.size(); ++b) {
    const int dl = 2 * d.in[b].l + 1, comp = d.in_comp[b];
    os << "      {\n        const uint32_t vo = static_cast<uint32_t>(u) * " << dl << "u * E;\n";
    for (int i = 0; i < dl; ++i)
      os << "        v[" << comp + i << "] = buf_load_s<T>(r, vo, (" << comp << "u * m + " << i << "u) * E);\n";
    os << "      }\n";
  }
  os << "    }\n  }\n\n";
  // gradient-row load (output layout) and input-gradient store (input layout)
  os << "  template <typename T, int LAYOUT>\n  __device__ __forceinline__ static void load_o(const T* __restrict__ row, int mul, int u, T* o) {\n";
  os << "    if constexpr (LAYOUT == kIrMul) {\n";
  for (int k = 0; k < d.nout; ++k) os << "      o[" << k << "] = row[" << k << " * mul + u];\n";
  os << "    } else {\n";
  for (size_t b = 0; b < d.out.size(); ++b) {
    const int dl = 2 * d.out[b].l + 1, comp = d.out_comp[b];
    os << "      {\n        const T* p = row + " << comp << " * mul + u * " << dl << ";\n";
    for (int i = 0; i < dl; ++i) os << "        o[" << comp + i << "] = p[" << i << "];\n";
    os << "      }\n";
  }
  os << "    }\n  }\n\n";
  os << "  template <typename T, int LAYOUT>\n  __device__ __forceinline__ static void store_v(T* __restrict__ row, int mul, int u, const T* v) {\n";
  os << "    if constexpr (LAYOUT == kIrMul) {\n";
  for (int m = 0; m < n; ++m) os << "      row[" << m << " * mul + u] = v[" << m << "];\n";
  os << "    } else {\n";
  for (size_t b = 0; b < d.in.size(); ++b) {
    const int dl = 2 * d.in[b].l + 1, comp = d.in_comp[b];
    os << "      {\n        T* p = row + " << comp << " * mul + u * " << dl << ";\n";
    for (int i = 0; i < dl; ++i) os << "        p[" << i << "] = v[" << comp + i << "];\n";
    os << "      }\n";
  }
  os << "    }\n  }\n\n";
  os << "  // dw[s] += d<g, out>/dw[s]\n";
  os << "  template <typename T>\n  __device__ __forceinline__ static void bwd_w(const T* v, const T* g, T* dw) {\n";
  os << bwd_w;
  os << "  }\n\n";
  os << "  // dx = d<g, out>/dv (overwritten)\n";
  os << "  template <typename T>\n  __device__ __forceinline__ static void bwd_x(const T* v, const T* g, const T* wv, T* dx) {\n";
  os << bwd_x;
  os << "  }\n\n";
  os << "  template <typename T>\n  __device__ __forceinline__ static void eval(const T* v, const T* wv, T* o) {\n";
  os << body.str();
  os << "  }\n\n";
  os << "  template <typename T, int LAYOUT>\n  __device__ __forceinline__ static void store_b(__amdgpu_buffer_rsrc_t r, int mul, int u, const T* o) {\n";
  os << "    constexpr uint32_t E = sizeof(T);\n    const uint32_t m = static_cast<uint32_t>(mul);\n";
  os << "    if constexpr (LAYOUT == kIrMul) {\n      const uint32_t vo = static_cast<uint32_t>(u) * E;\n";
  for (int k = 0; k < d.nout; ++k) os << "      buf_store_s<T>(r, vo, " << k << "u * m * E, o[" << k << "]);\n";
  os << "    } else {\n";
  for (size_t b = 0; b < d.out.size(); ++b) {
    const int dl = 2 * d.out[b].l + 1, comp = d.out_comp[b];
    os << "      {\n        const uint32_t vo = static_cast<uint32_t>(u) * " << dl << "u * E;\n";
    for (int i = 0; i < dl; ++i)
      os << "        buf_store_s<T>(r, vo, (" << comp << "u * m + " << i << "u) * E, o[" << comp + i << "]);\n";
    os << "      }\n";
  }
  os << "    }\n  }\n\n";
  os << "  template <typename T, int LAYOUT>\n  __device__ __forceinline__ static void store(T* __restrict__ row, int mul, int u, const T* o) {\n";
  os << "    if constexpr (LAYOUT == kIrMul) {\n";
  for (int k = 0; k < d.nout; ++k) os << "      row[" << k << " * mul + u] = o[" << k << "];\n";
  os << "    } else {\n";
  for (size_t b = 0; b < d.out.size(); ++b) {
    const int dl = 2 * d.out[b].l + 1, comp = d.out_comp[b];
    os << "      {\n        T* p = row + " << comp << " * mul + u * " << dl << ";\n";
    for (int i = 0; i < dl; ++i) os << "        p[" << i << "] = o[" << comp + i << "];\n";
    os << "      }\n";
  }
  os << "    }\n  }\n};\n\n}  // namespace kern\n\n";
  os << "int launch_symcon_" << name << "(const SymconArgs& a) {\n";
  if (dtypes & 1u) os << "  if (a.dtype == kF32) return kern::symcon_spec_dispatch<kern::" << S << ", float>(a);\n";
  if (dtypes & 2u) os << "  if (a.dtype == kF64) return kern::symcon_spec_dispatch<kern::" << S << ", double>(a);\n";
  os << "  return -1;\n}\n\n";
  os << "int launch_symcon_bwd_" << name << "(const SymconBwdArgs& a) {\n";
  if (dtypes & 1u) os << "  if (a.dtype == kF32) return kern::symcon_bwd_dispatch<kern::" << S << ", float>(a);\n";
  if (dtypes & 2u) os << "  if (a.dtype == kF64) return kern::symcon_bwd_dispatch<kern::" << S << ", double>(a);\n";
  os << "  return -1;\n}\n\n}  // namespace segpoly\n";
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::cerr << "usage: segpoly_codegen SPECS OUTDIR\n";
    return 2;
  }
  std::ifstream in(argv[1]);
  if (!in) {
    std::cerr << "cannot read " << argv[1] << "\n";
    return 2;
  }
  const std::string outdir = argv[2];
  struct Reg {
    std::string kind, name, key;
    unsigned dtypes;
  };
  std::vector<Reg> regs;
  std::string line;
  try {
    while (std::getline(in, line)) {
      line = trim(line);
      if (line.empty() || line[0] == '#') continue;
      auto parts = split(line, '|');
      if (parts.size() != 4) throw std::runtime_error("bad spec line: " + line);
      auto head = split(parts[0], ' ');
      std::vector<std::string> h;
      for (auto& t : head)
        if (!t.empty()) h.push_back(t);
      if (h.size() != 3) throw std::runtime_error("bad spec head: " + parts[0]);
      const std::string kind = h[0], name = h[1];
      const unsigned dt = dtype_mask(h[2]);
      const std::string path = outdir + "/" + kind + "_" + name + ".hip";
      std::ofstream os(path);
      if (kind == "tp" || kind == "tpm") {  // tpm: merged output blocks
        TPDescriptor d = build_tp(parts[1], parts[2], parts[3], kind == "tpm");
        emit_tp(name, dt, d, os);
        regs.push_back({"tp", name, d.key, dt});
      } else if (kind == "symcon") {
        std::vector<int> deg;
        for (auto& t : split(parts[3], ',')) deg.push_back(std::stoi(t));
        SymconDescriptor d = build_symcon(parts[1], parts[2], deg);
        emit_symcon(name, dt, d, os);
        regs.push_back({kind, name, d.key, dt});
      } else {
        throw std::runtime_error("unknown spec kind " + kind);
      }
      std::cout << path << "\n";
    }
  } catch (const std::exception& e) {
    std::cerr << "codegen: " << e.what() << "\n";
    return 1;
  }
  std::ofstream reg(outdir + "/registry.cpp");
  reg << "// Generated by codegen.cpp: structure key -> specialised launcher.\n#include \"launch.hpp\"\n\nnamespace segpoly {\n\n";
  for (const auto& r : regs) {
    reg << "int launch_" << r.kind << "_" << r.name << "(const " << (r.kind == "tp" ? "TPArgs" : "SymconArgs")
        << "&);\n";
    if (r.kind == "tp") reg << "int launch_tp_bwd_" << r.name << "(const TPBwdArgs&);\n";
    if (r.kind == "symcon") reg << "int launch_symcon_bwd_" << r.name << "(const SymconBwdArgs&);\n";
  }
  reg << "\nconst TPSpecEntry kTPSpecs[] = {\n";
  int ntp = 0, nsc = 0;
  for (const auto& r : regs)
    if (r.kind == "tp") {
      reg << "    {\"" << r.key << "\", \"" << r.name << "\", " << r.dtypes << "u, &launch_tp_" << r.name << ", &launch_tp_bwd_"
          << r.name << "},\n";
      ++ntp;
    }
  if (!ntp) reg << "    {\"\", \"\", 0u, nullptr, nullptr},\n";
  reg << "};\nconst int kNumTPSpecs = " << ntp << ";\n\nconst SymconSpecEntry kSymconSpecs[] = {\n";
  for (const auto& r : regs)
    if (r.kind == "symcon") {
      reg << "    {\"" << r.key << "\", \"" << r.name << "\", " << r.dtypes << "u, &launch_symcon_" << r.name
          << ", &launch_symcon_bwd_" << r.name << "},\n";
      ++nsc;
    }
  if (!nsc) reg << "    {\"\", \"\", 0u, nullptr, nullptr},\n";
  reg << "};\nconst int kNumSymconSpecs = " << nsc << ";\n\n}  // namespace segpoly\n";
  return 0;
}
