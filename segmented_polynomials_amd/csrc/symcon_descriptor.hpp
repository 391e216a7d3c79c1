// Descriptor of the symmetric contraction, host side.
//
// e3nn-course Lesson 12a, section 21.4.1: one row per degree nu,
// []*a[u]*b[u]...*b[u] -> C[u], every channel contracted with itself,
// weights carrying the channel; the cuequivariance-torch skill document
// ("Other operations and layers") adds per-atom element indices and uniform
// multiplicities.  Degrees are summed into one output.
//
// Per channel the input components form one vector v (blocks in order,
// components m = -l..l).  For each degree nu and output block (type L) the
// coupling basis is built by a fixed procedure (the pages fix none):
//   candidates: ordered block tuples in lexicographic order (and, for
//   nu = 3, the intermediate L12 ascending) whose parities multiply to that
//   of L and that satisfy the triangle rules; tensor = the real coupling
//   embedded at the blocks' offsets (identity for nu = 1, C(l1,l2,L) for
//   nu = 2, sum_a C(l1,l2,L12)[i,j,a] C(L12,l3,L)[a,k,M] for nu = 3);
//   symmetrise over the nu! slot permutations; accept the symmetrised
//   tensor when its Gram-Schmidt residual against the accepted span exceeds
//   1e-8 of its norm; scale it so that sum_{m..} U[m..,M] U[m..,M'] = delta.
// Weight segments: nu ascending, then output block, then coupling, each
// `mul` wide.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "irreps.hpp"

namespace segpoly {

struct MonoTerm {
  int m[3];   // sorted component indices (m[0] <= m[1] <= m[2]); unused = -1
  int M;      // output component within the output block
  double c;   // U[m.., M] times the number of distinct orderings of m
};

struct SymconCoupling {
  int nu, ob, k, L;
  std::vector<double> dense;     // [n]*nu x [2L+1], row-major
  std::vector<MonoTerm> terms;   // sorted-monomial form of `dense`
};

struct SymconDescriptor {
  std::vector<Irrep> in, out;
  std::vector<int> degrees;
  int mul = 0;
  int n = 0;                    // components per channel of the input
  int nout = 0;                 // components per channel of the output
  std::vector<int> in_comp;     // per input block: component offset
  std::vector<int> out_comp;    // per output block: component offset
  std::vector<SymconCoupling> couplings;  // weight-segment order
  int64_t dim_in = 0, dim_out = 0, numel = 0;
  std::string key;
  int64_t num_terms() const;
  // products a per-channel evaluation forms: one per distinct sorted pair
  // (m1, m2) that a degree-2 term or a degree-3 prefix needs, plus one per
  // distinct sorted triple
  int64_t num_monomial_products() const;
};

// Throws ParseError / std::invalid_argument (non-uniform multiplicities,
// degrees outside 1..3, l above the supported maximum).
SymconDescriptor build_symcon(const std::string& irreps_in, const std::string& irreps_out,
                              const std::vector<int>& degrees);

}  // namespace segpoly
