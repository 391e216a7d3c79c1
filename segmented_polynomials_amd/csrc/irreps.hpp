// O(3) irreps strings: "32x0e + 32x1o" is a sum of terms MULxLP with P = e
// (parity +1) or o (parity -1); a term without MULx has multiplicity 1
// (e3nn-course Lesson 12a, section 21.2).  Host code only.
#pragma once
#include <stdexcept>
#include <string>
#include <vector>

namespace segpoly {

struct ParseError : std::runtime_error {
  using std::runtime_error::runtime_error;
};

struct Irrep {
  int mul;
  int l;
  int p;  // +1 even, -1 odd
};

std::vector<Irrep> parse_irreps(const std::string& s);
int irreps_dim(const std::vector<Irrep>& v);
std::string irreps_str(const std::vector<Irrep>& v);
std::string type_str(int l, int p);

// Order of output irrep types: by l, and within one l the natural parity
// (-1)^l first: 0e, 0o, 1o, 1e, 2e, 2o, ...
inline int type_rank(int l, int p) {
  int natural = (l % 2 == 0) ? 1 : -1;
  return 2 * l + (p == natural ? 0 : 1);
}

}  // namespace segpoly
