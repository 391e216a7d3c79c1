// Descriptor of one channelwise (uvu) tensor product, host side.
//
// e3nn-course Lesson 12a, section 21.4: the descriptor
// [ijk]*a[uv]*b[iu]*c[jv] -> D[kuv] with a the weights, b input 1 (channel
// u), c input 2 (v = 1) and one path per non-zero coupling.  Paths follow the
// selection rule |l1-l2| <= lo <= l1+l2, output parity p1*p2.  The output
// argument selects irrep types, not multiplicities (cuequivariance-torch
// skill document, "Layouts and weights"): each kept path owns one output
// block of multiplicity mul_i.  Enumeration: input-1 block, input-2 block,
// lo ascending; then a stable sort by output type (l, natural parity
// first), which is also the order of the weight segments (one segment of
// mul_i weights per path, channel fastest).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "irreps.hpp"

namespace segpoly {

struct CGEntry {
  int i, j, k;  // component indices within the path's blocks
  double c;
};

struct TPPath {
  int b1, b2;        // input-1 block, input-2 block
  int l1, l2, lo, po;
  int mul;
  int64_t off1;      // element offset of the input-1 block in a row of x
  int64_t off2;      // element offset of the input-2 block in a row of sh
  int64_t offo;      // element offset of the output block in a row of out
  int64_t woff;      // offset of the weight segment in a row of w
  int xcomp;         // per-channel component offset of the input-1 block
  int kcomp;         // per-channel component offset of the output block
  std::vector<CGEntry> nz;  // non-zero coefficients, ordered by (k, i, j)
};

struct TPDescriptor {
  std::vector<Irrep> in1, in2, out;
  std::vector<TPPath> paths;
  int64_t dim1 = 0, dim2 = 0, dimo = 0, numel = 0;
  bool uniform_mul = false;  // every input-1 block has the same multiplicity
  int mul = 0;               // that multiplicity (if uniform)
  int nx = 0;                // components per channel of input 1 (sum 2l+1)
  int nk = 0;                // components per channel of the output
  bool merged = false;       // paths of one output type share one output block
  std::string key;           // structure key (independent of multiplicity)
  int64_t cg_nnz() const;
};

// Throws ParseError on bad strings, std::invalid_argument on unsupported
// input (input-2 multiplicity other than 1, an l above kMaxL in any of the
// three strings, so that no path couples to an output above kMaxL).
// merge: the paths of one output type sum into one block of that type (all
// of them must have the same multiplicity); output blocks in type order.
TPDescriptor build_tp(const std::string& irreps_in1, const std::string& irreps_in2,
                      const std::string& irreps_out, bool merge = false);

// Largest l of any block (inputs and output filter).  Every coupling tensor
// the builder can produce (l1, l2, lo <= 6) is compared entry by entry with
// the oracle's exact-arithmetic construction on the host.
constexpr int kMaxL = 6;

}  // namespace segpoly
