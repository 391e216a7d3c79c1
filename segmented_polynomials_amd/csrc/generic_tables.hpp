// Device-side tables of the table-driven kernels (plain structs, uploaded
// once per device by the C ABI).
#pragma once
#include <cstdint>

#include "launch.hpp"

namespace segpoly {

struct GPath {
  int l1, lo, mul, nz_begin, nz_end, kcomp, pad0, pad1;
  int64_t off1, off2, offo, woff;
};

struct GNz {
  int i, j, k, pad;
  double c;
};

struct GTerm {
  int m0, m1, m2, og, seg, pad;
  double c;
};

struct GBlock {
  int l, comp;
};

struct GenericTPInfo {
  const GPath* paths;
  const GNz* nz;
  int np, nk, max_mul;
  int64_t dim1, dim2, dimo;
};

struct GenericSymconInfo {
  const GTerm* terms;
  const GBlock* in_blocks;
  const GBlock* out_blocks;
  int n_terms, n_in_blocks, n_out_blocks, nv, no;
  int64_t numel;
};

int launch_tp_generic(const TPArgs& a, const GenericTPInfo& g);
int launch_symcon_generic(const SymconArgs& a, const GenericSymconInfo& g);

}  // namespace segpoly
