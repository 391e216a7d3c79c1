// Device-side tables of the table-driven kernels (plain structs, uploaded
// once per device by the C ABI).
#pragma once
#include <cstddef>
#include <cstdint>

#include "launch.hpp"

namespace segpoly {

struct GPath {
  int l1, lo, mul, nz_begin, nz_end, kcomp, xcomp, pad1;
  int64_t off1, off2, offo, woff;
};

// an input-1 block of the tensor product (for the backward's dx rows)
struct GIn {
  int l, comp, mul, pad;
  int64_t off;
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
  const GIn* in;      // input-1 blocks (backward only)
  int np, nk, max_mul, n_in, nx;
  int64_t dim1, dim2, dimo, numel;
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
// backward of the table-driven products (no workspace but the shared-weight
// rows and their chunk sums, laid out as for the generated kernels)
int launch_tp_generic_bwd(const TPBwdArgs& a, const GenericTPInfo& g);
// rp[n] = first i with key(i) >= n, n = 0 .. n_nodes; key(i) = keys[i]
// (sorted destinations), or keys[perm[i]] when perm is given (the sources
// in src_perm order)
int launch_rowptr_build(const void* keys, const void* perm, int idx, int64_t n_edges, int64_t n_nodes, void* rp,
                        void* stream);
int launch_symcon_generic_bwd(const SymconBwdArgs& a, const GenericSymconInfo& g);
// LDS the table-driven backward kernels need (bytes), for the C ABI's checks
size_t tp_generic_bwd_lds(int nx, int64_t dim2, int dtype);
size_t symcon_generic_bwd_lds(int nv, int no, int nseg, int dtype);

}  // namespace segpoly
