// Tables of the fully connected product with one weight row per sample
// (external per-item weights, [n, weight_numel]): built on the host from the
// descriptor, uploaded once per device with the handle's other tables.
//
// Per sample s, output block o and path p = (i, j, o):
//   out[s, o, k, w] += sum_(u, v) W_s[p][u, v, w] A[k, u, v],
//   A[k, u, v] = alpha_o sum over the entries (a, b) of k of C[a, b, k] x1[s, i, a, u] x2[s, j, b, v].
// Every weight is used by one sample only, so the product streams the
// weight rows.  A tile is one output block and up to 64 of its channels w;
// the (u, v) pairs of a path are taken 64 at a time (a "chunk").
#pragma once
#include <cstdint>

#include "launch.hpp"

namespace segpoly {

constexpr int kPsMaxD = 13;      // components of an output block (l <= 6)
constexpr int kPsChunk = 64;     // (u, v) pairs per chunk: one per lane when forming A
constexpr int kPsLdsLimit = 64 * 1024;

struct PsPath {
  int64_t woff;                  // weight segment in a row: [m1][m2][m3], w fastest
  int off1, off2;                // input blocks in the x1 and x2 rows
  int m1, m2, d1, d2;
  int k_list;                    // its d3 entry lists by output component (PsList)
  int a_list;                    // its d1 entry lists by input-1 component
  int b_list;                    // its d2 entry lists by input-2 component
  int pad;
};

struct PsList {
  int begin, end;                // a range of PsEnt
};

struct PsEnt {
  int a, b, k, pad;              // input-1, input-2 and output components
  double c;                      // coefficient C[a, b, k], alpha_o included
};

struct PsTile {
  int offo;                      // output block offset in a row
  int d3, m3, w0, nw;            // components, channels, channel range of the tile
  int path_begin, path_end;      // paths into the block
  int lane_bits;                 // log2 of the lanes per (u, v) pair (nw rounded up to a power of two)
};

struct FcPsArgs {
  const void* x1;                // [n, dim1]
  const void* x2;                // [n, dim2]
  const void* w;                 // [n, numel]
  const void* g;                 // backward: dL/d(out) [n, dimo]
  void* out;                     // forward [n, dimo]
  void* dx1;                     // backward, each may be null
  void* dx2;
  void* dw;                      // [n, numel]
  int64_t n, dim1, dim2, dimo, numel;
  const PsTile* tiles;           // device tables
  const PsPath* paths;
  const PsList* lists;
  const PsEnt* ents;
  int n_tiles, max_d;
  int vec;                       // backward: weight rows read and written in 16-byte pieces (aligned rows)
  size_t lds_bytes;
  int dtype, layout;
  void* stream;
};

// LDS of one workgroup (one wave): the sample's two input rows and one chunk
// of coupled values (forward); in the backward the two input rows, the two
// input-gradient rows, the tile's output gradient (64 channels per output
// component) and one chunk of weight-contracted values.
inline size_t ps_lds_fwd(int64_t dim1, int64_t dim2, int max_d, size_t elt) {
  return static_cast<size_t>(dim1 + dim2 + static_cast<int64_t>(kPsChunk) * max_d) * elt;
}
inline size_t ps_lds_bwd(int64_t dim1, int64_t dim2, int max_d, size_t elt) {
  return static_cast<size_t>(2 * (dim1 + dim2) + 2 * static_cast<int64_t>(kPsChunk) * max_d) * elt;
}

int launch_fctp_ps_fwd(const FcPsArgs& a);
int launch_fctp_ps_bwd(const FcPsArgs& a);

}  // namespace segpoly
