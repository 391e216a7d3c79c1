// Arguments of the edge-embedding assembly kernels (host and device).
#pragma once
#include <cstdint>

namespace segpoly {

struct EdgeScalarArgs {
  const void* emb;
  const void* ssc;
  const void* dsc;
  const void* src;
  const void* dst;
  const void* perm;
  const void* g;
  void* out;
  void* gemb;
  void* gsrc;
  void* gdst;
  int64_t d_emb, d_src, d_dst, n_edges, n_src, n_dst;
  int dtype, idx;
  void* stream;
};

int launch_edge_scalars(const EdgeScalarArgs& a, bool backward);

}  // namespace segpoly
