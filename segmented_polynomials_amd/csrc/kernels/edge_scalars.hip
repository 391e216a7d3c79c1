// Edge embedding assembly of the convolution layer (cuequivariance-torch
// skill document, "Other operations and layers": the layer's optional
// src_scalars and dst_scalars go with the edge embedding into its edge MLP):
//   out[e] = [edge_emb[e], src_scalars[src[e]], dst_scalars[dst[e]]]
// and the backward: the edge-embedding slice, and the sums of the other two
// slices over the edges that read each source row (source-major, in the
// caller's permutation order) and each destination row (destination-major,
// over the sorted edge ranges).  Deterministic, no atomics.  An index out of
// range gives a zero slice forward and contributes nothing backward.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../edge_scalars.hpp"
#include "../launch.hpp"
#include "tp_conv_bwd.hpp"
#include "tp_conv_spec.hpp"

namespace segpoly {

namespace kern {

// one wave per edge (four per workgroup), lanes over the row's columns
template <typename T, typename Index>
__global__ void __launch_bounds__(256)
edge_scalars_fwd_kernel(const T* __restrict__ emb, const T* __restrict__ ssc, const T* __restrict__ dsc,
                        const Index* __restrict__ src, const Index* __restrict__ dst, int64_t d_emb, int64_t d_src,
                        int64_t d_dst, int64_t n_edges, int64_t n_src, int64_t n_dst, T* __restrict__ out) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (e >= n_edges) return;
  const int64_t d = d_emb + d_src + d_dst;
  T* row = out + e * d;
  for (int64_t c = lane; c < d_emb; c += 64) row[c] = emb[e * d_emb + c];
  if (d_src) {
    const int64_t s = static_cast<int64_t>(src[e]);
    const bool ok = s >= 0 && s < n_src;
    for (int64_t c = lane; c < d_src; c += 64) row[d_emb + c] = ok ? ssc[s * d_src + c] : T(0);
  }
  if (d_dst) {
    const int64_t n = static_cast<int64_t>(dst[e]);
    const bool ok = n >= 0 && n < n_dst;
    for (int64_t c = lane; c < d_dst; c += 64) row[d_emb + d_src + c] = ok ? dsc[n * d_dst + c] : T(0);
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
edge_scalars_emb_grad_kernel(const T* __restrict__ g, int64_t d, int64_t d_emb, int64_t n_edges,
                             T* __restrict__ gemb) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (e >= n_edges) return;
  for (int64_t c = lane; c < d_emb; c += 64) gemb[e * d_emb + c] = g[e * d + c];
}

// gsrc[s] = sum over the edges with src = s (in permutation order) of g[e][col0 ..]
template <typename T, typename Index>
__global__ void __launch_bounds__(64)
edge_scalars_src_grad_kernel(const T* __restrict__ g, const Index* __restrict__ src, const Index* __restrict__ perm,
                             int64_t d, int64_t col0, int64_t width, int64_t n_edges, T* __restrict__ gsrc) {
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t i0 = lower_bound_perm(src, perm, n_edges, 0, n_edges, s);
  const int64_t i1 = lower_bound_perm(src, perm, n_edges, i0, n_edges, s + 1);
  for (int64_t c = lane; c < width; c += 64) {
    T acc = T(0);
    for (int64_t i = i0; i < i1; ++i) {
      const int64_t e = static_cast<int64_t>(perm[i]);
      if (e < 0 || e >= n_edges) continue;  // only an invalid permutation gets here
      acc += g[e * d + col0 + c];
    }
    gsrc[s * width + c] = acc;
  }
}

// gdst[n] = sum over the edges of n's (sorted) range of g[e][col0 ..]
template <typename T, typename Index>
__global__ void __launch_bounds__(64)
edge_scalars_dst_grad_kernel(const T* __restrict__ g, const Index* __restrict__ dst, int64_t d, int64_t col0,
                             int64_t width, int64_t n_edges, T* __restrict__ gdst) {
  const int64_t n = blockIdx.x;
  const int lane = threadIdx.x;
  int64_t e0, e1;
  edge_range(dst, n_edges, 0, n, e0, e1);
  for (int64_t c = lane; c < width; c += 64) {
    T acc = T(0);
    for (int64_t e = e0; e < e1; ++e) acc += g[e * d + col0 + c];
    gdst[n * width + c] = acc;
  }
}

template <typename T, typename Index>
int edge_scalars_launch(const EdgeScalarArgs& a, bool backward) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int64_t d = a.d_emb + a.d_src + a.d_dst;
  const unsigned eblocks = static_cast<unsigned>((a.n_edges + 3) / 4);
  if (!backward) {
    if (a.n_edges > 0)
      hipLaunchKernelGGL((edge_scalars_fwd_kernel<T, Index>), dim3(eblocks), dim3(256), 0, st,
                         static_cast<const T*>(a.emb), static_cast<const T*>(a.ssc), static_cast<const T*>(a.dsc),
                         static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst), a.d_emb, a.d_src, a.d_dst,
                         a.n_edges, a.n_src, a.n_dst, static_cast<T*>(a.out));
    return static_cast<int>(hipGetLastError());
  }
  if (a.n_edges > 0 && a.d_emb > 0)
    hipLaunchKernelGGL((edge_scalars_emb_grad_kernel<T>), dim3(eblocks), dim3(256), 0, st,
                       static_cast<const T*>(a.g), d, a.d_emb, a.n_edges, static_cast<T*>(a.gemb));
  if (a.d_src > 0 && a.n_src > 0)
    hipLaunchKernelGGL((edge_scalars_src_grad_kernel<T, Index>), dim3(static_cast<unsigned>(a.n_src)), dim3(64), 0, st,
                       static_cast<const T*>(a.g), static_cast<const Index*>(a.src),
                       static_cast<const Index*>(a.perm), d, a.d_emb, a.d_src, a.n_edges, static_cast<T*>(a.gsrc));
  if (a.d_dst > 0 && a.n_dst > 0)
    hipLaunchKernelGGL((edge_scalars_dst_grad_kernel<T, Index>), dim3(static_cast<unsigned>(a.n_dst)), dim3(64), 0, st,
                       static_cast<const T*>(a.g), static_cast<const Index*>(a.dst), d, a.d_emb + a.d_src, a.d_dst,
                       a.n_edges, static_cast<T*>(a.gdst));
  return static_cast<int>(hipGetLastError());
}

}  // namespace kern

int launch_edge_scalars(const EdgeScalarArgs& a, bool backward) {
  using namespace kern;
  if (a.dtype == kF32)
    return a.idx == kI64 ? edge_scalars_launch<float, int64_t>(a, backward) : edge_scalars_launch<float, int32_t>(a, backward);
  return a.idx == kI64 ? edge_scalars_launch<double, int64_t>(a, backward) : edge_scalars_launch<double, int32_t>(a, backward);
}

}  // namespace segpoly
