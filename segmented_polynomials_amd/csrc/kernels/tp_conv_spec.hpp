// Fused channelwise tensor-product convolution, specialised kernels (gfx950).
//
// One launch covers every (l1, l2, lo) path of the descriptor (e3nn-course
// Lesson 12a, sections 21.1 and 21.6: one fused kernel instead of one launch
// and one global-memory intermediate per path).  For each destination node n
// and channel u:
//   out[n, path p, k, u] = sum over edges e with dst[e] = n of
//       w[e, woff_p + u] * sum_ij C_p[i, j, k] x[src[e], blk1_p, i, u] sh[e, blk2_p, j]
// (cuequivariance-torch skill document, "SegmentedPolynomial: gather and
// scatter": repeated receivers sum, receivers without edges stay zero).
//
// Work decomposition: one wavefront (64 lanes) per (destination node,
// channel tile of 64*CPL channels); lane = channel, CPL channels per lane.
// The wave finds its node's edge range [e0, e1) in the dst-sorted edge list
// by two uniform binary searches, then walks the edges in order keeping
// every output component of its channels in registers, and writes each
// output row exactly once (zeros for an isolated node).  No atomics: the
// reduction order is the edge order, so results are deterministic.
//
// Per edge: src[e] and sh[e, :] are wave-uniform (scalar loads); the
// uniform products c * sh_j of the coupling coefficients are formed once per
// edge (S::coef) and shared by all channels of the wave; the weights
// w[e, p*mul + u] and the gathered features x[src, ...] are channel-
// contiguous vector loads.  The coupling coefficients are literal constants
// in S::coef / S::edge (generated per descriptor), so zeros cost nothing.
//
// S (generated) provides: NX (input-1 components per channel), NK (output
// components per channel), NP (paths), D2 (width of sh), NQ (uniform
// products); coef(sh_row, q); load_x<T, LAYOUT>(x_row, mul, u, xv);
// edge(xv, q, wv, acc); store<T, LAYOUT>(out_row, mul, u, acc).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "common.hpp"

namespace segpoly {
namespace kern {

constexpr int kWave = 64;

// First e in [lo, hi) with dst[e] >= key, dst sorted ascending.  All
// operands are wave-uniform, so this runs on the scalar unit.
template <typename Index>
__device__ __forceinline__ int64_t lower_bound_idx(const Index* __restrict__ dst, int64_t lo,
                                                   int64_t hi, int64_t key) {
  while (lo < hi) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if (static_cast<int64_t>(dst[mid]) < key)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

template <class S, typename T, typename Index, int LAYOUT, int CPL>
__global__ void __launch_bounds__(kWave)
tp_conv_spec_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                    const Index* __restrict__ src, const Index* __restrict__ dst, int64_t n_src,
                    int64_t n_edges, int64_t w_stride, int mul, int batch, T* __restrict__ out) {
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x;
  const int tile0 = blockIdx.y * (kWave * CPL);

  int64_t e0, e1;
  if (batch) {  // batch mode: edge e is node e
    e0 = node;
    e1 = node + 1;
  } else {
    e0 = lower_bound_idx(dst, 0, n_edges, node);
    e1 = lower_bound_idx(dst, e0, n_edges, node + 1);
  }

  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;
  T acc[CPL][S::NK];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int k = 0; k < S::NK; ++k) acc[c][k] = T(0);

  for (int64_t e = e0; e < e1; ++e) {
    const int64_t s = batch ? e : static_cast<int64_t>(src[e]);
    if (s < 0 || s >= n_src) continue;  // out-of-range sources contribute nothing
    T q[S::NQ];
    S::template coef<T>(sh + e * S::D2, q);
    const T* xrow = x + s * dim1;
    const T* wrow = w + e * w_stride;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int u = tile0 + c * kWave + lane;
      if (u < mul) {
        T xv[S::NX];
        T wv[S::NP];
        S::template load_x<T, LAYOUT>(xrow, mul, u, xv);
#pragma unroll
        for (int p = 0; p < S::NP; ++p) wv[p] = wrow[p * mul + u];
        S::template edge<T>(xv, q, wv, acc[c]);
      }
    }
  }

  T* orow = out + node * (static_cast<int64_t>(mul) * S::NK);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int u = tile0 + c * kWave + lane;
    if (u < mul) S::template store<T, LAYOUT>(orow, mul, u, acc[c]);
  }
}

template <class S, typename T, typename Index, int LAYOUT, int CPL>
int tp_conv_spec_launch(const TPArgs& a) {
  const int per_tile = kWave * CPL;
  dim3 grid(static_cast<unsigned>(a.n_nodes), static_cast<unsigned>((a.mul + per_tile - 1) / per_tile));
  hipLaunchKernelGGL((tp_conv_spec_kernel<S, T, Index, LAYOUT, CPL>), grid, dim3(kWave), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x),
                     static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                     static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst), a.n_src,
                     a.n_edges, a.w_stride, a.mul, a.batch, static_cast<T*>(a.out));
  return static_cast<int>(hipGetLastError());
}

template <class S, typename T, typename Index, int LAYOUT>
int tp_conv_spec_dispatch_cpl(const TPArgs& a) {
  if (a.mul > kWave) return tp_conv_spec_launch<S, T, Index, LAYOUT, 2>(a);
  return tp_conv_spec_launch<S, T, Index, LAYOUT, 1>(a);
}

template <class S, typename T>
int tp_conv_spec_dispatch(const TPArgs& a) {
  if (a.idx == kI32) {
    if (a.layout == kMulIr) return tp_conv_spec_dispatch_cpl<S, T, int32_t, kMulIr>(a);
    return tp_conv_spec_dispatch_cpl<S, T, int32_t, kIrMul>(a);
  }
  if (a.layout == kMulIr) return tp_conv_spec_dispatch_cpl<S, T, int64_t, kMulIr>(a);
  return tp_conv_spec_dispatch_cpl<S, T, int64_t, kIrMul>(a);
}

}  // namespace kern
}  // namespace segpoly
