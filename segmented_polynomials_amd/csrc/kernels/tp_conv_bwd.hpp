// Backward (vector-Jacobian product) of the fused channelwise
// tensor-product convolution, specialised kernels (gfx950).
//
// Given g = dL/d(out), with the forward out[n] = sum_{e: dst[e] = n} of
// w[e] * C(x[src[e]], sh[e]) over every path (cuequivariance-torch skill
// document, "CPU tensor product and backward" and "SegmentedPolynomial:
// gather and scatter", which check gradients of every operand):
//   dw[e, p, u]  = sum_k g[dst_e, p, k, u] sum_ij C_p[i,j,k] x[src_e, i, u] sh[e, j]
//   dsh[e, j]    = sum_{p, u} w[e, p, u] sum_ik C_p[i,j,k] x[src_e, i, u] g[dst_e, p, k, u]
//   dx[s, i, u]  = sum_{e: src_e = s} sum_p w[e, p, u] sum_jk C_p[i,j,k] sh[e, j] g[dst_e, p, k, u]
//
// Two launches, no atomics, deterministic:
//  K1 (destination-major, like the forward): one wave per destination node
//     holds g[node] in registers and walks the node's edges; per edge it
//     writes dw[e], the per-edge source message m[e] (the summand of dx) into
//     a workspace row, and dsh[e] after reducing over the wave's channels.
//     Edges whose destination lies outside [0, n_nodes) belong to no node:
//     the first node's wave zeroes those before its range and the last
//     node's wave those after it (dst is sorted), so every output row is
//     written.
//  K2 (source-major): one wave per source node sums the messages of its
//     edges, taken in the order of src_perm (a stable argsort of src), and
//     writes dx[s] (zero for a source without edges).
// In batch mode (edge e is node e and source e) K1 writes m[e] straight into
// dx and K2 is not launched.
//
// One channel tile per wave (mul <= 64, or <= 128 in aligned pairs): dsh is
// a reduction over all channels of an edge.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "common.hpp"
#include "tp_conv_spec.hpp"

namespace segpoly {
namespace kern {

// Sums over the 64 lanes of each of D values per lane (D a power of two,
// <= 64), by recursive halving: at each of the first log2(D) butterfly steps
// a lane keeps half of its values (the upper half when its partner bit is
// set) and adds the partner's copy of that half; the remaining steps are a
// plain butterfly.  D - 1 + 6 - log2(D) shuffles in all.  Afterwards every
// lane L holds the total of value L / (64 / D).
template <typename T, int D>
__device__ __forceinline__ T wave_sum_many(T (&v)[D]) {
  static_assert(D >= 1 && D <= kWave && (D & (D - 1)) == 0, "D must be a power of two <= 64");
  const int lane = threadIdx.x % kWave;
  int n = D;
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    if (n > 1) {
      const bool upper = lane & off;
#pragma unroll
      for (int i = 0; i < D / 2; ++i) {
        if (i < n / 2) {
          const T lo = v[i], hi = v[i + n / 2];
          const T give = upper ? lo : hi;
          const T keep = upper ? hi : lo;
          v[i] = keep + __shfl_xor(give, off);
        }
      }
      n >>= 1;
    } else {
      v[0] += __shfl_xor(v[0], off);
    }
  }
  return v[0];
}

template <int N>
struct Pow2Ceil {
  static constexpr int value = N <= 1 ? 1 : 2 * Pow2Ceil<(N + 1) / 2>::value;
};
template <>
struct Pow2Ceil<1> {
  static constexpr int value = 1;
};

template <class S, typename T, typename Index, int LAYOUT, int CPL>
__global__ void __launch_bounds__(kWave)
tp_bwd_edge_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                   const Index* __restrict__ src, const Index* __restrict__ dst, const T* __restrict__ g,
                   int64_t n_src, int64_t n_edges, int64_t n_nodes, int mul, int batch, T* __restrict__ dw,
                   T* __restrict__ dsh, T* __restrict__ msg) {
  constexpr int DP = Pow2Ceil<S::D2>::value;
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x % kWave;
  const int ub = lane * CPL;
  const bool active = ub < mul;
  const int ubl = active ? ub : 0;
  const int64_t numel = static_cast<int64_t>(mul) * S::NP;
  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;

  int64_t e0, e1;
  edge_range(dst, n_edges, batch, node, e0, e1);

  auto zero_edge = [&](int64_t e) {
    if (active) {
#pragma unroll
      for (int p = 0; p < S::NP; ++p) {
        if constexpr (CPL == 2)
          st2<T, false>(dw + e * numel + p * mul + ub, T(0), T(0));
        else
          dw[e * numel + p * mul + ub] = T(0);
      }
      T z[CPL][S::NX];
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int i = 0; i < S::NX; ++i) z[c][i] = T(0);
      S::template store_xs<T, LAYOUT, CPL>(msg + e * dim1, mul, ub, z);
    }
    if (lane < S::D2) dsh[e * S::D2 + lane] = T(0);
  };
  if (!batch) {
    if (node == 0)
      for (int64_t e = 0; e < e0; ++e) zero_edge(e);
    if (node == n_nodes - 1)
      for (int64_t e = e1; e < n_edges; ++e) zero_edge(e);
  }

  T gv[CPL][S::NK];
  S::template load_gs<T, LAYOUT, CPL>(g + node * (static_cast<int64_t>(mul) * S::NK), mul, ubl, gv);

  for (int64_t e = e0; e < e1; ++e) {
    const int64_t s = batch ? e : static_cast<int64_t>(src[e]);
    if (s < 0 || s >= n_src) {  // the edge contributed nothing: zero gradients
      zero_edge(e);
      continue;
    }
    T xv[CPL][S::NX];
    T wv[CPL][S::NP];
    T shv[S::D2];
    S::template load_xs<T, LAYOUT, CPL>(x + s * dim1, mul, ubl, xv);
    const T* wrow = w + e * numel + ubl;
#pragma unroll
    for (int p = 0; p < S::NP; ++p) {
      if constexpr (CPL == 2) {
        const auto t = ld2<T, true>(wrow + p * mul);
        wv[0][p] = t.x;
        wv[1][p] = t.y;
      } else {
        wv[0][p] = __builtin_nontemporal_load(wrow + p * mul);
      }
    }
#pragma unroll
    for (int j = 0; j < S::D2; ++j) shv[j] = sh[e * S::D2 + j];

    T dwv[CPL][S::NP];
    T mxv[CPL][S::NX];
    T hsh[DP];
    S::template bwd<T, CPL>(xv, shv, wv, gv, dwv, mxv, reinterpret_cast<T(&)[S::D2]>(hsh));
#pragma unroll
    for (int j = S::D2; j < DP; ++j) hsh[j] = T(0);
    if (!active) {
#pragma unroll
      for (int j = 0; j < DP; ++j) hsh[j] = T(0);
    }

    if (active) {
#pragma unroll
      for (int p = 0; p < S::NP; ++p) {
        if constexpr (CPL == 2)
          st2<T, false>(dw + e * numel + p * mul + ub, dwv[0][p], dwv[1][p]);
        else
          dw[e * numel + p * mul + ub] = dwv[0][p];
      }
      S::template store_xs<T, LAYOUT, CPL>(msg + e * dim1, mul, ub, mxv);
    }
    const T tot = wave_sum_many<T, DP>(hsh);
    constexpr int stride = kWave / DP;
    if (lane % stride == 0 && lane / stride < S::D2) dsh[e * S::D2 + lane / stride] = tot;
  }
}

// First i in [lo, hi) with src[perm[i]] >= key (src[perm[.]] ascending),
// by the same wave-cooperative search as the forward.  perm entries outside
// [0, n_edges) compare as +infinity.
template <typename Index>
__device__ __forceinline__ int64_t lower_bound_perm(const Index* __restrict__ src, const Index* __restrict__ perm,
                                                    int64_t n_edges, int64_t lo, int64_t hi, int64_t key) {
  const int lane = threadIdx.x % kWave;
  auto below = [&](int64_t i) -> bool {
    if (i >= hi) return false;
    const int64_t e = static_cast<int64_t>(perm[i]);
    return e >= 0 && e < n_edges && static_cast<int64_t>(src[e]) < key;
  };
  while (hi - lo > kWave) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    const int c = __popcll(__ballot(below(lo + lane * step)));
    const int64_t nlo = c == 0 ? lo : lo + (c - 1) * step + 1;
    const int64_t nhi = lo + c * step < hi ? lo + c * step : hi;
    lo = nlo;
    hi = nhi;
  }
  return lo + __popcll(__ballot(below(lo + lane)));
}

template <class S, typename T, typename Index, int LAYOUT, int CPL>
__global__ void __launch_bounds__(kWave)
tp_bwd_src_kernel(const Index* __restrict__ src, const Index* __restrict__ perm, const T* __restrict__ msg,
                  int64_t n_edges, int mul, T* __restrict__ dx) {
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x % kWave;
  const int ub = lane * CPL;
  const bool active = ub < mul;
  const int ubl = active ? ub : 0;
  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;
  const int64_t i0 = lower_bound_perm(src, perm, n_edges, 0, n_edges, s);
  const int64_t i1 = lower_bound_perm(src, perm, n_edges, i0, n_edges, s + 1);
  T acc[CPL][S::NX];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < S::NX; ++i) acc[c][i] = T(0);
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t e = static_cast<int64_t>(perm[i]);
    if (e < 0 || e >= n_edges) continue;  // only an invalid perm gets here
    T m[CPL][S::NX];
    S::template load_xs<T, LAYOUT, CPL>(msg + e * dim1, mul, ubl, m);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int k = 0; k < S::NX; ++k) acc[c][k] += m[c][k];
  }
  if (active) S::template store_xs<T, LAYOUT, CPL>(dx + s * dim1, mul, ub, acc);
}

template <typename T>
__global__ void __launch_bounds__(256) fill_zero_kernel(T* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = T(0);
}

template <typename T>
void fill_zero(T* p, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL((fill_zero_kernel<T>), dim3(static_cast<unsigned>(blocks < 2048 ? blocks : 2048)), dim3(256), 0,
                     st, p, n);
}

template <class S, typename T, typename Index, int LAYOUT, int CPL>
int tp_bwd_launch(const TPBwdArgs& a) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int64_t dim1 = static_cast<int64_t>(a.mul) * S::NX;
  T* const dx = static_cast<T*>(a.dx);
  if (a.n_edges == 0) {  // nothing reaches the output: dx is zero
    fill_zero(dx, a.n_src * dim1, st);
    return static_cast<int>(hipGetLastError());
  }
  if (a.n_nodes == 0) {  // every edge has a destination outside the output
    fill_zero(dx, a.n_src * dim1, st);
    fill_zero(static_cast<T*>(a.dw), a.n_edges * static_cast<int64_t>(a.mul) * S::NP, st);
    fill_zero(static_cast<T*>(a.dsh), a.n_edges * S::D2, st);
    return static_cast<int>(hipGetLastError());
  }
  T* const msg = a.batch ? dx : static_cast<T*>(a.workspace);
  hipLaunchKernelGGL((tp_bwd_edge_kernel<S, T, Index, LAYOUT, CPL>), dim3(static_cast<unsigned>(a.n_nodes)),
                     dim3(kWave), 0, st, static_cast<const T*>(a.x), static_cast<const T*>(a.sh),
                     static_cast<const T*>(a.w), static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                     static_cast<const T*>(a.g), a.n_src, a.n_edges, a.n_nodes, a.mul, a.batch,
                     static_cast<T*>(a.dw), static_cast<T*>(a.dsh), msg);
  int rc = static_cast<int>(hipGetLastError());
  if (rc) return rc;
  if (a.batch) {  // rows beyond the batch receive nothing
    fill_zero(dx + a.n_edges * dim1, (a.n_src - a.n_edges) * dim1, st);
  } else if (a.n_src > 0) {
    hipLaunchKernelGGL((tp_bwd_src_kernel<S, T, Index, LAYOUT, CPL>), dim3(static_cast<unsigned>(a.n_src)),
                       dim3(kWave), 0, st, static_cast<const Index*>(a.src), static_cast<const Index*>(a.perm),
                       static_cast<const T*>(a.workspace), a.n_edges, a.mul, dx);
  }
  return static_cast<int>(hipGetLastError());
}

// Returned when one wave cannot cover the multiplicity.
constexpr int kBwdNoTile = -2;

// One channel per lane up to 64 channels; two (aligned pairs) up to 128.
template <class S, typename T, typename Index, int LAYOUT>
int tp_bwd_dispatch_cpl(const TPBwdArgs& a) {
  if (a.mul <= kWave) return tp_bwd_launch<S, T, Index, LAYOUT, 1>(a);
  const size_t pa = 2 * sizeof(T);
  if (a.mul <= 2 * kWave && a.mul % 2 == 0 && aligned(a.x, pa) && aligned(a.w, pa) && aligned(a.g, pa) &&
      aligned(a.dw, pa) && aligned(a.dx, pa) && (a.batch || aligned(a.workspace, pa)))
    return tp_bwd_launch<S, T, Index, LAYOUT, 2>(a);
  return kBwdNoTile;
}

template <class S, typename T>
int tp_bwd_dispatch(const TPBwdArgs& a) {
  if (a.idx == kI32) {
    if (a.layout == kMulIr) return tp_bwd_dispatch_cpl<S, T, int32_t, kMulIr>(a);
    return tp_bwd_dispatch_cpl<S, T, int32_t, kIrMul>(a);
  }
  if (a.layout == kMulIr) return tp_bwd_dispatch_cpl<S, T, int64_t, kMulIr>(a);
  return tp_bwd_dispatch_cpl<S, T, int64_t, kIrMul>(a);
}

}  // namespace kern
}  // namespace segpoly
