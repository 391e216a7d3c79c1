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
// No atomics, deterministic:
//  K1 (destination-major, like the forward): one wave per (destination
//     node, channel tile) holds the tile of g[node] in registers and walks
//     the node's edges, loading the next edge while computing the current
//     one.  Per edge it writes dw[e], the per-edge source message m[e] (the
//     summand of dx) into a workspace row, and the edge's harmonic gradient
//     reduced over the tile's channels: dsh[e] itself with one tile, else a
//     partial row part[tile][e] that a fold adds up in tile order.  dw and
//     the messages are written once and not re-read by this kernel, so they
//     go out with non-temporal stores (measured 1.12x on the 600k-edge
//     graph: the kernel writes 1.5x the bytes it reads).
//     Edges whose destination lies outside [0, n_nodes) belong to no node:
//     the first node's waves zero those before its range and the last
//     node's waves those after it (dst is sorted), so every output row is
//     written.
//  K2 (source-major): one wave per (source node, channel tile) sums the
//     messages of its edges, taken in the order of src_perm (a stable
//     argsort of src), and writes dx[s] (zero for a source without edges).
//     Its range of src_perm positions comes from the caller's source row
//     pointers when given, else from a search of the sorted sources that a
//     small kernel writes first; K1's destination ranges likewise come
//     from row pointers or from a search of dst.
//  Fold (several tiles only): dsh[e] = sum over tiles of part[tile][e].
// In batch mode (edge e is node e and source e) K1 writes m[e] straight into
// dx and K2 is not launched.
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
// The same over each group of W consecutive lanes (W a power of two, D <=
// W <= 64): afterwards lane L of a group holds the group's total of value
// L / (W / D).
template <typename T, int D, int W = kWave>
__device__ __forceinline__ T wave_sum_many(T (&v)[D]) {
  static_assert(D >= 1 && D <= W && W <= kWave && (D & (D - 1)) == 0 && (W & (W - 1)) == 0,
                "D and W must be powers of two, D <= W <= 64");
  const int lane = threadIdx.x % kWave;
  int n = D;
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) {
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

// Message rows go out through LDS.  In mul_ir a lane's channels lie 2l + 1
// values apart within each block, so every direct store instruction writes
// a part of many cache lines, and with the non-temporal hint lines left the
// cache partly written (1.27x the message bytes on the 600k-edge graph).
// The tile's row is assembled in LDS (`stage`, kWave * CPL * NX values,
// 16-byte aligned) in the handle's layout with the tile width as the
// multiplicity; each slice that is contiguous in both places (a block in
// mul_ir, a component in ir_mul) is then written with 16-byte non-temporal
// stores.  (ir_mul rows are written directly: a lane's channel pair is
// contiguous there, and its stores assemble whole lines in L2.)
using raw16_t = unsigned int __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ void copy_slice_nt(T* __restrict__ gp, const T* __restrict__ sp, int len) {
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  const int lane = threadIdx.x % kWave;
  // sp is 16-byte aligned; gp may not be (then element by element)
  const int nv = (reinterpret_cast<uintptr_t>(gp) % 16) == 0 ? len / V : 0;
  for (int q = lane; q < nv; q += kWave)
    __builtin_nontemporal_store(*reinterpret_cast<const raw16_t*>(sp + q * V), reinterpret_cast<raw16_t*>(gp + q * V));
  for (int q = nv * V + lane; q < len; q += kWave) st1<T, true>(gp + q, sp[q]);
}

template <class S, typename T, int LAYOUT, int CPL>
__device__ __forceinline__ void store_msg_staged(T* __restrict__ grow, T* __restrict__ stage, int mul, int tile0,
                                                 const T (&v)[CPL][S::NX]) {
  constexpr int TW = kWave * CPL;
  const int lane = threadIdx.x % kWave;
  S::template store_xs<T, LAYOUT, CPL, false>(stage, TW, lane * CPL, v);
  __syncthreads();
  const int act = mul - tile0 < TW ? mul - tile0 : TW;
  if constexpr (LAYOUT == kMulIr) {
    int comp = 0;
#pragma unroll
    for (int b = 0; b < S::NXB; ++b) {
      const int d = S::xblock_dim(b);
      copy_slice_nt(grow + static_cast<int64_t>(comp) * mul + static_cast<int64_t>(tile0) * d, stage + comp * TW,
                    act * d);
      comp += d;
    }
  } else {
#pragma unroll
    for (int i = 0; i < S::NX; ++i)
      copy_slice_nt(grow + static_cast<int64_t>(i) * mul + tile0, stage + i * TW, act);
  }
  __syncthreads();
}

// PF: keep the next edge's operands in flight (two channels per lane; with
// one the extra registers cost more occupancy than the overlap gains).
// `dsh_out` is dsh [n_edges][D2] with one tile, else part [tiles][n_edges][D2].
// SHW: one weight row shared by every edge (dw rows still per edge).
template <class S, typename T, typename Index, int LAYOUT, int CPL, bool SHW>
__global__ void __launch_bounds__(kWave)
tp_bwd_edge_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                   const Index* __restrict__ src, const Index* __restrict__ dst, const Index* __restrict__ row_ptr,
                   const T* __restrict__ g, int64_t n_src, int64_t n_edges, int64_t n_nodes, int mul, int batch,
                   int mean, T* __restrict__ dw, T* __restrict__ dsh_out, T* __restrict__ msg) {
  constexpr int DP = Pow2Ceil<S::D2>::value;
  constexpr bool PF = CPL == 2;
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x % kWave;
  const int ub = blockIdx.y * (kWave * CPL) + lane * CPL;
  const bool active = ub < mul;
  const int ubl = active ? ub : 0;
  const int64_t numel = static_cast<int64_t>(mul) * S::NP;
  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;
  T* const hrow = dsh_out + static_cast<int64_t>(blockIdx.y) * n_edges * S::D2;
  __shared__ __align__(16) T stage[LAYOUT == kMulIr ? kWave * CPL * S::NX : 1];
  const int tile0 = blockIdx.y * (kWave * CPL);

  int64_t e0, e1;
  edge_range(dst, n_edges, batch, node, e0, e1, row_ptr);

  auto zero_edge = [&](int64_t e) {
    T z[CPL][S::NX];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int i = 0; i < S::NX; ++i) z[c][i] = T(0);
    if (active) {
#pragma unroll
      for (int p = 0; p < S::NP; ++p) {
        if constexpr (CPL == 2)
          st2<T, true>(dw + e * numel + p * mul + ub, T(0), T(0));
        else
          st1<T, true>(dw + e * numel + p * mul + ub, T(0));
      }
      if constexpr (LAYOUT != kMulIr) S::template store_xs<T, LAYOUT, CPL, true>(msg + e * dim1, mul, ub, z);
    }
    // the staged store needs the whole wave
    if constexpr (LAYOUT == kMulIr) store_msg_staged<S, T, LAYOUT, CPL>(msg + e * dim1, stage, mul, tile0, z);
    if (lane < S::D2) hrow[e * S::D2 + lane] = T(0);
  };
  if (!batch) {
    if (node == 0)
      for (int64_t e = 0; e < e0; ++e) zero_edge(e);
    if (node == n_nodes - 1)
      for (int64_t e = e1; e < n_edges; ++e) zero_edge(e);
  }

  T gv[CPL][S::NK];
  S::template load_gs<T, LAYOUT, CPL>(g + node * (static_cast<int64_t>(mul) * S::NK), mul, ubl, gv);
  if (mean && e1 > e0) {  // the forward divided the row by its number of edges
    const T inv = T(1) / static_cast<T>(e1 - e0);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int k = 0; k < S::NK; ++k) gv[c][k] *= inv;
  }

  auto source = [&](int64_t e) -> int64_t { return batch ? e : static_cast<int64_t>(src[e]); };
  auto load = [&](int64_t e, int64_t s, T (&xv)[CPL][S::NX], T (&wv)[CPL][S::NP], T (&shv)[S::D2]) {
    const int64_t sc = (s >= 0 && s < n_src) ? s : 0;
    S::template load_xs<T, LAYOUT, CPL>(x + sc * dim1, mul, ubl, xv);
    const T* wrow = w + (SHW ? 0 : e * numel) + ubl;
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
  };

  T xn[CPL][S::NX], wn[CPL][S::NP], shn[S::D2];
  int64_t s_next = 0;
  if (PF && e0 < e1) {
    s_next = source(e0);
    load(e0, s_next, xn, wn, shn);
  }
  for (int64_t e = e0; e < e1; ++e) {
    T xv[CPL][S::NX], wv[CPL][S::NP], shv[S::D2];
    int64_t s;
    if constexpr (PF) {
      s = s_next;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
#pragma unroll
        for (int i = 0; i < S::NX; ++i) xv[c][i] = xn[c][i];
#pragma unroll
        for (int p = 0; p < S::NP; ++p) wv[c][p] = wn[c][p];
      }
#pragma unroll
      for (int j = 0; j < S::D2; ++j) shv[j] = shn[j];
      if (e + 1 < e1) {
        s_next = source(e + 1);
        load(e + 1, s_next, xn, wn, shn);
      }
    } else {
      s = source(e);
      load(e, s, xv, wv, shv);
    }
    if (s < 0 || s >= n_src) {
      // the edge contributed nothing: with x and w zeroed every product
      // below is zero, so dw, dsh and the message come out zero
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
#pragma unroll
        for (int i = 0; i < S::NX; ++i) xv[c][i] = T(0);
#pragma unroll
        for (int p = 0; p < S::NP; ++p) wv[c][p] = T(0);
      }
    }

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
          st2<T, true>(dw + e * numel + p * mul + ub, dwv[0][p], dwv[1][p]);
        else
          st1<T, true>(dw + e * numel + p * mul + ub, dwv[0][p]);
      }
      if constexpr (LAYOUT != kMulIr) S::template store_xs<T, LAYOUT, CPL, true>(msg + e * dim1, mul, ub, mxv);
    }
    if constexpr (LAYOUT == kMulIr) store_msg_staged<S, T, LAYOUT, CPL>(msg + e * dim1, stage, mul, tile0, mxv);
    const T tot = wave_sum_many<T, DP>(hsh);
    constexpr int stride = kWave / DP;
    if (lane % stride == 0 && lane / stride < S::D2) hrow[e * S::D2 + lane / stride] = tot;
  }
}

// Edge-parallel form of K1 for multiplicities up to 32 (one channel per
// lane): every output of K1 belongs to one edge (dw[e], dsh[e] and the
// message m[e] need only g[dst[e]], x[src[e]], w[e] and sh[e]), so each
// half-wave takes one edge, with its destination's gradient row loaded per
// edge instead of once per destination.  The destination-major walk visits
// a destination's edges one after another, which on small graphs leaves a
// chain of dependent loads per edge (and half the lanes idle at 32
// channels); here every edge is in flight at once.  The harmonic gradient
// is reduced over the half-wave's lanes.  An edge whose destination or
// source lies outside its range gets zero gradients and a zero message.
// With reduce="mean" the destination's edge count comes from the row
// pointers (the host uses this form then only with them).
constexpr int kHalfWave = 32;

template <class S, typename T, typename Index, int LAYOUT, bool SHW>
__global__ void __launch_bounds__(kWave)
tp_bwd_edge_half_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                        const Index* __restrict__ src, const Index* __restrict__ dst,
                        const Index* __restrict__ row_ptr, const T* __restrict__ g, int64_t n_src,
                        int64_t n_edges, int64_t n_nodes, int mul, int batch, int mean, T* __restrict__ dw,
                        T* __restrict__ dsh, T* __restrict__ msg) {
  constexpr int DP = Pow2Ceil<S::D2>::value;
  static_assert(DP <= kHalfWave, "harmonics wider than a half-wave");
  const int lane = threadIdx.x % kWave;
  const int u = lane % kHalfWave;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 2 + lane / kHalfWave;
  const bool edge_ok = e < n_edges;
  const int64_t ee = edge_ok ? e : n_edges - 1;  // the idle half of an odd count repeats the last edge's loads
  const int ul = u < mul ? u : 0;
  const int64_t numel = static_cast<int64_t>(mul) * S::NP;
  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;
  const int64_t d = batch ? ee : static_cast<int64_t>(dst[ee]);
  const int64_t s = batch ? ee : static_cast<int64_t>(src[ee]);
  const bool ok = d >= 0 && d < n_nodes && s >= 0 && s < n_src;
  T gv[1][S::NK], xv[1][S::NX], wv[1][S::NP], shv[S::D2];
  S::template load_gs<T, LAYOUT, 1>(g + (ok ? d : 0) * (static_cast<int64_t>(mul) * S::NK), mul, ul, gv);
  S::template load_xs<T, LAYOUT, 1>(x + (ok ? s : 0) * dim1, mul, ul, xv);
  const T* wrow = w + (SHW ? 0 : ee * numel) + ul;
#pragma unroll
  for (int p = 0; p < S::NP; ++p) wv[0][p] = __builtin_nontemporal_load(wrow + p * mul);
#pragma unroll
  for (int j = 0; j < S::D2; ++j) shv[j] = sh[ee * S::D2 + j];
  T scale = ok ? T(1) : T(0);  // zero operands give zero gradients and message
  if (mean && ok && row_ptr) {  // the forward divided the row by its number of edges
    const int64_t c = static_cast<int64_t>(row_ptr[d + 1]) - static_cast<int64_t>(row_ptr[d]);
    scale = T(1) / static_cast<T>(c > 0 ? c : 1);
  }
#pragma unroll
  for (int k = 0; k < S::NK; ++k) gv[0][k] *= scale;
  if (!ok) {
#pragma unroll
    for (int i = 0; i < S::NX; ++i) xv[0][i] = T(0);
#pragma unroll
    for (int p = 0; p < S::NP; ++p) wv[0][p] = T(0);
#pragma unroll
    for (int k = 0; k < S::NK; ++k) gv[0][k] = T(0);
  }
  T dwv[1][S::NP];
  T mxv[1][S::NX];
  T hsh[DP];
  S::template bwd<T, 1>(xv, shv, wv, gv, dwv, mxv, reinterpret_cast<T(&)[S::D2]>(hsh));
#pragma unroll
  for (int j = S::D2; j < DP; ++j) hsh[j] = T(0);
  if (!edge_ok || u >= mul) {
#pragma unroll
    for (int j = 0; j < DP; ++j) hsh[j] = T(0);
  }
  if (edge_ok && u < mul) {
#pragma unroll
    for (int p = 0; p < S::NP; ++p) st1<T, true>(dw + e * numel + p * mul + u, dwv[0][p]);
    S::template store_xs<T, LAYOUT, 1, true>(msg + e * dim1, mul, u, mxv);
  }
  const T tot = wave_sum_many<T, DP, kHalfWave>(hsh);
  constexpr int stride = kHalfWave / DP;
  if (edge_ok && u % stride == 0 && u / stride < S::D2) dsh[e * S::D2 + u / stride] = tot;
}

// First i in [lo, hi) with src[perm[i]] >= key (src[perm[.]] ascending),
// by the same wave-cooperative search as the forward.  perm entries outside
// [0, n_edges) compare as +infinity.  (The source sums of the other
// backward kernels; this one searches the contiguous keys below.)
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

// keys[i] = src[perm[i]] clamped to [-1, n_src] (an entry of perm outside
// [0, n_edges) counts as n_src): the sources in sorted order as one
// contiguous int32 array, so that the source kernel's range searches probe
// 2.4 MB that stays in L2 on the 600k-edge graph instead of following
// perm into src at every probe (0.44 GB of L2-miss probes before).
template <typename Index>
__global__ void __launch_bounds__(256)
tp_bwd_keys_kernel(const Index* __restrict__ src, const Index* __restrict__ perm, int64_t n_edges, int64_t n_src,
                   int32_t* __restrict__ keys) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n_edges;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t e = static_cast<int64_t>(perm[i]);
    int64_t k = n_src;
    if (e >= 0 && e < n_edges) {
      const int64_t s = static_cast<int64_t>(src[e]);
      k = s < 0 ? -1 : (s > n_src ? n_src : s);
    }
    keys[i] = static_cast<int32_t>(k);
  }
}

constexpr int kSrcBatch = 4;

template <class S, typename T, typename Index, int LAYOUT, int CPL>
__global__ void __launch_bounds__(kWave)
tp_bwd_src_kernel(const int32_t* __restrict__ keys, const Index* __restrict__ src_row_ptr,
                  const Index* __restrict__ perm, const T* __restrict__ msg, int64_t n_edges, int mul,
                  T* __restrict__ dx) {
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x % kWave;
  const int ub = blockIdx.y * (kWave * CPL) + lane * CPL;
  const bool active = ub < mul;
  const int ubl = active ? ub : 0;
  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;
  // the source's range of perm positions: two loads from the caller's row
  // pointers (clamped to [0, n_edges]), or, as the keys ascend (src_perm
  // sorts the sources), the same wave-cooperative search as the forward's
  // destination ranges
  int64_t i0, i1;
  if (src_row_ptr) {
    const int64_t r0 = static_cast<int64_t>(src_row_ptr[s]);
    const int64_t r1 = static_cast<int64_t>(src_row_ptr[s + 1]);
    i0 = r0 < 0 ? 0 : (r0 > n_edges ? n_edges : r0);
    i1 = r1 < i0 ? i0 : (r1 > n_edges ? n_edges : r1);
  } else {
    i0 = lower_bound_wave(keys, 0, n_edges, s);
    i1 = lower_bound_wave(keys, i0, n_edges, s + 1);
  }
  T acc[CPL][S::NX];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < S::NX; ++i) acc[c][i] = T(0);
  // kSrcBatch edge ids, then their message rows, are loaded before any is
  // summed (several rows in flight per wave); the sum stays in perm order
  constexpr int B = kSrcBatch;
  for (int64_t i = i0; i < i1; i += B) {
    int64_t eb[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int64_t e = i + b < i1 ? static_cast<int64_t>(perm[i + b]) : -1;
      eb[b] = (e >= 0 && e < n_edges) ? e : -1;  // out of range only for an invalid perm
    }
    T m[B][CPL][S::NX];
#pragma unroll
    for (int b = 0; b < B; ++b)
      S::template load_xs<T, LAYOUT, CPL>(msg + (eb[b] >= 0 ? eb[b] : 0) * dim1, mul, ubl, m[b]);
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (eb[b] >= 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int k = 0; k < S::NX; ++k) acc[c][k] += m[b][c][k];
      }
  }
  if (active) S::template store_xs<T, LAYOUT, CPL>(dx + s * dim1, mul, ub, acc);
}

// dsh[i] = part[0][i] + part[1][i] + ... (tile order), i over n_edges * D2.
template <typename T>
__global__ void __launch_bounds__(256)
fold_partials_kernel(const T* __restrict__ part, int tiles, int64_t n, T* __restrict__ dsh) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    T v = part[i];
    for (int t = 1; t < tiles; ++t) v += part[t * n + i];
    dsh[i] = v;
  }
}

// Shared weights: part[c][j] = sum of dwe[e][j] over the edges e of chunk
// c (kTpDwChunk edges, in order); one thread per column j.
template <typename T>
__global__ void __launch_bounds__(256)
dw_edge_sum_kernel(const T* __restrict__ dwe, int64_t n_edges, int64_t numel, T* __restrict__ part) {
  const int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (j >= numel) return;
  const int64_t e0 = blockIdx.y * kTpDwChunk;
  const int64_t e1 = e0 + kTpDwChunk < n_edges ? e0 + kTpDwChunk : n_edges;
  T v = T(0);
  for (int64_t e = e0; e < e1; ++e) v += dwe[e * numel + j];
  part[blockIdx.y * numel + j] = v;
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

// Workspace layout: messages [n_edges][dim1] (not in batch mode), then,
// 256-byte aligned, the harmonic-gradient partials [tiles][n_edges][D2]
// (several tiles only), then (not in batch mode) the sorted source keys
// [n_edges] int32 at keys_ws_off, then the shared-weight rows at dw_ws_off.
// Sizes and offsets come from the C ABI (tp_bwd_ws in capi.cpp).
template <class S, typename T, typename Index, int LAYOUT, int CPL>
int tp_bwd_launch(const TPBwdArgs& a) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int64_t dim1 = static_cast<int64_t>(a.mul) * S::NX;
  const int tiles = (a.mul + kWave * CPL - 1) / (kWave * CPL);
  T* const dx = static_cast<T*>(a.dx);
  T* const dsh = static_cast<T*>(a.dsh);
  const int64_t numel = static_cast<int64_t>(a.mul) * S::NP;
  if (a.n_edges == 0) {  // nothing reaches the output: dx (and a shared dw) is zero
    fill_zero(dx, a.n_src * dim1, st);
    if (a.shared_w) fill_zero(static_cast<T*>(a.dw), numel, st);
    return static_cast<int>(hipGetLastError());
  }
  if (a.n_nodes == 0) {  // every edge has a destination outside the output
    fill_zero(dx, a.n_src * dim1, st);
    fill_zero(static_cast<T*>(a.dw), a.shared_w ? numel : a.n_edges * numel, st);
    fill_zero(dsh, a.n_edges * S::D2, st);
    return static_cast<int>(hipGetLastError());
  }
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  // shared weights: per-edge gradient rows in the workspace, summed below
  T* const dwe = a.shared_w ? reinterpret_cast<T*>(ws + a.dw_ws_off) : static_cast<T*>(a.dw);
  T* const msg = a.batch ? dx : reinterpret_cast<T*>(ws);
  T* const part =
      tiles > 1 ? reinterpret_cast<T*>(ws + (a.batch ? 0 : round_up_256(a.n_edges * dim1 * static_cast<int64_t>(sizeof(T))))) : dsh;
  const dim3 grid(static_cast<unsigned>(a.n_nodes), static_cast<unsigned>(tiles));
  // edge-parallel form: multiplicity up to 32, and with reduce="mean" only
  // when row pointers give the destinations' edge counts (its grid of
  // n_edges / 2 waves stays below 2^32 work-items up to 2^26 edges)
  constexpr bool kHalfOk = CPL == 1 && Pow2Ceil<S::D2>::value <= kHalfWave;
  const bool half = kHalfOk && a.mul <= kHalfWave && (!a.mean || a.row_ptr) && a.n_edges <= (int64_t(1) << 26);
  const dim3 hgrid(static_cast<unsigned>((a.n_edges + 1) / 2));
  if (half && a.shared_w)
    hipLaunchKernelGGL((tp_bwd_edge_half_kernel<S, T, Index, LAYOUT, true>), hgrid, dim3(kWave), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                       static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                       static_cast<const Index*>(a.row_ptr), static_cast<const T*>(a.g), a.n_src, a.n_edges,
                       a.n_nodes, a.mul, a.batch, a.mean, dwe, part, msg);
  else if (half)
    hipLaunchKernelGGL((tp_bwd_edge_half_kernel<S, T, Index, LAYOUT, false>), hgrid, dim3(kWave), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                       static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                       static_cast<const Index*>(a.row_ptr), static_cast<const T*>(a.g), a.n_src, a.n_edges,
                       a.n_nodes, a.mul, a.batch, a.mean, dwe, part, msg);
  else if (a.shared_w)
    hipLaunchKernelGGL((tp_bwd_edge_kernel<S, T, Index, LAYOUT, CPL, true>), grid, dim3(kWave), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                       static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                       static_cast<const Index*>(a.row_ptr), static_cast<const T*>(a.g), a.n_src, a.n_edges,
                       a.n_nodes, a.mul, a.batch, a.mean, dwe, part, msg);
  else
    hipLaunchKernelGGL((tp_bwd_edge_kernel<S, T, Index, LAYOUT, CPL, false>), grid, dim3(kWave), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                       static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                       static_cast<const Index*>(a.row_ptr), static_cast<const T*>(a.g), a.n_src, a.n_edges,
                       a.n_nodes, a.mul, a.batch, a.mean, dwe, part, msg);
  int rc = static_cast<int>(hipGetLastError());
  if (rc) return rc;
  if (a.shared_w) {
    const int64_t chunks = (a.n_edges + kTpDwChunk - 1) / kTpDwChunk;
    T* const dpart = reinterpret_cast<T*>(ws + a.dw_ws_off +
                                          round_up_256(a.n_edges * numel * static_cast<int64_t>(sizeof(T))));
    hipLaunchKernelGGL((dw_edge_sum_kernel<T>), dim3(static_cast<unsigned>((numel + 255) / 256),
                                                     static_cast<unsigned>(chunks)),
                       dim3(256), 0, st, dwe, a.n_edges, numel, dpart);
    const int64_t blocks = (numel + 255) / 256;
    hipLaunchKernelGGL((fold_partials_kernel<T>), dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                       dim3(256), 0, st, dpart, static_cast<int>(chunks), numel, static_cast<T*>(a.dw));
    rc = static_cast<int>(hipGetLastError());
    if (rc) return rc;
  }
  if (tiles > 1) {
    const int64_t n = a.n_edges * S::D2;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL((fold_partials_kernel<T>), dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                       dim3(256), 0, st, part, tiles, n, dsh);
  }
  if (a.batch) {  // rows beyond the batch receive nothing
    fill_zero(dx + a.n_edges * dim1, (a.n_src - a.n_edges) * dim1, st);
  } else if (a.n_src > 0) {
    int32_t* const keys = reinterpret_cast<int32_t*>(ws + a.keys_ws_off);
    if (!a.src_row_ptr) {  // the sorted sources, for the source kernel's range search
      const int64_t blocks = (a.n_edges + 255) / 256;
      hipLaunchKernelGGL((tp_bwd_keys_kernel<Index>), dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                         dim3(256), 0, st, static_cast<const Index*>(a.src), static_cast<const Index*>(a.perm),
                         a.n_edges, a.n_src, keys);
    }
    hipLaunchKernelGGL((tp_bwd_src_kernel<S, T, Index, LAYOUT, CPL>),
                       dim3(static_cast<unsigned>(a.n_src), static_cast<unsigned>(tiles)), dim3(kWave), 0, st,
                       keys, static_cast<const Index*>(a.src_row_ptr), static_cast<const Index*>(a.perm),
                       static_cast<const T*>(a.workspace), a.n_edges, a.mul, dx);
  }
  return static_cast<int>(hipGetLastError());
}

// Two channels per lane (aligned pairs) when the multiplicity fills more
// than one wave with single channels and is even; one otherwise.
template <class S, typename T, typename Index, int LAYOUT>
int tp_bwd_dispatch_cpl(const TPBwdArgs& a) {
  const size_t pa = 2 * sizeof(T);
  // with shared weights the per-edge dw rows (paired stores) sit in the
  // workspace, in batch mode too; a.dw is then written by the fold only
  const void* dwe = a.shared_w ? static_cast<const unsigned char*>(a.workspace) + a.dw_ws_off : a.dw;
  if (a.mul > kWave && a.mul % 2 == 0 && aligned(a.x, pa) && aligned(a.w, pa) && aligned(a.g, pa) &&
      aligned(dwe, pa) && aligned(a.dx, pa) && ((a.batch && !a.shared_w) || aligned(a.workspace, pa)))
    return tp_bwd_launch<S, T, Index, LAYOUT, 2>(a);
  return tp_bwd_launch<S, T, Index, LAYOUT, 1>(a);
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
