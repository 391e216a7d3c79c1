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
// channel tile of 64*CPL channels); each lane owns CPL adjacent channels
// (CPL = 2: every operand row is read as one aligned pair per lane).  The
// wave finds its node's edge range [e0, e1) in the dst-sorted edge list with
// a wave-cooperative 64-ary search, then walks the edges in order keeping
// every output component of its channels in registers, and writes each
// output row exactly once (zeros for an isolated node).  No atomics: the
// reduction order is the edge order, so results are deterministic.
//
// Per edge the loads of the next edge (its weights, the gathered source row,
// its harmonics) are issued before the current edge is computed, so one
// edge of traffic per wave is always in flight.  The weights are streamed
// once and carry the non-temporal hint.  Each path forms its uniform
// coefficient products c * sh_j just before use; the coefficients are
// literal constants in the generated S::edge, so zeros cost nothing.
//
// S (generated) provides NX (input-1 components per channel), NK (output
// components per channel), NP (paths), D2 (width of sh);
// load_xs<T, LAYOUT, CPL>(x_row, mul, u0, xv), edge<T, CPL>(xv, sh, wv, acc),
// store_s<T, LAYOUT, CPL>(out_row, mul, u0, acc).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "common.hpp"
#include "sh.hpp"

namespace segpoly {
namespace kern {

constexpr int kWave = 64;

// First e in [lo, hi) with dst[e] >= key, dst sorted ascending, found by
// the whole wave: each round every lane probes one of 64 evenly spaced
// positions and a ballot narrows [lo, hi) 64-fold, so about four dependent
// loads cover 10^6 edges.  Must be called by all 64 lanes together.
template <typename Index>
__device__ __forceinline__ int64_t lower_bound_wave(const Index* __restrict__ dst, int64_t lo, int64_t hi,
                                                    int64_t key) {
  const int lane = threadIdx.x % kWave;
  while (hi - lo > kWave) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    const int64_t idx = lo + lane * step;
    const bool below = idx < hi && static_cast<int64_t>(dst[idx]) < key;
    const int c = __popcll(__ballot(below));  // probes 0..c-1 are below key
    const int64_t nlo = c == 0 ? lo : lo + (c - 1) * step + 1;
    const int64_t nhi = lo + c * step < hi ? lo + c * step : hi;
    lo = nlo;
    hi = nhi;
  }
  const int64_t idx = lo + lane;
  const bool below = idx < hi && static_cast<int64_t>(dst[idx]) < key;
  return lo + __popcll(__ballot(below));
}

// lower_bound_wave from a position known to be at or below the answer,
// trying the 64 positions after it first: a node's edges usually end within
// 64 of where they start, and then one round of probes finds the end.
template <typename Index>
__device__ __forceinline__ int64_t lower_bound_wave_near(const Index* __restrict__ dst, int64_t lo, int64_t hi,
                                                         int64_t key) {
  const int lane = threadIdx.x % kWave;
  const int64_t idx = lo + lane;
  const bool below = idx < hi && static_cast<int64_t>(dst[idx]) < key;
  const int c = __popcll(__ballot(below));
  if (c < kWave || lo + kWave >= hi) return lo + c;  // the first position not below key is lo + c
  return lower_bound_wave(dst, lo + kWave, hi, key);
}

// Edge range of `node` (batch mode: edge e is node e).  With the caller's
// row pointers rp (rp[n] = first edge of destination n, rp[n_nodes] =
// n_edges) two independent loads replace the search; values are clamped to
// 0 <= e0 <= e1 <= n_edges, so inconsistent pointers cannot reach outside
// the edge arrays.
template <typename Index>
__device__ __forceinline__ void edge_range(const Index* __restrict__ dst, int64_t n_edges, int batch, int64_t node,
                                           int64_t& e0, int64_t& e1, const Index* __restrict__ rp = nullptr) {
  if (batch) {
    e0 = node;
    e1 = node + 1;
  } else if (rp) {
    const int64_t a = static_cast<int64_t>(rp[node]), b = static_cast<int64_t>(rp[node + 1]);
    e0 = a < 0 ? 0 : (a > n_edges ? n_edges : a);
    e1 = b < e0 ? e0 : (b > n_edges ? n_edges : b);
  } else {
    e0 = lower_bound_wave(dst, 0, n_edges, node);
    e1 = lower_bound_wave_near(dst, e0, n_edges, node + 1);
  }
}

// Requires mul % CPL == 0 and x, w, out aligned to CPL * sizeof(T).  NTS:
// non-temporal output stores (measured neutral on the 600k-edge graph, so
// off by default).
// l_max of a harmonics operand of width (l_max + 1)^2
constexpr int sh_lmax_of(int d2) {
  int l = 0;
  while ((l + 2) * (l + 2) <= d2) ++l;
  return l;
}

// SHV: the second operand is computed from the edge vectors vec [n_edges, 3]
// (degrees 0..L with D2 = (L + 1)^2) as the edge's operands are loaded.
template <class S, typename T, typename Index, int LAYOUT, int CPL, bool NTS = false, bool SHV = false>
__global__ void __launch_bounds__(kWave)
tp_conv_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
               const Index* __restrict__ src, const Index* __restrict__ dst, const Index* __restrict__ row_ptr,
               int64_t n_src, int64_t n_edges, int64_t w_stride, int mul, int batch, int mean, T* __restrict__ out,
               const T* __restrict__ vec = nullptr, int sh_normalize = 0, ShConsts shk = {}) {
  const int64_t node = blockIdx.x;
  const int ub = blockIdx.y * (kWave * CPL) + threadIdx.x * CPL;
  const bool active = ub < mul;
  const int ubl = active ? ub : 0;  // idle lanes load channel 0 and store nothing

  int64_t e0, e1;
  edge_range(dst, n_edges, batch, node, e0, e1, row_ptr);
  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;

  T acc[CPL][S::NK];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int k = 0; k < S::NK; ++k) acc[c][k] = T(0);

  auto source = [&](int64_t e) -> int64_t { return batch ? e : static_cast<int64_t>(src[e]); };
  auto load = [&](int64_t e, int64_t s, T (&xv)[CPL][S::NX], T (&wv)[CPL][S::NP], T (&shv)[S::D2]) {
    const int64_t sc = (s >= 0 && s < n_src) ? s : 0;
    S::template load_xs<T, LAYOUT, CPL>(x + sc * dim1, mul, ubl, xv);
    const T* wrow = w + e * w_stride + ubl;
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
    if constexpr (SHV) {
      static_assert((sh_lmax_of(S::D2) + 1) * (sh_lmax_of(S::D2) + 1) == S::D2, "operand 2 is not a harmonics set");
      const T* vr = vec + e * 3;
      sh_eval<T, sh_lmax_of(S::D2)>(vr[0], vr[1], vr[2], sh_normalize != 0, shk, shv);
    } else {
      const T* shrow = sh + e * S::D2;
#pragma unroll
      for (int j = 0; j < S::D2; ++j) shv[j] = shrow[j];
    }
  };

  // next edge's operands (in flight while the current edge is computed)
  T xv[CPL][S::NX];
  T wv[CPL][S::NP];
  T shv[S::D2];
  int64_t s_next = 0, s_after = 0;
  if (e0 < e1) {
    s_next = source(e0);
    s_after = e0 + 1 < e1 ? source(e0 + 1) : 0;
    load(e0, s_next, xv, wv, shv);
  }
  for (int64_t e = e0; e < e1; ++e) {
    const int64_t s_cur = s_next;
    T xc[CPL][S::NX];
    T wc[CPL][S::NP];
    T shc[S::D2];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
      for (int i = 0; i < S::NX; ++i) xc[c][i] = xv[c][i];
#pragma unroll
      for (int p = 0; p < S::NP; ++p) wc[c][p] = wv[c][p];
    }
#pragma unroll
    for (int j = 0; j < S::D2; ++j) shc[j] = shv[j];
    if (e + 1 < e1) {
      s_next = s_after;
      load(e + 1, s_next, xv, wv, shv);
      s_after = e + 2 < e1 ? source(e + 2) : 0;
    }
    if (s_cur >= 0 && s_cur < n_src)  // out-of-range sources contribute nothing
      S::template edge<T, CPL>(xc, shc, wc, acc);
  }

  if (mean && e1 > e0) {  // reduce="mean": divide by the node's number of edges
    const T inv = T(1) / static_cast<T>(e1 - e0);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int k = 0; k < S::NK; ++k) acc[c][k] *= inv;
  }
  if (active)
    S::template store_s<T, LAYOUT, CPL, NTS>(out + node * (static_cast<int64_t>(mul) * S::NK), mul, ub, acc);
}

// Small multiplicities (mul <= GW <= 32) with a graph: one workgroup of
// kSplitThreads lanes per destination node, split into EG = kSplitThreads /
// GW groups of GW lanes (lane = channel).  Group g takes the node's edges
// e0 + g, e0 + g + EG, ..., two at a time with the operands of both loaded
// before either is computed, so a node's chain of dependent loads is 2 EG
// times shorter than with one wave walking all of it (the molecular batch
// has about 15 edges per node, and 64 lanes per wave would leave half
// idle).  The groups' sums are added in group order through LDS and written
// once: deterministic, no atomics.
//
// Measured on the molecular batch and dropped: a range search seeded with
// node * n_edges / n_nodes (its first probes are node-specific cache lines,
// where the whole-range search shares its first rounds across nodes),
// finding the range end edge by edge from dst instead of searching it, and
// a search by all four waves together (256 probes per round through LDS
// counts and barriers: two dependent loads instead of four, 9.8 -> 10.1 us).
constexpr int kSplitThreads = 256;

template <class S, typename T, typename Index, int LAYOUT, int GW, bool SHV = false>
__global__ void __launch_bounds__(kSplitThreads)
tp_conv_split_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                     const Index* __restrict__ src, const Index* __restrict__ dst, const Index* __restrict__ row_ptr,
                     int64_t n_src, int64_t n_edges, int64_t w_stride, int mul, int mean, T* __restrict__ out,
                     const T* __restrict__ vec = nullptr, int sh_normalize = 0, ShConsts shk = {}) {
  constexpr int EG = kSplitThreads / GW;
  __shared__ T red[EG][S::NK][GW];
  const int64_t node = blockIdx.x;
  const int g = threadIdx.x / GW;
  const int ul = threadIdx.x % GW;
  const bool active = ul < mul;
  const int ub = active ? ul : 0;
  int64_t e0, e1;
  edge_range(dst, n_edges, 0, node, e0, e1, row_ptr);  // every wave finds the same range
  const int64_t dim1 = static_cast<int64_t>(mul) * S::NX;

  T acc[1][S::NK];
#pragma unroll
  for (int k = 0; k < S::NK; ++k) acc[0][k] = T(0);
  auto load_edge = [&](int64_t e, T (&wv)[1][S::NP], T (&shv)[S::D2]) {
    const T* wrow = w + e * w_stride + ub;
#pragma unroll
    for (int p = 0; p < S::NP; ++p) wv[0][p] = __builtin_nontemporal_load(wrow + p * mul);
    if constexpr (SHV) {
      const T* vr = vec + e * 3;
      sh_eval<T, sh_lmax_of(S::D2)>(vr[0], vr[1], vr[2], sh_normalize != 0, shk, shv);
    } else {
      const T* shrow = sh + e * S::D2;
#pragma unroll
      for (int j = 0; j < S::D2; ++j) shv[j] = shrow[j];
    }
  };
  auto mask = [](bool keep, T (&xv)[1][S::NX], T (&wv)[1][S::NP], T (&shv)[S::D2]) {
#pragma unroll
    for (int i = 0; i < S::NX; ++i) xv[0][i] = keep ? xv[0][i] : T(0);
#pragma unroll
    for (int p = 0; p < S::NP; ++p) wv[0][p] = keep ? wv[0][p] : T(0);
#pragma unroll
    for (int j = 0; j < S::D2; ++j) shv[j] = keep ? shv[j] : T(0);
  };
  for (int64_t e = e0 + g; e < e1; e += 2 * EG) {
    const bool has_f = e + EG < e1;
    const int64_t f = has_f ? e + EG : e;  // clamped: every load below is unconditional
    const int64_t se = static_cast<int64_t>(src[e]), sfl = static_cast<int64_t>(src[f]);
    T we[1][S::NP], she[S::D2], wf[1][S::NP], shf[S::D2], xe[1][S::NX], xf[1][S::NX];
    load_edge(e, we, she);
    load_edge(f, wf, shf);
    S::template load_xs<T, LAYOUT, 1>(x + ((se >= 0 && se < n_src) ? se : 0) * dim1, mul, ub, xe);
    S::template load_xs<T, LAYOUT, 1>(x + ((sfl >= 0 && sfl < n_src) ? sfl : 0) * dim1, mul, ub, xf);
    // a missing second edge, or an out-of-range source, adds exact zeros: its
    // operands are zeroed by selects rather than skipped by a branch (behind
    // a branch the compiler issues the loads one after another)
    mask(se >= 0 && se < n_src, xe, we, she);
    mask(has_f && sfl >= 0 && sfl < n_src, xf, wf, shf);
    S::template edge<T, 1>(xe, she, we, acc);
    S::template edge<T, 1>(xf, shf, wf, acc);
  }
#pragma unroll
  for (int k = 0; k < S::NK; ++k) red[g][k][ul] = acc[0][k];
  __syncthreads();
  // the group sums, in group order, by the whole workgroup: thread (g, ul)
  // adds up components k = g, g + EG, ... of channel ul into red[0][k][ul]
  // (one thread per (k, ul), so the in-place write meets no other reader),
  // instead of the first GW lanes doing all NK * EG reads in turn
  for (int k = g; k < S::NK; k += EG) {
    T t = red[0][k][ul];
#pragma unroll
    for (int q = 1; q < EG; ++q) t += red[q][k][ul];
    red[0][k][ul] = t;
  }
  __syncthreads();
  if (threadIdx.x < GW && active) {
    const T scale = (mean && e1 > e0) ? T(1) / static_cast<T>(e1 - e0) : T(1);
    T v[1][S::NK];
#pragma unroll
    for (int k = 0; k < S::NK; ++k) v[0][k] = mean ? red[0][k][ul] * scale : red[0][k][ul];
    S::template store_s<T, LAYOUT, 1, false>(out + node * (static_cast<int64_t>(mul) * S::NK), mul, ul, v);
  }
}

template <class S, typename T, typename Index, int LAYOUT, int GW>
int tp_conv_split_launch(const TPArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.n_nodes));
  if (a.vec) {
    constexpr bool is_sh = (sh_lmax_of(S::D2) + 1) * (sh_lmax_of(S::D2) + 1) == S::D2 && sh_lmax_of(S::D2) <= kShMaxL;
    if constexpr (is_sh) {
      hipLaunchKernelGGL((tp_conv_split_kernel<S, T, Index, LAYOUT, GW, true>), grid, dim3(kSplitThreads), 0,
                         static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x), nullptr,
                         static_cast<const T*>(a.w), static_cast<const Index*>(a.src),
                         static_cast<const Index*>(a.dst), static_cast<const Index*>(a.row_ptr), a.n_src,
                         a.n_edges, a.w_stride, a.mul, a.mean,
                         static_cast<T*>(a.out), static_cast<const T*>(a.vec), a.sh_normalize, *a.sh_consts);
      return static_cast<int>(hipGetLastError());
    } else {
      return -2;  // operand 2 is not a harmonics set
    }
  }
  hipLaunchKernelGGL((tp_conv_split_kernel<S, T, Index, LAYOUT, GW>), grid, dim3(kSplitThreads), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x), static_cast<const T*>(a.sh),
                     static_cast<const T*>(a.w), static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                     static_cast<const Index*>(a.row_ptr),
                     a.n_src, a.n_edges, a.w_stride, a.mul, a.mean, static_cast<T*>(a.out));
  return static_cast<int>(hipGetLastError());
}

template <class S, typename T, typename Index, int LAYOUT, int CPL, bool NTS = false>
int tp_conv_launch(const TPArgs& a) {
  const int per_tile = kWave * CPL;
  dim3 grid(static_cast<unsigned>(a.n_nodes), static_cast<unsigned>((a.mul + per_tile - 1) / per_tile));
  if (a.vec) {
    constexpr bool is_sh = (sh_lmax_of(S::D2) + 1) * (sh_lmax_of(S::D2) + 1) == S::D2 && sh_lmax_of(S::D2) <= kShMaxL;
    if constexpr (is_sh) {
      hipLaunchKernelGGL((tp_conv_kernel<S, T, Index, LAYOUT, CPL, NTS, true>), grid, dim3(kWave), 0,
                         static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x), nullptr,
                         static_cast<const T*>(a.w), static_cast<const Index*>(a.src),
                         static_cast<const Index*>(a.dst), static_cast<const Index*>(a.row_ptr), a.n_src,
                         a.n_edges, a.w_stride, a.mul, a.batch, a.mean,
                         static_cast<T*>(a.out), static_cast<const T*>(a.vec), a.sh_normalize, *a.sh_consts);
      return static_cast<int>(hipGetLastError());
    } else {
      return -2;  // operand 2 is not a harmonics set
    }
  }
  hipLaunchKernelGGL((tp_conv_kernel<S, T, Index, LAYOUT, CPL, NTS>), grid, dim3(kWave), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x),
                     static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                     static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                     static_cast<const Index*>(a.row_ptr), a.n_src,
                     a.n_edges, a.w_stride, a.mul, a.batch, a.mean, static_cast<T*>(a.out));
  return static_cast<int>(hipGetLastError());
}

inline bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Two channels per lane when the multiplicity fills more than one wave with
// single channels and the pair accesses are aligned; one otherwise.
template <class S, typename T, typename Index, int LAYOUT>
int tp_conv_dispatch_cpl(const TPArgs& a) {
  // graphs with at most 32 channels: the destination-split kernel (its LDS
  // reduction buffer is kSplitThreads * NK values)
  if constexpr (kSplitThreads * S::NK * sizeof(T) <= 64 * 1024) {
    if (!a.batch && a.mul <= 32) {
      if (a.mul <= 16) return tp_conv_split_launch<S, T, Index, LAYOUT, 16>(a);
      return tp_conv_split_launch<S, T, Index, LAYOUT, 32>(a);
    }
  }
  const size_t pa = 2 * sizeof(T);
  if (a.mul > kWave && a.mul % 2 == 0 && aligned(a.x, pa) && aligned(a.w, pa) && aligned(a.out, pa))
    return tp_conv_launch<S, T, Index, LAYOUT, 2>(a);
  return tp_conv_launch<S, T, Index, LAYOUT, 1>(a);
}

template <class S, typename T>
int tp_conv_dispatch(const TPArgs& a) {
  if (a.idx == kI32) {
    if (a.layout == kMulIr) return tp_conv_dispatch_cpl<S, T, int32_t, kMulIr>(a);
    return tp_conv_dispatch_cpl<S, T, int32_t, kIrMul>(a);
  }
  if (a.layout == kMulIr) return tp_conv_dispatch_cpl<S, T, int64_t, kMulIr>(a);
  return tp_conv_dispatch_cpl<S, T, int64_t, kIrMul>(a);
}

}  // namespace kern
}  // namespace segpoly
