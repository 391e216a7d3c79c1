// Backward (vector-Jacobian product) of the symmetric contraction,
// specialised kernels (gfx950).
//
// The forward out[a, M, u] = sum_s w[species_a, s, u] sum over the sorted
// monomials of s of c * prod v[a, m_i, u] (e3nn-course Lesson 12a, section
// 21.4.1) is linear in the weights and a polynomial of degree <= 3 in x.
// Its gradients for g = dL/d(out) (the pages check the gradients of every
// module input: cuequivariance-torch skill document, "CPU tensor product and
// backward"):
//   dx[a, m, u] = sum_s w[species_a, s, u] sum_M g[a, M, u] d(poly_s,M)/dv_m
//                 (the product rule; per atom, no reduction);
//   dw[e, s, u] = sum over the atoms a of element e of sum_M g[a, M, u] poly_s,M(v_a)
//                 (a reduction over the atoms of each element).
//
// Deterministic, no atomics, over the atoms in element order (species_perm,
// a stable argsort of species, supplied by the caller like the sorted
// destinations of the convolution):
//  1. table kernel (one workgroup): the segments of the sorted order,
//     elements below 0, each element 0..E-1, elements >= E, and their split
//     into chunks of kSymconBwdChunk atoms with the chunk prefix sums;
//  2. chunk kernel: one wave per (chunk, channel tile), lane = channel.  The
//     chunk's element is uniform, so its weight row is loaded once into
//     registers; per atom the wave gathers v and g (row perm[i], the next
//     atom's rows in flight while the current one is computed), writes dx
//     and accumulates dw in registers; at the end it writes the chunk's
//     partial dw row.  Chunks of out-of-range elements write zero dx.
//     Measured on 50k atoms (10 elements, 128 channels): chunks of 8 atoms
//     beat 16 and 32 (more waves), and the prefetch gains 8 %.  It runs as
//     two launches, WHICH = 1 (dw partials) and WHICH = 2 (dx), each of
//     which holds fewer values than the fused pass (two or three waves per
//     SIMD instead of one: 0.61 -> 0.51 ms, the rows read twice);
//  3. fold kernel: dw[e] = sum of its chunks' partial rows in a fixed order
//     (zero for an element without atoms).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "bufload.hpp"
#include "common.hpp"
#include "tp_conv_spec.hpp"

namespace segpoly {
namespace kern {

// Table layout (int64): bounds[0..E+2] (segment g = [bounds[g], bounds[g+1])
// of the sorted order; g = 0: elements < 0, g = 1 + e: element e, g = E + 1:
// elements >= E), then cstart[0..E+2] (first chunk of each segment; the last
// entry is the number of chunks).
// One workgroup of kTableThreads; each wave finds some of the boundaries
// with the wave-cooperative 64-ary search over the permuted elements.
constexpr int kTableThreads = 1024;

template <typename Index>
__global__ void __launch_bounds__(kTableThreads)
symcon_table_kernel(const Index* __restrict__ species, const Index* __restrict__ perm, int64_t n, int ne,
                    int chunk, int64_t* __restrict__ table) {
  int64_t* bounds = table;
  int64_t* cstart = table + ne + 3;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  // element at sorted position i; entries of perm outside [0, n) compare as
  // +infinity
  auto elem = [&](int64_t i) -> int64_t {
    const int64_t a = static_cast<int64_t>(perm[i]);
    return (a >= 0 && a < n) ? static_cast<int64_t>(species[a]) : INT64_MAX;
  };
  // bounds[1 + t] = first sorted position whose element is >= t (t = 0..E)
  for (int t = wave; t <= ne; t += kTableThreads / kWave) {
    int64_t lo = 0, hi = n;
    while (hi - lo > kWave) {
      const int64_t step = (hi - lo + kWave - 1) / kWave;
      const int64_t idx = lo + lane * step;
      const int c = __popcll(__ballot(idx < hi && elem(idx) < t));
      const int64_t nlo = c == 0 ? lo : lo + (c - 1) * step + 1;
      const int64_t nhi = lo + c * step < hi ? lo + c * step : hi;
      lo = nlo;
      hi = nhi;
    }
    const int64_t idx = lo + lane;
    const int64_t r = lo + __popcll(__ballot(idx < hi && elem(idx) < t));
    if (lane == 0) bounds[1 + t] = r;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    bounds[0] = 0;
    bounds[ne + 2] = n;
    int64_t c = 0;
    for (int g = 0; g <= ne + 1; ++g) {
      cstart[g] = c;
      const int64_t len = bounds[g + 1] - bounds[g];
      c += len > 0 ? (len + chunk - 1) / chunk : 0;
    }
    cstart[ne + 2] = c;
  }
}

template <class S, typename T, typename Index, int LAYOUT, int WHICH>
__global__ void __launch_bounds__(kWave)
symcon_bwd_kernel(const T* __restrict__ x, const Index* __restrict__ perm, const T* __restrict__ w,
                  const T* __restrict__ g, int64_t n_atoms, int ne, int mul, const int64_t* __restrict__ table,
                  T* __restrict__ dx, T* __restrict__ part) {
  const int64_t* bounds = table;
  const int64_t* cstart = table + ne + 3;
  const int64_t t = blockIdx.x;
  if (t >= cstart[ne + 2]) return;  // grid sized for the most chunks possible
  const int lane = threadIdx.x % kWave;
  const int u = blockIdx.y * kWave + lane;
  const bool active = u < mul;
  const int ul = active ? u : 0;
  // segment of chunk t: the last g with cstart[g] <= t
  const int64_t seg = lower_bound_wave(cstart, 0, ne + 3, t + 1) - 1;
  const int64_t i0 = bounds[seg] + (t - cstart[seg]) * kSymconBwdChunk;
  const int64_t i1 = i0 + kSymconBwdChunk < bounds[seg + 1] ? i0 + kSymconBwdChunk : bounds[seg + 1];
  const bool valid = seg >= 1 && seg <= ne;  // an element in range
  const int64_t dim_in = static_cast<int64_t>(mul) * S::NV;
  const int64_t dim_out = static_cast<int64_t>(mul) * S::NO;
  const int64_t numel = static_cast<int64_t>(mul) * S::NS;

  T wv[S::NS];
  T dw[S::NS];
  const T* wrow = w + (valid ? seg - 1 : 0) * numel;
#pragma unroll
  for (int s = 0; s < S::NS; ++s) {
    wv[s] = valid ? wrow[s * mul + ul] : T(0);
    dw[s] = T(0);
  }
  // the next atom's rows are loaded while the current one is computed
  auto atom = [&](int64_t i) -> int64_t { return static_cast<int64_t>(perm[i]); };
  auto ok = [&](int64_t a) { return a >= 0 && a < n_atoms; };  // false only for an invalid perm
  T vn[S::NV], gn[S::NO];
  // ir_mul rows through buffer resources (lane offset in a register,
  // component offsets as scalar operands: no per-element address
  // arithmetic); mul_ir rows hold a channel's components of a block
  // contiguously, so plain pointers need one address per block and the
  // block's elements load as one vector
  auto load = [&](int64_t a) {
    const int64_t ac = ok(a) ? a : 0;
    if constexpr (LAYOUT == kIrMul) {
      S::template load_v_b<T, LAYOUT>(buf_rsrc(x + ac * dim_in, dim_in * static_cast<int64_t>(sizeof(T))), mul, ul,
                                      vn);
      S::template load_o_b<T, LAYOUT>(buf_rsrc(g + ac * dim_out, dim_out * static_cast<int64_t>(sizeof(T))), mul,
                                      ul, gn);
    } else {
      S::template load_v<T, LAYOUT>(x + ac * dim_in, mul, ul, vn);
      S::template load_o<T, LAYOUT>(g + ac * dim_out, mul, ul, gn);
    }
  };
  int64_t a_next = i0 < i1 ? atom(i0) : 0;
  if (valid && i0 < i1) load(a_next);
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t a = a_next;
    T dv[S::NV];
    if (valid) {
      T v[S::NV], go[S::NO];
#pragma unroll
      for (int m = 0; m < S::NV; ++m) v[m] = vn[m];
#pragma unroll
      for (int m = 0; m < S::NO; ++m) go[m] = gn[m];
      if (i + 1 < i1) {
        a_next = atom(i + 1);
        load(a_next);
      }
      if (ok(a)) {
        if constexpr ((WHICH & 1) != 0) S::template bwd_w<T>(v, go, dw);
        if constexpr ((WHICH & 2) != 0) S::template bwd_x<T>(v, go, wv, dv);
      }
    } else {
      if (i + 1 < i1) a_next = atom(i + 1);
#pragma unroll
      for (int m = 0; m < S::NV; ++m) dv[m] = T(0);
    }
    if constexpr ((WHICH & 2) != 0)
      if (active && ok(a)) {
        if constexpr (LAYOUT == kIrMul)
          S::template store_v_b<T, LAYOUT>(buf_rsrc(dx + a * dim_in, dim_in * static_cast<int64_t>(sizeof(T))), mul,
                                           u, dv);
        else
          S::template store_v<T, LAYOUT>(dx + a * dim_in, mul, u, dv);
      }
  }
  if ((WHICH & 1) != 0 && valid && active) {
    T* prow = part + t * numel;
#pragma unroll
    for (int s = 0; s < S::NS; ++s) prow[s * mul + u] = dw[s];
  }
}

// dw[e, col] = sum over the chunks of element e of part[chunk, col].  One
// workgroup per (64 columns, element): wave k sums the chunks k, k + 16, ...
// in order, then the sixteen sums are added in wave order (fixed order).
constexpr int kFoldWaves = 16;

template <typename T>
__global__ void __launch_bounds__(kFoldWaves * kWave)
symcon_fold_kernel(const T* __restrict__ part, const int64_t* __restrict__ table, int ne, int64_t numel,
                   T* __restrict__ dw) {
  __shared__ T sum[kFoldWaves][kWave];
  const int64_t* cstart = table + ne + 3;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t e = blockIdx.y;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const bool in = col < numel;
  const int64_t c0 = cstart[1 + e], c1 = cstart[2 + e];
  T acc = T(0);
  if (in) {
#pragma unroll 4
    for (int64_t c = c0 + wave; c < c1; c += kFoldWaves) acc += part[c * numel + col];
  }
  sum[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && in) {
    T v = sum[0][lane];
#pragma unroll
    for (int k = 1; k < kFoldWaves; ++k) v += sum[k][lane];
    dw[e * numel + col] = v;
  }
}

template <class S, typename T, typename Index, int LAYOUT>
int symcon_bwd_launch(const SymconBwdArgs& a) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int ne = a.num_elements;
  const int64_t numel = static_cast<int64_t>(a.mul) * S::NS;
  int64_t* table = static_cast<int64_t*>(a.workspace);
  T* part = reinterpret_cast<T*>(static_cast<unsigned char*>(a.workspace) + symcon_bwd_table_bytes(ne));
  hipLaunchKernelGGL((symcon_table_kernel<Index>), dim3(1), dim3(kTableThreads), 0, st,
                     static_cast<const Index*>(a.species),
                     static_cast<const Index*>(a.perm), a.n_atoms, ne, kSymconBwdChunk, table);
  int rc = static_cast<int>(hipGetLastError());
  if (rc) return rc;
  const int64_t chunks = symcon_bwd_max_chunks(a.n_atoms, ne);
  const unsigned tiles = static_cast<unsigned>((a.mul + kWave - 1) / kWave);
  if (a.n_atoms > 0) {
    hipLaunchKernelGGL((symcon_bwd_kernel<S, T, Index, LAYOUT, 1>), dim3(static_cast<unsigned>(chunks), tiles),
                       dim3(kWave), 0, st, static_cast<const T*>(a.x), static_cast<const Index*>(a.perm),
                       static_cast<const T*>(a.w), static_cast<const T*>(a.g), a.n_atoms, ne, a.mul, table,
                       static_cast<T*>(a.dx), part);
    rc = static_cast<int>(hipGetLastError());
    if (rc) return rc;
    hipLaunchKernelGGL((symcon_bwd_kernel<S, T, Index, LAYOUT, 2>), dim3(static_cast<unsigned>(chunks), tiles),
                       dim3(kWave), 0, st, static_cast<const T*>(a.x), static_cast<const Index*>(a.perm),
                       static_cast<const T*>(a.w), static_cast<const T*>(a.g), a.n_atoms, ne, a.mul, table,
                       static_cast<T*>(a.dx), part);
    rc = static_cast<int>(hipGetLastError());
    if (rc) return rc;
  }
  hipLaunchKernelGGL((symcon_fold_kernel<T>),
                     dim3(static_cast<unsigned>((numel + kWave - 1) / kWave), static_cast<unsigned>(ne)),
                     dim3(kFoldWaves * kWave), 0, st, part, table, ne, numel, static_cast<T*>(a.dw));
  return static_cast<int>(hipGetLastError());
}

template <class S, typename T>
int symcon_bwd_dispatch(const SymconBwdArgs& a) {
  if (a.idx == kI32) {
    if (a.layout == kMulIr) return symcon_bwd_launch<S, T, int32_t, kMulIr>(a);
    return symcon_bwd_launch<S, T, int32_t, kIrMul>(a);
  }
  if (a.layout == kMulIr) return symcon_bwd_launch<S, T, int64_t, kMulIr>(a);
  return symcon_bwd_launch<S, T, int64_t, kIrMul>(a);
}

}  // namespace kern
}  // namespace segpoly
