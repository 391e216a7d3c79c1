// Table-driven kernels for descriptors that have no generated specialisation
// (any irreps within the envelope; non-uniform multiplicities allowed for
// the tensor product).  Same mathematics as the specialised kernels, with
// the coefficients read from a device table instead of literal constants
// and the per-channel accumulators in LDS (each lane owns one LDS column,
// so no barrier is needed).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../generic_tables.hpp"
#include "../launch.hpp"
#include "common.hpp"
#include "tp_conv_bwd.hpp"
#include "tp_conv_spec.hpp"

namespace segpoly {
namespace kern {

constexpr int kGW = 64;

template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(kGW)
tp_conv_generic_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                       const Index* __restrict__ src, const Index* __restrict__ dst,
                       const Index* __restrict__ row_ptr, const GPath* __restrict__ paths, const GNz* __restrict__ nz, int np, int nk,
                       int64_t dim1, int64_t dim2, int64_t dimo, int64_t n_src, int64_t n_edges,
                       int64_t w_stride, int batch, int mean, T* __restrict__ out) {
  extern __shared__ unsigned char smem_raw[];
  T* acc = reinterpret_cast<T*>(smem_raw);
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x;
  const int u = blockIdx.y * kGW + lane;
  for (int k = 0; k < nk; ++k) acc[k * kGW + lane] = T(0);

  int64_t e0, e1;
  edge_range(dst, n_edges, batch, node, e0, e1, row_ptr);
  for (int64_t e = e0; e < e1; ++e) {
    const int64_t s = batch ? e : static_cast<int64_t>(src[e]);
    if (s < 0 || s >= n_src) continue;
    const T* xrow = x + s * dim1;
    const T* shrow = sh + e * dim2;
    const T* wrow = w + e * w_stride;
    for (int p = 0; p < np; ++p) {
      const GPath P = paths[p];
      if (u >= P.mul) continue;
      const T wv = wrow[P.woff + u];
      const int d1 = 2 * P.l1 + 1;
      for (int n = P.nz_begin; n < P.nz_end; ++n) {
        const GNz z = nz[n];
        const T xi = (LAYOUT == kIrMul) ? xrow[P.off1 + static_cast<int64_t>(z.i) * P.mul + u]
                                        : xrow[P.off1 + static_cast<int64_t>(u) * d1 + z.i];
        T& a = acc[(P.kcomp + z.k) * kGW + lane];
        a = fmadd(static_cast<T>(z.c) * shrow[P.off2 + z.j], xi * wv, a);
      }
    }
  }
  T* orow = out + node * dimo;
  const T scale = (mean && e1 > e0) ? T(1) / static_cast<T>(e1 - e0) : T(1);
  for (int p = 0; p < np; ++p) {
    const GPath P = paths[p];
    if (u >= P.mul) continue;
    const int dl = 2 * P.lo + 1;
    for (int k = 0; k < dl; ++k) {
      const T v = scale * acc[(P.kcomp + k) * kGW + lane];
      if (LAYOUT == kIrMul)
        orow[P.offo + static_cast<int64_t>(k) * P.mul + u] = v;
      else
        orow[P.offo + static_cast<int64_t>(u) * dl + k] = v;
    }
  }
}

template <typename T, typename Index, int LAYOUT>
int tp_generic_launch(const TPArgs& a, const GenericTPInfo& g) {
  dim3 grid(static_cast<unsigned>(a.n_nodes), static_cast<unsigned>((g.max_mul + kGW - 1) / kGW));
  size_t lds = static_cast<size_t>(g.nk) * kGW * sizeof(T);
  hipLaunchKernelGGL((tp_conv_generic_kernel<T, Index, LAYOUT>), grid, dim3(kGW), lds,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x),
                     static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                     static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                     static_cast<const Index*>(a.row_ptr), g.paths, g.nz, g.np, g.nk, g.dim1, g.dim2, g.dimo,
                     a.n_src, a.n_edges, a.w_stride, a.batch, a.mean, static_cast<T*>(a.out));
  return static_cast<int>(hipGetLastError());
}

template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(kGW)
symcon_generic_kernel(const T* __restrict__ x, const Index* __restrict__ species, const T* __restrict__ w,
                      const GTerm* __restrict__ terms, const GBlock* __restrict__ in_blocks,
                      const GBlock* __restrict__ out_blocks, int n_terms, int n_in_blocks,
                      int n_out_blocks, int nv, int no, int mul, int64_t numel, int num_elements,
                      T* __restrict__ out) {
  extern __shared__ unsigned char smem_raw[];
  T* v = reinterpret_cast<T*>(smem_raw);  // [nv][64]
  T* o = v + nv * kGW;                    // [no][64]
  const int64_t atom = blockIdx.x;
  const int lane = threadIdx.x;
  const int u = blockIdx.y * kGW + lane;
  if (u >= mul) return;  // no barrier below: each lane owns its LDS columns
  const int64_t sp = static_cast<int64_t>(species[atom]);
  const bool valid = sp >= 0 && sp < num_elements;
  const T* xrow = x + atom * (static_cast<int64_t>(mul) * nv);
  T* orow = out + atom * (static_cast<int64_t>(mul) * no);
  for (int b = 0; b < n_in_blocks; ++b) {
    const GBlock B = in_blocks[b];
    const int dl = 2 * B.l + 1;
    for (int i = 0; i < dl; ++i)
      v[(B.comp + i) * kGW + lane] = (LAYOUT == kIrMul)
                                         ? xrow[static_cast<int64_t>(B.comp + i) * mul + u]
                                         : xrow[static_cast<int64_t>(B.comp) * mul + static_cast<int64_t>(u) * dl + i];
  }
  for (int k = 0; k < no; ++k) o[k * kGW + lane] = T(0);
  if (valid) {
    const T* wrow = w + sp * numel;
    for (int t = 0; t < n_terms; ++t) {
      const GTerm z = terms[t];
      T m = v[z.m0 * kGW + lane];
      if (z.m1 >= 0) m *= v[z.m1 * kGW + lane];
      if (z.m2 >= 0) m *= v[z.m2 * kGW + lane];
      T& a = o[z.og * kGW + lane];
      a = fmadd(static_cast<T>(z.c) * wrow[static_cast<int64_t>(z.seg) * mul + u], m, a);
    }
  }
  for (int b = 0; b < n_out_blocks; ++b) {
    const GBlock B = out_blocks[b];
    const int dl = 2 * B.l + 1;
    for (int i = 0; i < dl; ++i) {
      const T val = o[(B.comp + i) * kGW + lane];
      if (LAYOUT == kIrMul)
        orow[static_cast<int64_t>(B.comp + i) * mul + u] = val;
      else
        orow[static_cast<int64_t>(B.comp) * mul + static_cast<int64_t>(u) * dl + i] = val;
    }
  }
}

template <typename T, typename Index, int LAYOUT>
int symcon_generic_launch(const SymconArgs& a, const GenericSymconInfo& g) {
  dim3 grid(static_cast<unsigned>(a.n_atoms), static_cast<unsigned>((a.mul + kGW - 1) / kGW));
  size_t lds = static_cast<size_t>(g.nv + g.no) * kGW * sizeof(T);
  hipLaunchKernelGGL((symcon_generic_kernel<T, Index, LAYOUT>), grid, dim3(kGW), lds,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x),
                     static_cast<const Index*>(a.species), static_cast<const T*>(a.w), g.terms,
                     g.in_blocks, g.out_blocks, g.n_terms, g.n_in_blocks, g.n_out_blocks, g.nv, g.no,
                     a.mul, g.numel, a.num_elements, static_cast<T*>(a.out));
  return static_cast<int>(hipGetLastError());
}

// ------------------------------------------------------------- backward
//
// Vector-Jacobian products of the two table-driven kernels above, for g =
// dL/d(out) (the gradients of every operand that the cuequivariance-torch
// skill document's examples check, "CPU tensor product and backward"):
//   dw[e, p, u] = sum_k g[dst_e, p, k, u] sum_ij C_p[i,j,k] x[src_e, i, u] sh[e, j]
//   dsh[e, j]   = sum_{p, u} w[e, p, u] sum_ik C_p[i,j,k] x[src_e, i, u] g[dst_e, p, k, u]
//   dx[s, i, u] = sum_{e: src_e = s} sum_p w[e, p, u] sum_jk C_p[i,j,k] sh[e, j] g[dst_e, p, k, u]
// (the same sums as the generated backward, coefficients from the device
// table).  No workspace: the source-major kernel recomputes each edge's
// contribution from w, sh and g[dst] instead of reading a stored message.
// Deterministic: fixed edge order in every sum, lane sums by a fixed
// butterfly, no atomics.

template <int LAYOUT>
__device__ __forceinline__ int64_t gen_idx(int comp, int u, int l, int mul) {
  return LAYOUT == kIrMul ? static_cast<int64_t>(comp) * mul + u : static_cast<int64_t>(u) * (2 * l + 1) + comp;
}

template <typename T>
__device__ __forceinline__ T wave_total(T v) {
#pragma unroll
  for (int off = kGW / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Destination-major: one wave per destination node, looping over channel
// tiles; per edge the weight gradients (per channel) and the harmonic
// gradient (lane partials in LDS, then summed over the wave).  Edges whose
// destination is outside [0, n_nodes) get zero rows (node 0 takes those
// before its range, the last node those after it).
template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(kGW)
tp_generic_bwd_edge_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                           const Index* __restrict__ src, const Index* __restrict__ dst,
                           const Index* __restrict__ row_ptr, const T* __restrict__ g,
                           const GPath* __restrict__ paths, const GNz* __restrict__ nz, int np, int tiles,
                           int64_t dim1, int64_t dim2, int64_t dimo, int64_t numel, int64_t n_src,
                           int64_t n_edges, int64_t n_nodes, int64_t w_stride, int batch, int mean,
                           T* __restrict__ dw, T* __restrict__ dsh) {
  extern __shared__ unsigned char smem_raw[];
  T* hsh = reinterpret_cast<T*>(smem_raw);  // [dim2][kGW]
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x;
  int64_t e0, e1;
  edge_range(dst, n_edges, batch, node, e0, e1, row_ptr);
  auto zero_edge = [&](int64_t e) {
    for (int64_t c = lane; c < numel; c += kGW) dw[e * numel + c] = T(0);
    for (int64_t j = lane; j < dim2; j += kGW) dsh[e * dim2 + j] = T(0);
  };
  if (!batch) {
    if (node == 0)
      for (int64_t e = 0; e < e0; ++e) zero_edge(e);
    if (node == n_nodes - 1)
      for (int64_t e = e1; e < n_edges; ++e) zero_edge(e);
  }
  const T scale = (mean && e1 > e0) ? T(1) / static_cast<T>(e1 - e0) : T(1);
  const T* grow = g + node * dimo;
  for (int64_t e = e0; e < e1; ++e) {
    const int64_t s = batch ? e : static_cast<int64_t>(src[e]);
    const bool valid = s >= 0 && s < n_src;  // an out-of-range source contributes nothing
    const T* xrow = x + (valid ? s : 0) * dim1;
    const T* shrow = sh + e * dim2;
    const T* wrow = w + e * w_stride;
    for (int64_t j = 0; j < dim2; ++j) hsh[j * kGW + lane] = T(0);
    for (int t = 0; t < tiles; ++t) {
      const int u = t * kGW + lane;
      for (int p = 0; p < np; ++p) {
        const GPath P = paths[p];
        if (u >= P.mul) continue;
        const T wv = valid ? wrow[P.woff + u] : T(0);
        T dwacc = T(0);
        for (int n = P.nz_begin; n < P.nz_end; ++n) {
          const GNz z = nz[n];
          const T xi = valid ? xrow[P.off1 + gen_idx<LAYOUT>(z.i, u, P.l1, P.mul)] : T(0);
          const T gk = scale * grow[P.offo + gen_idx<LAYOUT>(z.k, u, P.lo, P.mul)];
          const T cx = static_cast<T>(z.c) * xi;
          dwacc = fmadd(cx * shrow[P.off2 + z.j], gk, dwacc);
          T& h = hsh[(P.off2 + z.j) * kGW + lane];
          h = fmadd(cx * wv, gk, h);
        }
        dw[e * numel + P.woff + u] = dwacc;
      }
    }
    for (int64_t j = 0; j < dim2; ++j) {
      const T tot = wave_total(hsh[j * kGW + lane]);
      if (lane == 0) dsh[e * dim2 + j] = tot;
    }
  }
}

// Source-major: one wave per (source node, channel tile) walks the source's
// edges in src_perm order (batch mode: edge s only) and sums their
// contributions to dx[s] in LDS columns (zero rows for a source without
// edges).  With reduce="mean" each edge's g row is divided by its
// destination's edge count.
template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(kGW)
tp_generic_bwd_src_kernel(const T* __restrict__ sh, const T* __restrict__ w, const Index* __restrict__ src,
                          const Index* __restrict__ dst, const Index* __restrict__ row_ptr,
                          const Index* __restrict__ src_row_ptr, const Index* __restrict__ perm,
                          const T* __restrict__ g,
                          const GPath* __restrict__ paths, const GNz* __restrict__ nz, int np,
                          const GIn* __restrict__ in, int n_in, int nx, int64_t dim1, int64_t dim2, int64_t dimo,
                          int64_t n_edges, int64_t n_nodes, int64_t w_stride, int batch, int mean,
                          T* __restrict__ dx) {
  extern __shared__ unsigned char smem_raw[];
  T* acc = reinterpret_cast<T*>(smem_raw);  // [nx][kGW]
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x;
  const int u = blockIdx.y * kGW + lane;
  for (int c = 0; c < nx; ++c) acc[c * kGW + lane] = T(0);
  int64_t i0, i1;
  if (batch) {
    i0 = s;
    i1 = s < n_edges ? s + 1 : s;
  } else if (src_row_ptr) {  // the caller's row pointers, clamped to [0, n_edges]
    const int64_t r0 = static_cast<int64_t>(src_row_ptr[s]);
    const int64_t r1 = static_cast<int64_t>(src_row_ptr[s + 1]);
    i0 = r0 < 0 ? 0 : (r0 > n_edges ? n_edges : r0);
    i1 = r1 < i0 ? i0 : (r1 > n_edges ? n_edges : r1);
  } else {
    i0 = lower_bound_perm(src, perm, n_edges, 0, n_edges, s);
    i1 = lower_bound_perm(src, perm, n_edges, i0, n_edges, s + 1);
  }
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t e = batch ? i : static_cast<int64_t>(perm[i]);
    if (e < 0 || e >= n_edges) continue;  // only an invalid perm gets here
    const int64_t d = batch ? e : static_cast<int64_t>(dst[e]);
    if (d < 0 || d >= n_nodes) continue;  // the edge reached no output row
    T scale = T(1);
    if (mean && !batch) {
      int64_t d0, d1;
      edge_range(dst, n_edges, 0, d, d0, d1, row_ptr);
      scale = T(1) / static_cast<T>(d1 - d0);
    }
    const T* grow = g + d * dimo;
    const T* shrow = sh + e * dim2;
    const T* wrow = w + e * w_stride;
    for (int p = 0; p < np; ++p) {
      const GPath P = paths[p];
      if (u >= P.mul) continue;
      const T wv = scale * wrow[P.woff + u];
      for (int n = P.nz_begin; n < P.nz_end; ++n) {
        const GNz z = nz[n];
        const T gk = grow[P.offo + gen_idx<LAYOUT>(z.k, u, P.lo, P.mul)];
        T& a = acc[(P.xcomp + z.i) * kGW + lane];
        a = fmadd(static_cast<T>(z.c) * shrow[P.off2 + z.j], wv * gk, a);
      }
    }
  }
  T* xrow = dx + s * dim1;
  for (int b = 0; b < n_in; ++b) {
    const GIn B = in[b];
    if (u >= B.mul) continue;
    for (int c = 0; c < 2 * B.l + 1; ++c) xrow[B.off + gen_idx<LAYOUT>(c, u, B.l, B.mul)] = acc[(B.comp + c) * kGW + lane];
  }
}

template <typename T, typename Index, int LAYOUT>
int tp_generic_bwd_launch(const TPBwdArgs& a, const GenericTPInfo& g) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  T* const dx = static_cast<T*>(a.dx);
  T* const dsh = static_cast<T*>(a.dsh);
  if (a.n_edges == 0) {  // nothing reaches the output: dx (and a shared dw) is zero
    fill_zero(dx, a.n_src * g.dim1, st);
    if (a.shared_w) fill_zero(static_cast<T*>(a.dw), g.numel, st);
    return static_cast<int>(hipGetLastError());
  }
  if (a.n_nodes == 0) {  // every edge has a destination outside the output
    fill_zero(dx, a.n_src * g.dim1, st);
    fill_zero(static_cast<T*>(a.dw), a.shared_w ? g.numel : a.n_edges * g.numel, st);
    fill_zero(dsh, a.n_edges * g.dim2, st);
    return static_cast<int>(hipGetLastError());
  }
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  T* const dwe = a.shared_w ? reinterpret_cast<T*>(ws + a.dw_ws_off) : static_cast<T*>(a.dw);
  const int tiles = (g.max_mul + kGW - 1) / kGW;
  const int64_t w_stride = a.shared_w ? 0 : g.numel;
  hipLaunchKernelGGL((tp_generic_bwd_edge_kernel<T, Index, LAYOUT>), dim3(static_cast<unsigned>(a.n_nodes)),
                     dim3(kGW), static_cast<size_t>(g.dim2 > 0 ? g.dim2 : 1) * kGW * sizeof(T), st,
                     static_cast<const T*>(a.x), static_cast<const T*>(a.sh), static_cast<const T*>(a.w),
                     static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                     static_cast<const Index*>(a.row_ptr), static_cast<const T*>(a.g),
                     g.paths, g.nz, g.np, tiles, g.dim1, g.dim2, g.dimo, g.numel, a.n_src, a.n_edges, a.n_nodes,
                     w_stride, a.batch, a.mean, dwe, dsh);
  int rc = static_cast<int>(hipGetLastError());
  if (rc) return rc;
  if (a.shared_w) {  // the per-edge rows summed in chunks, then the chunks in order
    const int64_t chunks = (a.n_edges + kTpDwChunk - 1) / kTpDwChunk;
    T* const dpart = reinterpret_cast<T*>(ws + a.dw_ws_off +
                                          round_up_256(a.n_edges * g.numel * static_cast<int64_t>(sizeof(T))));
    hipLaunchKernelGGL((dw_edge_sum_kernel<T>), dim3(static_cast<unsigned>((g.numel + 255) / 256),
                                                     static_cast<unsigned>(chunks)),
                       dim3(256), 0, st, dwe, a.n_edges, g.numel, dpart);
    const int64_t blocks = (g.numel + 255) / 256;
    hipLaunchKernelGGL((fold_partials_kernel<T>), dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                       dim3(256), 0, st, dpart, static_cast<int>(chunks), g.numel, static_cast<T*>(a.dw));
    rc = static_cast<int>(hipGetLastError());
    if (rc) return rc;
  }
  if (a.n_src > 0) {
    hipLaunchKernelGGL((tp_generic_bwd_src_kernel<T, Index, LAYOUT>),
                       dim3(static_cast<unsigned>(a.n_src), static_cast<unsigned>(tiles)), dim3(kGW),
                       static_cast<size_t>(g.nx > 0 ? g.nx : 1) * kGW * sizeof(T), st, static_cast<const T*>(a.sh),
                       static_cast<const T*>(a.w), static_cast<const Index*>(a.src),
                       static_cast<const Index*>(a.dst), static_cast<const Index*>(a.row_ptr),
                       static_cast<const Index*>(a.src_row_ptr), static_cast<const Index*>(a.perm),
                       static_cast<const T*>(a.g), g.paths, g.nz, g.np, g.in, g.n_in, g.nx, g.dim1, g.dim2, g.dimo,
                       a.n_edges, a.n_nodes, w_stride, a.batch, a.mean, dx);
  }
  return static_cast<int>(hipGetLastError());
}

// Symmetric contraction, dx: per (atom, channel), the derivative of every
// sorted monomial by the product rule (one term per slot: v_a v_b v_c gives
// v_b v_c to a, v_a v_c to b, v_a v_b to c, so repeated components count
// twice or three times), weighted by c w[species, seg, u] g[og].  Lane-owned
// LDS columns, as in the forward.
template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(kGW)
symcon_generic_bwd_dx_kernel(const T* __restrict__ x, const Index* __restrict__ species, const T* __restrict__ w,
                             const T* __restrict__ g, const GTerm* __restrict__ terms,
                             const GBlock* __restrict__ in_blocks, const GBlock* __restrict__ out_blocks,
                             int n_terms, int n_in_blocks, int n_out_blocks, int nv, int no, int mul, int64_t numel,
                             int num_elements, T* __restrict__ dx) {
  extern __shared__ unsigned char smem_raw[];
  T* v = reinterpret_cast<T*>(smem_raw);  // [nv][64]
  T* go = v + nv * kGW;                   // [no][64]
  T* dv = go + no * kGW;                  // [nv][64]
  const int64_t atom = blockIdx.x;
  const int lane = threadIdx.x;
  const int u = blockIdx.y * kGW + lane;
  if (u >= mul) return;  // no barrier below: each lane owns its LDS columns
  const int64_t sp = static_cast<int64_t>(species[atom]);
  const bool valid = sp >= 0 && sp < num_elements;
  const int64_t dim_in = static_cast<int64_t>(mul) * nv, dim_out = static_cast<int64_t>(mul) * no;
  const T* xrow = x + atom * dim_in;
  const T* grow = g + atom * dim_out;
  for (int b = 0; b < n_in_blocks; ++b) {
    const GBlock B = in_blocks[b];
    for (int i = 0; i < 2 * B.l + 1; ++i) {
      v[(B.comp + i) * kGW + lane] = xrow[static_cast<int64_t>(B.comp) * mul + gen_idx<LAYOUT>(i, u, B.l, mul)];
      dv[(B.comp + i) * kGW + lane] = T(0);
    }
  }
  for (int b = 0; b < n_out_blocks; ++b) {
    const GBlock B = out_blocks[b];
    for (int i = 0; i < 2 * B.l + 1; ++i)
      go[(B.comp + i) * kGW + lane] = grow[static_cast<int64_t>(B.comp) * mul + gen_idx<LAYOUT>(i, u, B.l, mul)];
  }
  if (valid) {
    const T* wrow = w + sp * numel;
    for (int t = 0; t < n_terms; ++t) {
      const GTerm z = terms[t];
      const T f = static_cast<T>(z.c) * wrow[static_cast<int64_t>(z.seg) * mul + u] * go[z.og * kGW + lane];
      const T a = v[z.m0 * kGW + lane];
      const T b = z.m1 >= 0 ? v[z.m1 * kGW + lane] : T(1);
      const T c = z.m2 >= 0 ? v[z.m2 * kGW + lane] : T(1);
      dv[z.m0 * kGW + lane] += f * (b * c);
      if (z.m1 >= 0) dv[z.m1 * kGW + lane] += f * (a * c);
      if (z.m2 >= 0) dv[z.m2 * kGW + lane] += f * (a * b);
    }
  }
  T* drow = dx + atom * dim_in;
  for (int b = 0; b < n_in_blocks; ++b) {
    const GBlock B = in_blocks[b];
    for (int i = 0; i < 2 * B.l + 1; ++i)
      drow[static_cast<int64_t>(B.comp) * mul + gen_idx<LAYOUT>(i, u, B.l, mul)] = dv[(B.comp + i) * kGW + lane];
  }
}

// Symmetric contraction, dw: one workgroup per (channel tile, element); its
// waves find the element's atoms in species_perm order (a wave-cooperative
// search over species[perm[.]]; entries of perm outside [0, n_atoms) count
// as past every element), wave k takes the atoms k, k + waves, ...,
// accumulates sum_M g poly per weight segment in its LDS columns, and wave
// 0 adds the waves' sums in wave order (zero for an element without atoms).
template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(kGW * 8)
symcon_generic_bwd_dw_kernel(const T* __restrict__ x, const Index* __restrict__ species, const Index* __restrict__ perm,
                             const T* __restrict__ g, const GTerm* __restrict__ terms,
                             const GBlock* __restrict__ in_blocks, const GBlock* __restrict__ out_blocks,
                             int n_terms, int n_in_blocks, int n_out_blocks, int nv, int no, int nseg, int mul,
                             int64_t n_atoms, T* __restrict__ dw) {
  extern __shared__ unsigned char smem_raw[];
  const int lane = threadIdx.x % kGW;
  const int wave = threadIdx.x / kGW;
  const int waves = blockDim.x / kGW;
  const int per_wave = (nv + no + nseg) * kGW;
  T* v = reinterpret_cast<T*>(smem_raw) + wave * per_wave;  // [nv][64]
  T* go = v + nv * kGW;                                      // [no][64]
  T* acc = go + no * kGW;                                    // [nseg][64]
  const int64_t e = blockIdx.y;
  const int u = blockIdx.x * kGW + lane;
  const bool active = u < mul;
  const int ul = active ? u : 0;
  auto elem = [&](int64_t i) -> int64_t {
    const int64_t a = static_cast<int64_t>(perm[i]);
    return (a >= 0 && a < n_atoms) ? static_cast<int64_t>(species[a]) : INT64_MAX;
  };
  auto first_at_least = [&](int64_t key) -> int64_t {  // first sorted position with element >= key
    int64_t lo = 0, hi = n_atoms;
    while (hi - lo > kGW) {
      const int64_t step = (hi - lo + kGW - 1) / kGW;
      const int64_t idx = lo + lane * step;
      const int c = __popcll(__ballot(idx < hi && elem(idx) < key));
      const int64_t nlo = c == 0 ? lo : lo + (c - 1) * step + 1;
      const int64_t nhi = lo + c * step < hi ? lo + c * step : hi;
      lo = nlo;
      hi = nhi;
    }
    return lo + __popcll(__ballot(lo + lane < hi && elem(lo + lane) < key));
  };
  const int64_t i0 = first_at_least(e), i1 = first_at_least(e + 1);
  for (int s = 0; s < nseg; ++s) acc[s * kGW + lane] = T(0);
  const int64_t dim_in = static_cast<int64_t>(mul) * nv, dim_out = static_cast<int64_t>(mul) * no;
  for (int64_t i = i0 + wave; i < i1; i += waves) {
    const int64_t a = static_cast<int64_t>(perm[i]);
    const T* xrow = x + a * dim_in;
    const T* grow = g + a * dim_out;
    for (int b = 0; b < n_in_blocks; ++b) {
      const GBlock B = in_blocks[b];
      for (int q = 0; q < 2 * B.l + 1; ++q)
        v[(B.comp + q) * kGW + lane] = xrow[static_cast<int64_t>(B.comp) * mul + gen_idx<LAYOUT>(q, ul, B.l, mul)];
    }
    for (int b = 0; b < n_out_blocks; ++b) {
      const GBlock B = out_blocks[b];
      for (int q = 0; q < 2 * B.l + 1; ++q)
        go[(B.comp + q) * kGW + lane] = grow[static_cast<int64_t>(B.comp) * mul + gen_idx<LAYOUT>(q, ul, B.l, mul)];
    }
    for (int t = 0; t < n_terms; ++t) {
      const GTerm z = terms[t];
      T m = v[z.m0 * kGW + lane];
      if (z.m1 >= 0) m *= v[z.m1 * kGW + lane];
      if (z.m2 >= 0) m *= v[z.m2 * kGW + lane];
      T& r = acc[z.seg * kGW + lane];
      r = fmadd(static_cast<T>(z.c) * go[z.og * kGW + lane], m, r);
    }
  }
  __syncthreads();
  if (wave == 0 && active) {
    const int64_t numel = static_cast<int64_t>(mul) * nseg;
    const T* base = reinterpret_cast<const T*>(smem_raw);
    for (int s = 0; s < nseg; ++s) {
      T tot = T(0);
      for (int k = 0; k < waves; ++k) tot += base[k * per_wave + (nv + no + s) * kGW + lane];
      dw[e * numel + static_cast<int64_t>(s) * mul + u] = tot;
    }
  }
}

constexpr size_t kGenericBwdLds = 64 * 1024;

template <typename T, typename Index, int LAYOUT>
int symcon_generic_bwd_launch(const SymconBwdArgs& a, const GenericSymconInfo& g) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int tiles = (a.mul + kGW - 1) / kGW;
  const int nseg = a.mul > 0 ? static_cast<int>(g.numel / a.mul) : 0;
  if (a.n_atoms > 0) {
    hipLaunchKernelGGL((symcon_generic_bwd_dx_kernel<T, Index, LAYOUT>),
                       dim3(static_cast<unsigned>(a.n_atoms), static_cast<unsigned>(tiles)), dim3(kGW),
                       static_cast<size_t>(2 * g.nv + g.no) * kGW * sizeof(T), st, static_cast<const T*>(a.x),
                       static_cast<const Index*>(a.species), static_cast<const T*>(a.w), static_cast<const T*>(a.g),
                       g.terms, g.in_blocks, g.out_blocks, g.n_terms, g.n_in_blocks, g.n_out_blocks, g.nv, g.no, a.mul,
                       g.numel, a.num_elements, static_cast<T*>(a.dx));
    const int rc = static_cast<int>(hipGetLastError());
    if (rc) return rc;
  }
  if (g.numel == 0) return 0;
  const size_t per_wave = static_cast<size_t>(g.nv + g.no + nseg) * kGW * sizeof(T);
  int waves = static_cast<int>(kGenericBwdLds / per_wave);
  waves = waves > 8 ? 8 : (waves < 1 ? 1 : waves);
  hipLaunchKernelGGL((symcon_generic_bwd_dw_kernel<T, Index, LAYOUT>),
                     dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(a.num_elements)), dim3(kGW * waves),
                     per_wave * waves, st, static_cast<const T*>(a.x), static_cast<const Index*>(a.species),
                     static_cast<const Index*>(a.perm), static_cast<const T*>(a.g), g.terms, g.in_blocks,
                     g.out_blocks, g.n_terms, g.n_in_blocks, g.n_out_blocks, g.nv, g.no, nseg, a.mul, a.n_atoms,
                     static_cast<T*>(a.dw));
  return static_cast<int>(hipGetLastError());
}

}  // namespace kern

size_t tp_generic_bwd_lds(int nx, int64_t dim2, int dtype) {
  const size_t esz = dtype == kF32 ? 4 : 8;
  const size_t a = static_cast<size_t>(nx) * kern::kGW * esz, b = static_cast<size_t>(dim2) * kern::kGW * esz;
  return a > b ? a : b;
}

size_t symcon_generic_bwd_lds(int nv, int no, int nseg, int dtype) {
  const size_t esz = dtype == kF32 ? 4 : 8;
  const size_t a = static_cast<size_t>(2 * nv + no) * kern::kGW * esz;
  const size_t b = static_cast<size_t>(nv + no + nseg) * kern::kGW * esz;  // one wave of the dw kernel
  return a > b ? a : b;
}

int launch_tp_generic_bwd(const TPBwdArgs& a, const GenericTPInfo& g) {
  using namespace kern;
  if (a.dtype == kF32) {
    if (a.idx == kI32)
      return a.layout == kMulIr ? tp_generic_bwd_launch<float, int32_t, kMulIr>(a, g)
                                : tp_generic_bwd_launch<float, int32_t, kIrMul>(a, g);
    return a.layout == kMulIr ? tp_generic_bwd_launch<float, int64_t, kMulIr>(a, g)
                              : tp_generic_bwd_launch<float, int64_t, kIrMul>(a, g);
  }
  if (a.idx == kI32)
    return a.layout == kMulIr ? tp_generic_bwd_launch<double, int32_t, kMulIr>(a, g)
                              : tp_generic_bwd_launch<double, int32_t, kIrMul>(a, g);
  return a.layout == kMulIr ? tp_generic_bwd_launch<double, int64_t, kMulIr>(a, g)
                            : tp_generic_bwd_launch<double, int64_t, kIrMul>(a, g);
}

int launch_symcon_generic_bwd(const SymconBwdArgs& a, const GenericSymconInfo& g) {
  using namespace kern;
  if (a.dtype == kF32) {
    if (a.idx == kI32)
      return a.layout == kMulIr ? symcon_generic_bwd_launch<float, int32_t, kMulIr>(a, g)
                                : symcon_generic_bwd_launch<float, int32_t, kIrMul>(a, g);
    return a.layout == kMulIr ? symcon_generic_bwd_launch<float, int64_t, kMulIr>(a, g)
                              : symcon_generic_bwd_launch<float, int64_t, kIrMul>(a, g);
  }
  if (a.idx == kI32)
    return a.layout == kMulIr ? symcon_generic_bwd_launch<double, int32_t, kMulIr>(a, g)
                              : symcon_generic_bwd_launch<double, int32_t, kIrMul>(a, g);
  return a.layout == kMulIr ? symcon_generic_bwd_launch<double, int64_t, kMulIr>(a, g)
                            : symcon_generic_bwd_launch<double, int64_t, kIrMul>(a, g);
}

int launch_tp_generic(const TPArgs& a, const GenericTPInfo& g) {
  using namespace kern;
  if (a.dtype == kF32) {
    if (a.idx == kI32)
      return a.layout == kMulIr ? tp_generic_launch<float, int32_t, kMulIr>(a, g)
                                : tp_generic_launch<float, int32_t, kIrMul>(a, g);
    return a.layout == kMulIr ? tp_generic_launch<float, int64_t, kMulIr>(a, g)
                              : tp_generic_launch<float, int64_t, kIrMul>(a, g);
  }
  if (a.idx == kI32)
    return a.layout == kMulIr ? tp_generic_launch<double, int32_t, kMulIr>(a, g)
                              : tp_generic_launch<double, int32_t, kIrMul>(a, g);
  return a.layout == kMulIr ? tp_generic_launch<double, int64_t, kMulIr>(a, g)
                            : tp_generic_launch<double, int64_t, kIrMul>(a, g);
}

int launch_symcon_generic(const SymconArgs& a, const GenericSymconInfo& g) {
  using namespace kern;
  if (a.dtype == kF32) {
    if (a.idx == kI32)
      return a.layout == kMulIr ? symcon_generic_launch<float, int32_t, kMulIr>(a, g)
                                : symcon_generic_launch<float, int32_t, kIrMul>(a, g);
    return a.layout == kMulIr ? symcon_generic_launch<float, int64_t, kMulIr>(a, g)
                              : symcon_generic_launch<float, int64_t, kIrMul>(a, g);
  }
  if (a.idx == kI32)
    return a.layout == kMulIr ? symcon_generic_launch<double, int32_t, kMulIr>(a, g)
                              : symcon_generic_launch<double, int32_t, kIrMul>(a, g);
  return a.layout == kMulIr ? symcon_generic_launch<double, int64_t, kMulIr>(a, g)
                            : symcon_generic_launch<double, int64_t, kIrMul>(a, g);
}

namespace kern {

// rp[n] = first i with key(i) >= n, for n = 0 .. n_nodes, where key(i) =
// keys[i] (destinations sorted ascending), or keys[perm[i]] (sources in the
// order of their stable argsort; a perm entry outside [0, n_edges) counts
// as larger than every key): one thread per entry, a binary search each.
template <typename Index>
__global__ void __launch_bounds__(256)
rowptr_build_kernel(const Index* __restrict__ keys, const Index* __restrict__ perm, int64_t n_edges,
                    int64_t n_nodes, Index* __restrict__ rp) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (n > n_nodes) return;
  auto below = [&](int64_t i) -> bool {
    int64_t e = i;
    if (perm) {
      e = static_cast<int64_t>(perm[i]);
      if (e < 0 || e >= n_edges) return false;
    }
    return static_cast<int64_t>(keys[e]) < n;
  };
  int64_t lo = 0, hi = n_edges;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (below(mid))
      lo = mid + 1;
    else
      hi = mid;
  }
  rp[n] = static_cast<Index>(lo);
}

}  // namespace kern

int launch_rowptr_build(const void* keys, const void* perm, int idx, int64_t n_edges, int64_t n_nodes, void* rp,
                        void* stream) {
  const unsigned blocks = static_cast<unsigned>((n_nodes + 1 + 255) / 256);
  if (idx == kI64)
    hipLaunchKernelGGL((kern::rowptr_build_kernel<int64_t>), dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const int64_t*>(keys),
                       static_cast<const int64_t*>(perm), n_edges, n_nodes, static_cast<int64_t*>(rp));
  else
    hipLaunchKernelGGL((kern::rowptr_build_kernel<int32_t>), dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const int32_t*>(keys),
                       static_cast<const int32_t*>(perm), n_edges, n_nodes, static_cast<int32_t*>(rp));
  return static_cast<int>(hipGetLastError());
}

}  // namespace segpoly
