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
#include "tp_conv_spec.hpp"

namespace segpoly {
namespace kern {

constexpr int kGW = 64;

template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(kGW)
tp_conv_generic_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                       const Index* __restrict__ src, const Index* __restrict__ dst,
                       const GPath* __restrict__ paths, const GNz* __restrict__ nz, int np, int nk,
                       int64_t dim1, int64_t dim2, int64_t dimo, int64_t n_src, int64_t n_edges,
                       int64_t w_stride, int batch, int mean, T* __restrict__ out) {
  extern __shared__ unsigned char smem_raw[];
  T* acc = reinterpret_cast<T*>(smem_raw);
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x;
  const int u = blockIdx.y * kGW + lane;
  for (int k = 0; k < nk; ++k) acc[k * kGW + lane] = T(0);

  int64_t e0, e1;
  edge_range(dst, n_edges, batch, node, e0, e1);
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
                     static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst), g.paths, g.nz,
                     g.np, g.nk, g.dim1, g.dim2, g.dimo, a.n_src, a.n_edges, a.w_stride, a.batch, a.mean,
                     static_cast<T*>(a.out));
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

}  // namespace kern

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

}  // namespace segpoly
