// Symmetric contraction, degrees 1..3, specialised kernels (gfx950).
//
// e3nn-course Lesson 12a, section 21.4.1: one row per degree nu,
// []*a[u]*b[u]...*b[u] -> C[u], all rows evaluated in one launch; weights
// chosen per atom by its element index (cuequivariance-torch skill
// document, "Other operations and layers").  For atom a and channel u, with
// v the per-channel input components:
//   out[a, L block, M, u] = sum_nu sum_k w[species[a], seg(nu, L, k)*mul + u]
//                           * sum_{m1 <= .. <= mnu} c[m.., M] v[m1] .. v[mnu]
// where c is the coupling tensor in sorted-monomial form (symmetric tensor
// entries times their number of distinct orderings), generated per
// descriptor as literal constants in S::eval.
//
// One wavefront per (atom, channel tile of 64*CPL channels), lane = channel.
// species[a] is a scalar load; the per-species weights (a few hundred KB for
// all elements) stay in L2; x and out are channel-contiguous in ir_mul.
//
// S (generated) provides: NV (input components per channel), NO (output
// components per channel), NS (weight segments); load_v<T, LAYOUT>,
// eval(v, wv, o), store<T, LAYOUT>.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "bufload.hpp"
#include "common.hpp"

namespace segpoly {
namespace kern {

constexpr int kSymconWave = 64;

template <class S, typename T, typename Index, int LAYOUT, int CPL>
__global__ void __launch_bounds__(kSymconWave)
symcon_spec_kernel(const T* __restrict__ x, const Index* __restrict__ species,
                   const T* __restrict__ w, int num_elements, int mul, T* __restrict__ out) {
  const int64_t atom = blockIdx.x;
  const int lane = threadIdx.x;
  const int tile0 = blockIdx.y * (kSymconWave * CPL);
  const int64_t sp = static_cast<int64_t>(species[atom]);
  const bool valid = sp >= 0 && sp < num_elements;  // out-of-range element: zero row
  // the atom's rows as buffer resources: per element the lane's offset is a
  // register and the component's offset a scalar, so the ir_mul loads and
  // stores and the weight loads need no per-element address arithmetic
  // (rows stay below 2 GiB: the host uses this kernel only then); mul_ir
  // rows hold a channel's components of a block contiguously, so plain
  // pointers need one address per block and load the block as one vector
  const int64_t m = mul;
  const T* xrow = x + atom * (m * S::NV);
  T* orow = out + atom * (m * S::NO);
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(xrow, m * S::NV * sizeof(T));
  const __amdgpu_buffer_rsrc_t wr = buf_rsrc(w + (valid ? sp : 0) * (m * S::NS), m * S::NS * sizeof(T));
  const __amdgpu_buffer_rsrc_t orr = buf_rsrc(orow, m * S::NO * sizeof(T));
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int u = tile0 + c * kSymconWave + lane;
    if (u < mul) {
      T o[S::NO];
      if (valid) {
        T v[S::NV];
        T wv[S::NS];
        if constexpr (LAYOUT == kIrMul)
          S::template load_v_b<T, LAYOUT>(xr, mul, u, v);
        else
          S::template load_v<T, LAYOUT>(xrow, mul, u, v);
#pragma unroll
        for (int s = 0; s < S::NS; ++s)
          wv[s] = buf_load_s<T>(wr, static_cast<uint32_t>(u) * sizeof(T), static_cast<uint32_t>(s * mul) * sizeof(T));
        S::template eval<T>(v, wv, o);
      } else {
#pragma unroll
        for (int k = 0; k < S::NO; ++k) o[k] = T(0);
      }
      if constexpr (LAYOUT == kIrMul)
        S::template store_b<T, LAYOUT>(orr, mul, u, o);
      else
        S::template store<T, LAYOUT>(orow, mul, u, o);
    }
  }
}

template <class S, typename T, typename Index, int LAYOUT, int CPL>
int symcon_spec_launch(const SymconArgs& a) {
  const int per_tile = kSymconWave * CPL;
  dim3 grid(static_cast<unsigned>(a.n_atoms), static_cast<unsigned>((a.mul + per_tile - 1) / per_tile));
  hipLaunchKernelGGL((symcon_spec_kernel<S, T, Index, LAYOUT, CPL>), grid, dim3(kSymconWave), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x),
                     static_cast<const Index*>(a.species), static_cast<const T*>(a.w), a.num_elements,
                     a.mul, static_cast<T*>(a.out));
  return static_cast<int>(hipGetLastError());
}

template <class S, typename T>
int symcon_spec_dispatch(const SymconArgs& a) {
  if (a.idx == kI32) {
    if (a.layout == kMulIr) return symcon_spec_launch<S, T, int32_t, kMulIr, 1>(a);
    return symcon_spec_launch<S, T, int32_t, kIrMul, 1>(a);
  }
  if (a.layout == kMulIr) return symcon_spec_launch<S, T, int64_t, kMulIr, 1>(a);
  return symcon_spec_launch<S, T, int64_t, kIrMul, 1>(a);
}

}  // namespace kern
}  // namespace segpoly
