// Real spherical harmonics of edge vectors and their vector-Jacobian
// product (see sh.hpp for the basis).  One thread per vector; a workgroup's
// vectors, harmonics and gradients pass through LDS so that every global
// access is a contiguous run of the block's rows.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "sh.hpp"

namespace segpoly {
namespace kern {

constexpr int kShThreads = 256;

// rows (vectors) per workgroup: 256, or 128 when the staged rows of a
// double-precision high-degree workgroup would not fit 60 KB of LDS
template <typename T, int LMAX>
constexpr int sh_rows() {
  return (kShThreads * ((LMAX + 1) * (LMAX + 1) + 3) * static_cast<int>(sizeof(T)) <= 60000) ? kShThreads
                                                                                              : kShThreads / 2;
}

template <typename T, int LMAX>
__global__ void __launch_bounds__(kShThreads)
sh_fwd_kernel(const T* __restrict__ vec, int64_t n, int normalize, ShConsts K, T* __restrict__ out) {
  constexpr int NY = (LMAX + 1) * (LMAX + 1);
  constexpr int B = sh_rows<T, LMAX>();
  __shared__ T sv[B * 3];
  __shared__ T sy[B * NY];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * B;
  const int rows = n - base < B ? static_cast<int>(n - base) : B;
  for (int i = threadIdx.x; i < rows * 3; i += B) sv[i] = vec[base * 3 + i];
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < rows) {
    T Y[NY];
    sh_eval<T, LMAX>(sv[threadIdx.x * 3], sv[threadIdx.x * 3 + 1], sv[threadIdx.x * 3 + 2], normalize != 0, K, Y);
#pragma unroll
    for (int j = 0; j < NY; ++j) sy[threadIdx.x * NY + j] = Y[j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rows * NY; i += B) out[base * NY + i] = sy[i];
}

template <typename T, int LMAX>
__global__ void __launch_bounds__(kShThreads)
sh_bwd_kernel(const T* __restrict__ vec, const T* __restrict__ g, int64_t n, int normalize, ShConsts K,
              T* __restrict__ dvec) {
  constexpr int NY = (LMAX + 1) * (LMAX + 1);
  constexpr int B = sh_rows<T, LMAX>();
  __shared__ T sv[B * 3];
  __shared__ T sg[B * NY];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * B;
  const int rows = n - base < B ? static_cast<int>(n - base) : B;
  for (int i = threadIdx.x; i < rows * 3; i += B) sv[i] = vec[base * 3 + i];
  for (int i = threadIdx.x; i < rows * NY; i += B) sg[i] = g[base * NY + i];
  __syncthreads();
  T gx = T(0), gy = T(0), gz = T(0);
  if (static_cast<int>(threadIdx.x) < rows) {
    T gr[NY];
#pragma unroll
    for (int j = 0; j < NY; ++j) gr[j] = sg[threadIdx.x * NY + j];
    sh_vjp<T, LMAX>(sv[threadIdx.x * 3], sv[threadIdx.x * 3 + 1], sv[threadIdx.x * 3 + 2], normalize != 0, K, gr,
                    gx, gy, gz);
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < rows) {
    sv[threadIdx.x * 3] = gx;
    sv[threadIdx.x * 3 + 1] = gy;
    sv[threadIdx.x * 3 + 2] = gz;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rows * 3; i += B) dvec[base * 3 + i] = sv[i];
}

template <typename T, int LMAX>
int sh_launch(const ShArgs& a) {
  constexpr int B = sh_rows<T, LMAX>();
  const unsigned blocks = static_cast<unsigned>((a.n + B - 1) / B);
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  if (a.grad == nullptr)
    hipLaunchKernelGGL((sh_fwd_kernel<T, LMAX>), dim3(blocks), dim3(B), 0, st,
                       static_cast<const T*>(a.vec), a.n, a.normalize, *a.consts, static_cast<T*>(a.out));
  else
    hipLaunchKernelGGL((sh_bwd_kernel<T, LMAX>), dim3(blocks), dim3(B), 0, st,
                       static_cast<const T*>(a.vec), static_cast<const T*>(a.grad), a.n, a.normalize, *a.consts,
                       static_cast<T*>(a.out));
  return static_cast<int>(hipGetLastError());
}

template <typename T>
int sh_dispatch(const ShArgs& a) {
  switch (a.lmax) {
    case 0: return sh_launch<T, 0>(a);
    case 1: return sh_launch<T, 1>(a);
    case 2: return sh_launch<T, 2>(a);
    case 3: return sh_launch<T, 3>(a);
    case 4: return sh_launch<T, 4>(a);
    case 5: return sh_launch<T, 5>(a);
    default: return sh_launch<T, 6>(a);
  }
}

}  // namespace kern

int launch_sh(const ShArgs& a) {
  if (a.n == 0) return 0;
  return a.dtype == kF32 ? kern::sh_dispatch<float>(a) : kern::sh_dispatch<double>(a);
}

}  // namespace segpoly
