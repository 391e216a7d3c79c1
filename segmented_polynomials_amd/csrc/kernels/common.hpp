// Small device helpers shared by the kernel skeletons.
#pragma once
#include <hip/hip_runtime.h>

namespace segpoly {
namespace kern {

__device__ __forceinline__ float fmadd(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fmadd(double a, double b, double c) { return __builtin_fma(a, b, c); }

template <typename T>
using pair_t = T __attribute__((ext_vector_type(2)));

// One aligned pair (address aligned to 2 * sizeof(T)); NT: non-temporal.
template <typename T, bool NT>
__device__ __forceinline__ pair_t<T> ld2(const T* __restrict__ p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const pair_t<T>*>(p));
  else
    return *reinterpret_cast<const pair_t<T>*>(p);
}

template <typename T, bool NT>
__device__ __forceinline__ void st2(T* __restrict__ p, T a, T b) {
  pair_t<T> t;
  t.x = a;
  t.y = b;
  if constexpr (NT)
    __builtin_nontemporal_store(t, reinterpret_cast<pair_t<T>*>(p));
  else
    *reinterpret_cast<pair_t<T>*>(p) = t;
}

template <typename T, bool NT>
__device__ __forceinline__ T ld1(const T* __restrict__ p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <typename T, bool NT>
__device__ __forceinline__ void st1(T* __restrict__ p, T a) {
  if constexpr (NT)
    __builtin_nontemporal_store(a, p);
  else
    *p = a;
}

}  // namespace kern
}  // namespace segpoly
