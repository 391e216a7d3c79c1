// Small device helpers shared by the kernel skeletons.
#pragma once
#include <hip/hip_runtime.h>

namespace segpoly {
namespace kern {

__device__ __forceinline__ float fmadd(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fmadd(double a, double b, double c) { return __builtin_fma(a, b, c); }

}  // namespace kern
}  // namespace segpoly
