// Matrix-core (gfx950 MFMA) wrappers shared by the GEMM-shaped kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace segpoly {
namespace kern {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

// v_mfma_f32_16x16x4f32: lane l supplies A[l % 16][l / 16], B[l / 16][l % 16];
// accumulator j of lane l is C[4 (l / 16) + j][l % 16].
template <>
struct Mfma<float> {
  using acc_t = v4f;
  __device__ __forceinline__ static acc_t mma(float a, float b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static int row(int lane, int j) { return 4 * (lane / 16) + j; }
};

// v_mfma_f64_16x16x4f64: same operands; accumulator j of lane l is
// C[4 j + l / 16][l % 16].
template <>
struct Mfma<double> {
  using acc_t = v4d;
  __device__ __forceinline__ static acc_t mma(double a, double b, acc_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static int row(int lane, int j) { return 4 * j + lane / 16; }
};

}  // namespace kern
}  // namespace segpoly
