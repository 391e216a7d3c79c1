// Loads through a buffer resource (gfx9 raw buffer, stride 0): the hardware
// checks each offset against the resource's byte count and an offset at or
// past it reads zero without touching memory.  A masked operand element is
// then one select on a 32-bit offset before the load instead of a branch or
// a select on the loaded value, and the loads of a staging pass can all be in
// flight together.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace segpoly {
namespace kern {

// word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle
constexpr int kBufWord3 = 0x00020000;
// an offset no resource reaches (byte counts are kept below it)
constexpr uint32_t kBufMasked = 0x80000000u;
constexpr int64_t kBufMaxBytes = 0x7fffffff;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  const int n = static_cast<int>(bytes < kBufMaxBytes ? bytes : kBufMaxBytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufWord3);
}

template <typename T>
__device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off);

template <>
__device__ __forceinline__ float buf_load<float>(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

template <>
__device__ __forceinline__ double buf_load<double>(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// Loads and stores with a lane offset `voff` and a wave-uniform offset
// `soff` (a scalar operand of the instruction): an element of component c
// of a channel-major row is (u, c * mul), with u per lane and c * mul the
// same for every lane.  A store at an offset past the range is dropped.
template <typename T>
__device__ __forceinline__ T buf_load_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);

template <>
__device__ __forceinline__ float buf_load_s<float>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

template <>
__device__ __forceinline__ double buf_load_s<double>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

template <typename T>
__device__ __forceinline__ void buf_store_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, T v);

template <>
__device__ __forceinline__ void buf_store_s<float>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, soff, 0);
}

template <>
__device__ __forceinline__ void buf_store_s<double>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                    double v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r,
                                        voff, soff, 0);
}

}  // namespace kern
}  // namespace segpoly
