// Measurement probe (not part of the method): the memory traffic of the
// fused TP-conv forward on the large benchmark graph, replayed with trivial
// arithmetic, to time the ceiling of the access pattern itself.
//
// One 64-lane wave per destination node walks the node's edges (uniform
// in-degree, destination-sorted: node n owns edges [n deg, (n + 1) deg)),
// each lane holding two of the 128 channels, exactly as the fused kernel
// does: per edge the weight row as 13 two-float non-temporal loads, the
// gathered source row as 9 two-float loads and the 16 harmonics as uniform
// loads; the output row (43 blocks of 128 channels) is written once.  The
// shape is that of 128x0e+128x1o+128x2e with harmonics up to l = 3 and the
// 13 paths into 0e+1o+2e; other shapes are rejected.
//
// Modes: 0 weight rows only; 1 weight rows and output rows; 2 the full
// traffic (weights, gathered rows, harmonics, output rows).  nt: output rows
// written with non-temporal stores.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f2 __attribute__((ext_vector_type(2)));
constexpr int kWP = 13, kXP = 9, kOP = 43, kSH = 16, kMul = 128;

template <int MODE, bool NT>
__global__ void __launch_bounds__(64)
replay_kernel(const float* __restrict__ w, const float* __restrict__ x, const float* __restrict__ sh,
              const int* __restrict__ src, float* __restrict__ out, int64_t n_src, int deg) {
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x;
  float a0 = 0.f, a1 = 0.f;
  const int64_t e_end = (node + 1) * deg;
  for (int64_t e = node * deg; e < e_end; ++e) {
    const float* wr = w + e * (kWP * kMul) + 2 * lane;
    f2 t[kWP];
#pragma unroll
    for (int p = 0; p < kWP; ++p) t[p] = __builtin_nontemporal_load(reinterpret_cast<const f2*>(wr + p * kMul));
    if (MODE == 2) {
      int64_t s = src[e];
      s = s < 0 ? 0 : (s >= n_src ? n_src - 1 : s);  // a probe never faults on a bad index
      const float* xr = x + s * (kXP * kMul) + 2 * lane;
      f2 q[kXP];
#pragma unroll
      for (int m = 0; m < kXP; ++m) q[m] = *reinterpret_cast<const f2*>(xr + m * kMul);
      float hs = 0.f;
#pragma unroll
      for (int j = 0; j < kSH; ++j) hs += sh[e * kSH + j];
#pragma unroll
      for (int m = 0; m < kXP; ++m) {
        a0 += q[m].x * hs;
        a1 += q[m].y * hs;
      }
    }
#pragma unroll
    for (int p = 0; p < kWP; ++p) {
      a0 += t[p].x;
      a1 += t[p].y;
    }
  }
  if (MODE == 0) {
    if (a0 == 1234.5f) out[node * (kOP * kMul) + 2 * lane] = a1;  // keeps the loads; never true for the inputs used
    return;
  }
  float* orow = out + node * (kOP * kMul) + 2 * lane;
#pragma unroll
  for (int k = 0; k < kOP; ++k) {
    f2 v = {a0 + k, a1 - k};
    if (NT)
      __builtin_nontemporal_store(v, reinterpret_cast<f2*>(orow + k * kMul));
    else
      *reinterpret_cast<f2*>(orow + k * kMul) = v;
  }
}

template <int MODE, bool NT>
int launch(const float* w, const float* x, const float* sh, const int* src, float* out, int64_t n_nodes,
           int64_t n_src, int deg, hipStream_t stream) {
  hipLaunchKernelGGL((replay_kernel<MODE, NT>), dim3(static_cast<unsigned>(n_nodes)), dim3(64), 0, stream, w, x, sh,
                     src, out, n_src, deg);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

// Returns 0, -1 for a shape or argument it does not replay, or the HIP
// error of the launch.  Buffers: w [n_nodes deg, 1664], x [n_src, 1152],
// sh [n_nodes deg, 16], src [n_nodes deg] int32, out [n_nodes, 5504], all
// float32 on the device.
extern "C" int segpoly_bench_traffic_replay(int mode, int nt, const void* w, const void* x, const void* sh,
                                            const void* src, void* out, int64_t n_nodes, int64_t n_src, int deg,
                                            int64_t weight_numel, int64_t dim_in1, int64_t dim_in2, int64_t dim_out,
                                            void* stream) {
  if (weight_numel != kWP * kMul || dim_in1 != kXP * kMul || dim_in2 != kSH || dim_out != kOP * kMul) return -1;
  if (n_nodes <= 0 || n_nodes > 0x7fffffff || n_src <= 0 || deg <= 0 || !w || !out) return -1;
  if (mode == 2 && (!x || !sh || !src)) return -1;
  const auto* W = static_cast<const float*>(w);
  const auto* X = static_cast<const float*>(x);
  const auto* S = static_cast<const float*>(sh);
  const auto* I = static_cast<const int*>(src);
  auto* O = static_cast<float*>(out);
  auto st = static_cast<hipStream_t>(stream);
  switch (mode * 2 + (nt ? 1 : 0)) {
    case 0: case 1: return launch<0, false>(W, X, S, I, O, n_nodes, n_src, deg, st);
    case 2: return launch<1, false>(W, X, S, I, O, n_nodes, n_src, deg, st);
    case 3: return launch<1, true>(W, X, S, I, O, n_nodes, n_src, deg, st);
    case 4: return launch<2, false>(W, X, S, I, O, n_nodes, n_src, deg, st);
    case 5: return launch<2, true>(W, X, S, I, O, n_nodes, n_src, deg, st);
    default: return -1;
  }
}
