// The fully connected product with one weight row per sample (external
// per-item weights: cuequivariance-torch skill document, "Layouts and
// weights", shared_weights=False with a [batch, weight_numel] operand; the
// three channel indices of the weights follow Lesson 12a exercise 1).  For
// sample s, output block o and path p = (i, j, o):
//   out[s, o, k, w] = sum over paths into o of sum_(u, v) W_s[p][u, v, w] A[k, u, v],
//   A[k, u, v] = alpha_o sum_(a, b) C[a, b, k] x1[s, i, a, u] x2[s, j, b, v].
// Every weight is read for one sample only, so both kernels stream the
// weight rows (and the backward writes the weight-gradient rows once).
//
// Forward: one wave per (sample, tile), a tile being an output block and up
// to 64 of its channels w.  The wave takes a path's (u, v) pairs 64 at a
// time: first lane q forms A[., u, v] of pair q of the chunk from the staged
// input rows into LDS, then lane (slot, c) with c the channel reads
// W_s[p][u, v, w0 + c] for pairs slot, slot + S, ... (S = 64 / M slots of M
// lanes, M the tile's channels rounded up to a power of two, so a step reads
// S consecutive weight rows of M channels) and accumulates acc[k] += W A[k].
// The slots are summed with cross-lane shuffles at the end of the tile.
//
// Backward: one wave per sample, all tiles in turn, with the tile's output
// gradient g[s, o, ., w] and the input-gradient rows in LDS.  Lane q owns
// pair q of a chunk: it forms A[., u, v] in registers and walks the weight
// row W_s[p][u, v, .] of its tile (16-byte loads where the rows are aligned),
// writing the weight gradient dW_s[p][u, v, w] = sum_k A[k, u, v] g[s, o, k, w]
// once and summing the weight-contracted output gradient
// R[k, u, v] = sum_w W_s[p][u, v, w] g[s, o, k, w] in registers, no
// cross-lane traffic.  Then the lanes each own input-gradient elements of
// the chunk (pairs (a, u), then (b, v)) and add
//   dx1[a, u] += sum_v sum_(b, k) C[a, b, k] x2[b, v] R[k, u, v],
//   dx2[b, v] += sum_u sum_(a, k) C[a, b, k] x1[a, u] R[k, u, v]
// (alpha_o folded into C), so no two lanes write one element and every sum
// is taken in a fixed order.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../fctp_ps_tables.hpp"
#include "../launch.hpp"
#include "bufload.hpp"
#include "common.hpp"

namespace segpoly {
namespace kern {

namespace {

// The block is one wave: its LDS operations complete in issue order, so a
// compiler barrier orders the lanes' LDS writes before other lanes' reads.
__device__ __forceinline__ void ps_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
constexpr int ps_batch() {
  return sizeof(T) == 4 ? 16 : 8;  // weight loads in flight per lane
}

// Element (comp, ch) of a block of d components and m channels.
template <int LAYOUT>
__device__ __forceinline__ int ps_idx(int comp, int ch, int d, int m) {
  return LAYOUT == kIrMul ? comp * m + ch : ch * d + comp;
}

// A[k, u, v] of pair c0 + lane of path P into As[lane][k] (zero past the
// path's pairs).
template <typename T, int LAYOUT, int D>
__device__ __forceinline__ void ps_coupled(const PsPath& P, int c0, int nuv, int lane, const T* xs1, const T* xs2,
                                           T* As, const PsList* __restrict__ lists, const PsEnt* __restrict__ ents) {
  const int j = c0 + lane;
  const bool ok = j < nuv;
  const int u = ok ? j / P.m2 : 0;
  const int v = ok ? j - u * P.m2 : 0;
  const int sa = LAYOUT == kIrMul ? P.m1 : 1;
  const int sb = LAYOUT == kIrMul ? P.m2 : 1;
  const T* r1 = xs1 + P.off1 + (LAYOUT == kIrMul ? u : u * P.d1);
  const T* r2 = xs2 + P.off2 + (LAYOUT == kIrMul ? v : v * P.d2);
#pragma unroll
  for (int k = 0; k < D; ++k) {
    const PsList L = lists[P.k_list + k];
    T s = T(0);
    for (int e = L.begin; e < L.end; ++e) {
      const PsEnt E = ents[e];
      s = fmadd(static_cast<T>(E.c) * r1[E.a * sa], r2[E.b * sb], s);
    }
    As[lane * D + k] = ok ? s : T(0);
  }
}

template <typename T, int LAYOUT, int D>
__device__ __forceinline__ void ps_fwd_tile(__amdgpu_buffer_rsrc_t wr, const T* xs1, const T* xs2, T* As,
                                            const PsTile& t, const PsPath* __restrict__ paths,
                                            const PsList* __restrict__ lists, const PsEnt* __restrict__ ents,
                                            int lane, int slot, int c, int S, T (&acc)[D]) {
  constexpr int B = ps_batch<T>();
  const bool wlane = c < t.nw;
  const int w = t.w0 + c;
  for (int p = t.path_begin; p < t.path_end; ++p) {
    const PsPath P = paths[p];
    const int nuv = P.m1 * P.m2;
    for (int c0 = 0; c0 < nuv; c0 += kPsChunk) {
      ps_coupled<T, LAYOUT, D>(P, c0, nuv, lane, xs1, xs2, As, lists, ents);
      ps_wave_sync();
      const int n_in = min(kPsChunk, nuv - c0);
      const int steps = (n_in + S - 1) / S;
      for (int s0 = 0; s0 < steps; s0 += B) {
        T wv[B];
#pragma unroll
        for (int q = 0; q < B; ++q) {
          const int j = (s0 + q) * S + slot;
          const bool ok = wlane && j < n_in;
          const uint32_t off =
              ok ? static_cast<uint32_t>((P.woff + static_cast<int64_t>(c0 + j) * t.m3 + w) * sizeof(T)) : kBufMasked;
          wv[q] = s0 + q < steps ? buf_load<T>(wr, off) : T(0);
        }
#pragma unroll
        for (int q = 0; q < B; ++q) {
          const int j = (s0 + q) * S + slot;
          if (j < n_in) {
            const T* a = As + j * D;
#pragma unroll
            for (int k = 0; k < D; ++k) acc[k] = fmadd(wv[q], a[k], acc[k]);
          }
        }
      }
      ps_wave_sync();
    }
  }
}

template <typename T, int LAYOUT, int DMAX>
__global__ __launch_bounds__(64) void fctp_ps_fwd_kernel(const T* __restrict__ x1, const T* __restrict__ x2,
                                                         const T* __restrict__ w, T* __restrict__ out, int64_t dim1,
                                                         int64_t dim2, int64_t dimo, int64_t numel,
                                                         const PsTile* __restrict__ tiles,
                                                         const PsPath* __restrict__ paths,
                                                         const PsList* __restrict__ lists,
                                                         const PsEnt* __restrict__ ents, int max_d) {
  extern __shared__ __align__(16) unsigned char ps_fwd_smem[];
  T* xs1 = reinterpret_cast<T*>(ps_fwd_smem);
  T* xs2 = xs1 + dim1;
  T* As = xs2 + dim2;
  const int64_t s = blockIdx.x;
  const PsTile t = tiles[blockIdx.y];
  const int lane = threadIdx.x;
  for (int64_t i = lane; i < dim1; i += 64) xs1[i] = x1[s * dim1 + i];
  for (int64_t i = lane; i < dim2; i += 64) xs2[i] = x2[s * dim2 + i];
  ps_wave_sync();
  const __amdgpu_buffer_rsrc_t wr = buf_rsrc(w + s * numel, numel * static_cast<int64_t>(sizeof(T)));
  const int M = 1 << t.lane_bits, S = 64 >> t.lane_bits;
  const int slot = lane >> t.lane_bits, c = lane & (M - 1);
  T* orow = out + s * dimo + t.offo;
#define SEGPOLY_PS_FWD_CASE(DD)                                                                  \
  case DD: if constexpr (DD <= DMAX) {                                                           \
    T acc[DD];                                                                                   \
    _Pragma("unroll") for (int k = 0; k < DD; ++k) acc[k] = T(0);                                \
    ps_fwd_tile<T, LAYOUT, DD>(wr, xs1, xs2, As, t, paths, lists, ents, lane, slot, c, S, acc);  \
    for (int off = M; off < 64; off <<= 1) {                                                     \
      _Pragma("unroll") for (int k = 0; k < DD; ++k) acc[k] += __shfl_xor(acc[k], off, 64);      \
    }                                                                                            \
    if (slot == 0 && c < t.nw) {                                                                 \
      _Pragma("unroll") for (int k = 0; k < DD; ++k) orow[ps_idx<LAYOUT>(k, t.w0 + c, DD, t.m3)] = acc[k]; \
    }                                                                                            \
  }                                                                                              \
  break;
  switch (t.d3) {
    SEGPOLY_PS_FWD_CASE(1)
    SEGPOLY_PS_FWD_CASE(3)
    SEGPOLY_PS_FWD_CASE(5)
    SEGPOLY_PS_FWD_CASE(7)
    SEGPOLY_PS_FWD_CASE(9)
    SEGPOLY_PS_FWD_CASE(11)
    SEGPOLY_PS_FWD_CASE(13)
    default: break;
  }
#undef SEGPOLY_PS_FWD_CASE
  (void)max_d;
}

// Input-gradient contributions of one chunk, from R[k, u, v] in Rs.
template <typename T, int LAYOUT, int D>
__device__ __forceinline__ void ps_dx(const PsPath& P, int c0, int nuv, int lane, const T* xs1, const T* xs2,
                                      const T* Rs, T* dx1a, T* dx2a, bool want1, bool want2,
                                      const PsList* __restrict__ lists, const PsEnt* __restrict__ ents) {
  const int c1 = min(c0 + kPsChunk, nuv);
  const int m1 = P.m1, m2 = P.m2, d1 = P.d1, d2 = P.d2;
  const int sa = LAYOUT == kIrMul ? m1 : 1;
  const int sb = LAYOUT == kIrMul ? m2 : 1;
  const int u_lo = c0 / m2, u_hi = (c1 - 1) / m2;
  if (want1) {
    const int npair = d1 * (u_hi - u_lo + 1);
    for (int q = lane; q < npair; q += 64) {
      const int uu = q / d1, a = q - uu * d1, u = u_lo + uu;
      const int vb = max(0, c0 - u * m2), ve = min(m2, c1 - u * m2);
      const PsList L = lists[P.a_list + a];
      T acc = T(0);
      for (int e = L.begin; e < L.end; ++e) {
        const PsEnt E = ents[e];
        const T ce = static_cast<T>(E.c);
        const T* r2 = xs2 + P.off2 + E.b * sb;
        for (int v = vb; v < ve; ++v)
          acc = fmadd(ce * r2[LAYOUT == kIrMul ? v : v * d2], Rs[(u * m2 + v - c0) * D + E.k], acc);
      }
      dx1a[P.off1 + ps_idx<LAYOUT>(a, u, d1, m1)] += acc;
    }
  }
  if (want2) {
    const int vlo = u_hi > u_lo ? 0 : c0 - u_lo * m2;
    const int vhi = u_hi > u_lo ? m2 - 1 : c1 - 1 - u_lo * m2;
    const int npair = d2 * (vhi - vlo + 1);
    for (int q = lane; q < npair; q += 64) {
      const int vv = q / d2, b = q - vv * d2, v = vlo + vv;
      const int ub = c0 > v ? (c0 - v + m2 - 1) / m2 : 0;
      const int ue = c1 - 1 >= v ? (c1 - 1 - v) / m2 : -1;
      const PsList L = lists[P.b_list + b];
      T acc = T(0);
      for (int e = L.begin; e < L.end; ++e) {
        const PsEnt E = ents[e];
        const T ce = static_cast<T>(E.c);
        const T* r1 = xs1 + P.off1 + E.a * sa;
        for (int u = ub; u <= ue; ++u)
          acc = fmadd(ce * r1[LAYOUT == kIrMul ? u : u * d1], Rs[(u * m2 + v - c0) * D + E.k], acc);
      }
      dx2a[P.off2 + ps_idx<LAYOUT>(b, v, d2, m2)] += acc;
    }
  }
}

// A[k, u, v] of pair j of path P in registers (zero if !ok).
template <typename T, int LAYOUT, int D>
__device__ __forceinline__ void ps_coupled_regs(const PsPath& P, int j, bool ok, const T* xs1, const T* xs2,
                                                const PsList* __restrict__ lists, const PsEnt* __restrict__ ents,
                                                T (&A)[D]) {
  const int u = ok ? j / P.m2 : 0;
  const int v = ok ? j - u * P.m2 : 0;
  const int sa = LAYOUT == kIrMul ? P.m1 : 1;
  const int sb = LAYOUT == kIrMul ? P.m2 : 1;
  const T* r1 = xs1 + P.off1 + (LAYOUT == kIrMul ? u : u * P.d1);
  const T* r2 = xs2 + P.off2 + (LAYOUT == kIrMul ? v : v * P.d2);
#pragma unroll
  for (int k = 0; k < D; ++k) {
    const PsList L = lists[P.k_list + k];
    T s = T(0);
    for (int e = L.begin; e < L.end; ++e) {
      const PsEnt E = ents[e];
      s = fmadd(static_cast<T>(E.c) * r1[E.a * sa], r2[E.b * sb], s);
    }
    A[k] = ok ? s : T(0);
  }
}

// Elements of a weight row a lane handles at a time: four 16-byte pieces.
template <typename T>
constexpr int ps_piece() {
  return 64 / static_cast<int>(sizeof(T));
}

// The first `cnt` (uniform) elements of a piece at byte offset `off` of a
// row, zero past them or when !ok.  VEC: 16-byte loads (the offset and cnt
// are multiples of 16 bytes).
template <typename T, bool VEC>
__device__ __forceinline__ void ps_load_piece(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok, int cnt,
                                              T (&v)[ps_piece<T>()]) {
  constexpr int PW = ps_piece<T>();
  if constexpr (VEC) {
    constexpr int VW = 16 / static_cast<int>(sizeof(T));
#pragma unroll
    for (int q = 0; q < PW / VW; ++q) {
      const uint32_t o = ok && q * VW < cnt ? off + 16u * q : kBufMasked;
      const auto raw = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
      const auto t = __builtin_bit_cast(T __attribute__((ext_vector_type(VW))), raw);
#pragma unroll
      for (int e = 0; e < VW; ++e) v[q * VW + e] = t[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < PW; ++e)
      v[e] = buf_load<T>(r, ok && e < cnt ? off + static_cast<uint32_t>(e * sizeof(T)) : kBufMasked);
  }
}

// Stores of the same elements (a masked offset drops the store).
template <typename T, bool VEC>
__device__ __forceinline__ void ps_store_piece(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok, int cnt,
                                               const T (&v)[ps_piece<T>()]) {
  constexpr int PW = ps_piece<T>();
  if constexpr (VEC) {
    constexpr int VW = 16 / static_cast<int>(sizeof(T));
#pragma unroll
    for (int q = 0; q < PW / VW; ++q) {
      if (q * VW >= cnt) break;
      T __attribute__((ext_vector_type(VW))) t;
#pragma unroll
      for (int e = 0; e < VW; ++e) t[e] = v[q * VW + e];
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, t), r,
                                             ok ? off + 16u * q : kBufMasked, 0, 0);
    }
  } else {
#pragma unroll
    for (int e = 0; e < PW; ++e) {
      if (e >= cnt) break;
      const uint32_t o = ok ? off + static_cast<uint32_t>(e * sizeof(T)) : kBufMasked;
      if constexpr (sizeof(T) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[e]), r, o, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v[e]),
                                              r, o, 0, 0);
    }
  }
}

template <typename T, int LAYOUT, int D, bool VEC>
__device__ __forceinline__ void ps_bwd_tile(__amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t dwr, bool want_dw,
                                            const T* __restrict__ grow, const T* xs1, const T* xs2, T* gsl, T* Rs,
                                            T* dx1a, T* dx2a, bool want1, bool want2, const PsTile& t,
                                            const PsPath* __restrict__ paths, const PsList* __restrict__ lists,
                                            const PsEnt* __restrict__ ents, int lane) {
  constexpr int PW = ps_piece<T>();
  const bool want_dx = want1 || want2;
  // the tile's output gradient: gsl[k * 64 + c] = g[s, o, k, w0 + c]
  for (int i = lane; i < D * t.nw; i += 64) {
    const int k = i / t.nw, c = i - k * t.nw;
    gsl[k * 64 + c] = grow[t.offo + ps_idx<LAYOUT>(k, t.w0 + c, D, t.m3)];
  }
  ps_wave_sync();
  for (int p = t.path_begin; p < t.path_end; ++p) {
    const PsPath P = paths[p];
    const int nuv = P.m1 * P.m2;
    for (int c0 = 0; c0 < nuv; c0 += kPsChunk) {
      const int j = c0 + lane;
      const bool ok = j < nuv;
      T A[D];
      if (want_dw) ps_coupled_regs<T, LAYOUT, D>(P, j, ok, xs1, xs2, lists, ents, A);
      T R[D];
#pragma unroll
      for (int k = 0; k < D; ++k) R[k] = T(0);
      const int64_t row = P.woff + static_cast<int64_t>(ok ? j : 0) * t.m3 + t.w0;
      for (int wc = 0; wc < t.nw; wc += PW) {
        const int cnt = min(PW, t.nw - wc);
        const uint32_t off = static_cast<uint32_t>((row + wc) * static_cast<int64_t>(sizeof(T)));
        T wv[PW], dv[PW];
        if (want_dx) ps_load_piece<T, VEC>(wr, off, ok, cnt, wv);
#pragma unroll
        for (int e = 0; e < PW; ++e) {
          dv[e] = T(0);
          if (e < cnt) {
            T gk[D];
#pragma unroll
            for (int k = 0; k < D; ++k) gk[k] = gsl[k * 64 + wc + e];
            if (want_dx) {
#pragma unroll
              for (int k = 0; k < D; ++k) R[k] = fmadd(wv[e], gk[k], R[k]);
            }
            if (want_dw) {
              T d = T(0);
#pragma unroll
              for (int k = 0; k < D; ++k) d = fmadd(A[k], gk[k], d);
              dv[e] = d;
            }
          }
        }
        if (want_dw) ps_store_piece<T, VEC>(dwr, off, ok, cnt, dv);
      }
      if (want_dx) {
#pragma unroll
        for (int k = 0; k < D; ++k) Rs[lane * D + k] = R[k];
        ps_wave_sync();
        ps_dx<T, LAYOUT, D>(P, c0, nuv, lane, xs1, xs2, Rs, dx1a, dx2a, want1, want2, lists, ents);
        ps_wave_sync();
      }
    }
  }
  ps_wave_sync();  // the next tile rewrites gsl
}

template <typename T, int LAYOUT, bool VEC, int DMAX>
__global__ __launch_bounds__(64) void fctp_ps_bwd_kernel(const T* __restrict__ x1, const T* __restrict__ x2,
                                                         const T* __restrict__ w, const T* __restrict__ g,
                                                         T* __restrict__ dx1, T* __restrict__ dx2,
                                                         T* __restrict__ dw, int64_t dim1, int64_t dim2,
                                                         int64_t dimo, int64_t numel,
                                                         const PsTile* __restrict__ tiles,
                                                         const PsPath* __restrict__ paths,
                                                         const PsList* __restrict__ lists,
                                                         const PsEnt* __restrict__ ents, int n_tiles, int max_d) {
  extern __shared__ __align__(16) unsigned char ps_bwd_smem[];
  T* xs1 = reinterpret_cast<T*>(ps_bwd_smem);
  T* xs2 = xs1 + dim1;
  T* dx1a = xs2 + dim2;
  T* dx2a = dx1a + dim1;
  T* gsl = dx2a + dim2;
  T* Rs = gsl + kPsChunk * max_d;
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x;
  const bool want1 = dx1 != nullptr, want2 = dx2 != nullptr;
  // an input no requested gradient reads may be null (then staged as zero)
  for (int64_t i = lane; i < dim1; i += 64) {
    xs1[i] = x1 ? x1[s * dim1 + i] : T(0);
    dx1a[i] = T(0);
  }
  for (int64_t i = lane; i < dim2; i += 64) {
    xs2[i] = x2 ? x2[s * dim2 + i] : T(0);
    dx2a[i] = T(0);
  }
  ps_wave_sync();
  const int64_t rb = numel * static_cast<int64_t>(sizeof(T));
  const __amdgpu_buffer_rsrc_t wr = buf_rsrc(w ? w + s * numel : w, w ? rb : 0);
  const __amdgpu_buffer_rsrc_t dwr = buf_rsrc(dw ? dw + s * numel : dw, dw ? rb : 0);
  const T* grow = g + s * dimo;
  const bool want_dw = dw != nullptr;
  for (int ti = 0; ti < n_tiles; ++ti) {
    const PsTile t = tiles[ti];
#define SEGPOLY_PS_BWD_CASE(DD)                                                                                  \
  case DD:                                                                                                       \
    if constexpr (DD <= DMAX)                                                                                    \
    ps_bwd_tile<T, LAYOUT, DD, VEC>(wr, dwr, want_dw, grow, xs1, xs2, gsl, Rs, dx1a, dx2a, want1, want2, t,      \
                                    paths, lists, ents, lane);                                                   \
    break;
    switch (t.d3) {
      SEGPOLY_PS_BWD_CASE(1)
      SEGPOLY_PS_BWD_CASE(3)
      SEGPOLY_PS_BWD_CASE(5)
      SEGPOLY_PS_BWD_CASE(7)
      SEGPOLY_PS_BWD_CASE(9)
      SEGPOLY_PS_BWD_CASE(11)
      SEGPOLY_PS_BWD_CASE(13)
      default: break;
    }
#undef SEGPOLY_PS_BWD_CASE
  }
  ps_wave_sync();
  if (want1)
    for (int64_t i = lane; i < dim1; i += 64) dx1[s * dim1 + i] = dx1a[i];
  if (want2)
    for (int64_t i = lane; i < dim2; i += 64) dx2[s * dim2 + i] = dx2a[i];
}

// The kernels are compiled for output blocks up to DMAX components (3, 7 or
// 13): registers are allocated for the largest block a kernel handles.
template <typename T, int LAYOUT, int DMAX>
int ps_fwd_launch(const FcPsArgs& a) {
  const dim3 grid(static_cast<unsigned>(a.n), static_cast<unsigned>(a.n_tiles));
  hipLaunchKernelGGL((fctp_ps_fwd_kernel<T, LAYOUT, DMAX>), grid, dim3(64), a.lds_bytes, static_cast<hipStream_t>(a.stream),
                     static_cast<const T*>(a.x1), static_cast<const T*>(a.x2), static_cast<const T*>(a.w),
                     static_cast<T*>(a.out), a.dim1, a.dim2, a.dimo, a.numel, a.tiles, a.paths, a.lists, a.ents,
                     a.max_d);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int LAYOUT, bool VEC, int DMAX>
int ps_bwd_launch(const FcPsArgs& a) {
  hipLaunchKernelGGL((fctp_ps_bwd_kernel<T, LAYOUT, VEC, DMAX>), dim3(static_cast<unsigned>(a.n)), dim3(64), a.lds_bytes,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x1), static_cast<const T*>(a.x2),
                     static_cast<const T*>(a.w), static_cast<const T*>(a.g), static_cast<T*>(a.dx1),
                     static_cast<T*>(a.dx2), static_cast<T*>(a.dw), a.dim1, a.dim2, a.dimo, a.numel, a.tiles,
                     a.paths, a.lists, a.ents, a.n_tiles, a.max_d);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int DMAX>
int ps_fwd_dispatch(const FcPsArgs& a) {
  return a.layout == kIrMul ? ps_fwd_launch<T, kIrMul, DMAX>(a) : ps_fwd_launch<T, kMulIr, DMAX>(a);
}

template <typename T>
int ps_fwd_dispatch(const FcPsArgs& a) {
  if (a.max_d <= 3) return ps_fwd_dispatch<T, 3>(a);
  if (a.max_d <= 7) return ps_fwd_dispatch<T, 7>(a);
  return ps_fwd_dispatch<T, kPsMaxD>(a);
}

template <typename T, int DMAX>
int ps_bwd_dispatch(const FcPsArgs& a) {
  if (a.vec)
    return a.layout == kIrMul ? ps_bwd_launch<T, kIrMul, true, DMAX>(a) : ps_bwd_launch<T, kMulIr, true, DMAX>(a);
  return a.layout == kIrMul ? ps_bwd_launch<T, kIrMul, false, DMAX>(a) : ps_bwd_launch<T, kMulIr, false, DMAX>(a);
}

template <typename T>
int ps_bwd_dispatch(const FcPsArgs& a) {
  if (a.max_d <= 3) return ps_bwd_dispatch<T, 3>(a);
  if (a.max_d <= 7) return ps_bwd_dispatch<T, 7>(a);
  return ps_bwd_dispatch<T, kPsMaxD>(a);
}

}  // namespace

}  // namespace kern

int launch_fctp_ps_fwd(const FcPsArgs& a) {
  if (a.n == 0 || a.n_tiles == 0) return 0;
  return a.dtype == kF32 ? kern::ps_fwd_dispatch<float>(a) : kern::ps_fwd_dispatch<double>(a);
}

int launch_fctp_ps_bwd(const FcPsArgs& a) {
  if (a.n == 0) return 0;
  return a.dtype == kF32 ? kern::ps_bwd_dispatch<float>(a) : kern::ps_bwd_dispatch<double>(a);
}

}  // namespace segpoly
