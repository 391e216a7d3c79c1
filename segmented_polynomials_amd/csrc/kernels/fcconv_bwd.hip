// Backward (vector-Jacobian product) of the fully connected convolution
// with per-edge weights.  With G = dL/d(out)[dst_e] (divided by the in-degree
// for reduce="mean") and, per path p = (i, j, o) of edge e,
//   y[p, k, u] = alpha_o sum_(a, b) C[a, b, k] x[src_e, i, a, u] sh[e, j, b]   (the forward's rows)
//   z[p, k, u] = sum_w W_e[p][u, w] G[o, k, w]
// the gradients are
//   dW_e[p][u, w]     = sum_k y[p, k, u] G[o, k, w]
//   dsh[e, j, b]     += alpha_o sum_(a, k, u) C[a, b, k] x[src_e, i, a, u] z[p, k, u]
//   msg_e[i, a, u]   += alpha_o sum_(b, k) C[a, b, k] sh[e, j, b] z[p, k, u]
//   dx[s]             = sum over the edges e with src_e = s of msg_e.
// fcconv_bwd_edge_kernel: one wave per destination, the forward's lane
// slots (S edges at once, lane (slot, c)); dW and dsh are written per edge
// (each edge belongs to one destination), the messages go to the workspace.
// Edges whose destination lies outside [0, n_nodes) get zero gradients
// (written by the first and the last destination's wave).
// fcconv_bwd_src_kernel: one wave per source sums its edges' messages in
// the order of the caller's source permutation (deterministic, no atomics).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../fcconv_tables.hpp"
#include "../launch.hpp"
#include "common.hpp"
#include "tp_conv_bwd.hpp"
#include "tp_conv_spec.hpp"

namespace segpoly {
namespace kern {

__device__ __forceinline__ void fcb_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One path of one edge and one u tile (input channels ub .. ub + M - 1), for
// an output block of D components:
//   z[row + k, u] = sum_w W[u, w] G[k, w]     (lane = input channel u, the
//                                            weight row read once, 16 channels at a time)
//   dW[u, w]      = sum_k y[row + k, u] G[k, w] (lane = output channel w, G[., w] in registers)
template <typename T, int LAYOUT, int D, bool SHW, bool WIDE>
__device__ __forceinline__ void fcb_path(const FcvBPath& P, const T* __restrict__ w, int64_t e, int64_t numel,
                                         bool valid, int M, int c, int ub_, const T* Gs, const T* ys, T* zs,
                                         T* __restrict__ dw) {
  const int ub = WIDE ? ub_ : 0;  // one u tile: every channel of the path is a lane
  auto gi = [&](int k, int wc) -> int {
    return static_cast<int>(P.g_off) + (LAYOUT == kIrMul ? k * P.m3 + wc : wc * D + k);
  };
  {  // every lane stores its z rows (zero past mul1: the message phase reads them all)
    T z[D];
#pragma unroll
    for (int k = 0; k < D; ++k) z[k] = T(0);
    if (valid && ub + c < P.m1) {
      const T* wr = w + (SHW ? 0 : e * numel) + P.w_off + static_cast<int64_t>(ub + c) * P.m3;
      int w0 = 0;
      // 16-byte vector loads where the row is aligned (it is whenever m3
      // is a multiple of 16 / sizeof(T) channels), else plain loads
      const bool vec = (reinterpret_cast<uintptr_t>(wr) % 16) == 0 && (P.m3 * sizeof(T)) % 16 == 0;
      for (; w0 + 16 <= P.m3; w0 += 16) {
        T wv[16];
        if (vec) {
          constexpr int kV = 16 / sizeof(T);
          typedef T vec_t __attribute__((ext_vector_type(kV)));
#pragma unroll
          for (int i = 0; i < 16; i += kV) {
            const vec_t v = *reinterpret_cast<const vec_t*>(wr + w0 + i);
#pragma unroll
            for (int j = 0; j < kV; ++j) wv[i + j] = v[j];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) wv[i] = wr[w0 + i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int k = 0; k < D; ++k) z[k] = fmadd(wv[i], Gs[gi(k, w0 + i)], z[k]);
      }
      for (; w0 < P.m3; ++w0) {
        const T wv = wr[w0];
#pragma unroll
        for (int k = 0; k < D; ++k) z[k] = fmadd(wv, Gs[gi(k, w0)], z[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < D; ++k) zs[(P.row + k) * M + c] = z[k];
  }
  if (valid)
    for (int wc = c; wc < P.m3; wc += M) {
      T gk[D];
#pragma unroll
      for (int k = 0; k < D; ++k) gk[k] = Gs[gi(k, wc)];
      T* dwr = dw + e * numel + P.w_off + wc;
      const T* yr = ys + P.row * M - ub;
      const int u1 = WIDE && ub + M < P.m1 ? ub + M : P.m1;
#pragma unroll 4
      for (int u = ub; u < u1; ++u) {
        T t = T(0);
#pragma unroll
        for (int k = 0; k < D; ++k) t = fmadd(yr[k * M + u], gk[k], t);
        dwr[static_cast<int64_t>(u) * P.m3] = t;
      }
    }
}

// SHW: one weight row shared by every edge (the dw rows stay per edge).
// WIDE: input-1 blocks of more than 64 channels, taken a u tile at a time
// (a separate instance: the u-tile loop costs the one-tile case registers,
// 167 -> 237 VGPRs for float ir_mul, and a wave per SIMD).
template <typename T, typename Index, int LAYOUT, bool SHW, bool WIDE>
__global__ void __launch_bounds__(64)
fcconv_bwd_edge_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                       const T* __restrict__ g, const Index* __restrict__ src, const Index* __restrict__ dst,
                       int64_t n_src, int64_t n_edges, int64_t n_nodes, int64_t dim1, int64_t dim2, int64_t dimo,
                       int64_t numel, int mean, T* __restrict__ dsh, T* __restrict__ dw, T* __restrict__ msg,
                       const FcvBlock* __restrict__ blocks, const FcvQK* __restrict__ qks,
                       const FcvEnt* __restrict__ ents, const FcvBPath* __restrict__ bpaths, int n_blocks,
                       int n_bpaths, int nrows, int ncomp, int lane_bits, int n_ut) {
  extern __shared__ __align__(16) unsigned char fcb_smem[];
  T* lds = reinterpret_cast<T*>(fcb_smem);
  const int64_t node = blockIdx.x;
  const int lane = threadIdx.x;
  const int M = 1 << lane_bits;
  const int S = 64 >> lane_bits;
  const int slot = lane >> lane_bits, c = lane & (M - 1);
  // per-slot regions, strides padded by one: x, harmonics, y rows, z rows,
  // messages, harmonic-gradient partials; then the node's gradient row
  const int XS = ncomp * M + 1, SH = static_cast<int>(dim2) + 1, YS = nrows * M + 1, HS = static_cast<int>(dim2) * M + 1;
  const int per_slot = 2 * XS + SH + 2 * YS + HS;
  T* base = lds + slot * per_slot;
  T* xs = base;
  T* ms = xs + XS;
  T* shs = ms + XS;
  T* ys = shs + SH;
  T* zs = ys + YS;
  T* hp = zs + YS;
  T* Gs = lds + S * per_slot;

  int64_t e0, e1;
  edge_range(dst, n_edges, 0, node, e0, e1);

  // edges of no destination: zero gradients and messages
  auto zero_edges = [&](int64_t a, int64_t b) {
    for (int64_t e = a; e < b; ++e) {
      for (int64_t i = lane; i < numel; i += 64) dw[e * numel + i] = T(0);
      for (int64_t i = lane; i < dim2; i += 64) dsh[e * dim2 + i] = T(0);
      for (int64_t i = lane; i < dim1; i += 64) msg[e * dim1 + i] = T(0);
    }
  };
  if (node == 0) zero_edges(0, e0);
  if (node == n_nodes - 1) zero_edges(e1, n_edges);

  const T scale = (mean && e1 > e0) ? T(1) / static_cast<T>(e1 - e0) : T(1);
  for (int64_t i = lane; i < dimo; i += 64) Gs[i] = scale * g[node * dimo + i];
  fcb_wave_sync();

  for (int64_t eb = e0; eb < e1; eb += S) {
    const int64_t e = eb + slot;
    const bool valid = e < e1;
    const int64_t s = valid ? static_cast<int64_t>(src[e]) : int64_t(-1);
    const bool ok = s >= 0 && s < n_src;
    // one u tile (input channels ub .. ub + M - 1) at a time; one tile when
    // no block has more than 64 channels
    const int nut = WIDE ? n_ut : 1;
    for (int ut = 0; ut < nut; ++ut) {
      const int ub = ut * kFcvUTile;
      const int u = ub + c;  // this lane's input channel
      // stage x[src] (zero for an out-of-range source)
      for (int bi = 0; bi < n_blocks; ++bi) {
        const FcvBlock B = blocks[bi];
        const bool on = ok && u < B.m;
        for (int a = 0; a < B.d; ++a) {
          const int64_t off = LAYOUT == kIrMul ? B.off + static_cast<int64_t>(a) * B.m + u
                                               : B.off + static_cast<int64_t>(u) * B.d + a;
          xs[(B.comp + a) * M + c] = on ? x[s * dim1 + off] : T(0);
          ms[(B.comp + a) * M + c] = T(0);
        }
      }
      if (ut == 0) {  // the harmonics, and the harmonic-gradient partials every u tile adds to
        for (int b = c; b < dim2; b += M) shs[b] = valid ? sh[e * dim2 + b] : T(0);
        for (int b = 0; b < dim2; ++b) hp[b * M + c] = T(0);
      }
      fcb_wave_sync();
      // coupled rows y (lane = input channel)
      for (int r = 0; r < nrows; ++r) {
        const FcvQK Q = qks[r];
        T t = T(0);
        for (int en = Q.ent_begin; en < Q.ent_end; ++en) {
          const FcvEnt E = ents[en];
          t = fmadd(static_cast<T>(E.c) * shs[E.b], xs[E.a * M + c], t);
        }
        ys[r * M + c] = t;
      }
      fcb_wave_sync();
      // per path: z rows (lane = input channel) and dW (lane = output channel)
      for (int pi = 0; pi < n_bpaths; ++pi) {
        const FcvBPath P = bpaths[pi];
        switch (P.d3) {
          case 1: fcb_path<T, LAYOUT, 1, SHW, WIDE>(P, w, e, numel, valid, M, c, ub, Gs, ys, zs, dw); break;
          case 3: fcb_path<T, LAYOUT, 3, SHW, WIDE>(P, w, e, numel, valid, M, c, ub, Gs, ys, zs, dw); break;
          case 5: fcb_path<T, LAYOUT, 5, SHW, WIDE>(P, w, e, numel, valid, M, c, ub, Gs, ys, zs, dw); break;
          case 7: fcb_path<T, LAYOUT, 7, SHW, WIDE>(P, w, e, numel, valid, M, c, ub, Gs, ys, zs, dw); break;
          case 9: fcb_path<T, LAYOUT, 9, SHW, WIDE>(P, w, e, numel, valid, M, c, ub, Gs, ys, zs, dw); break;
          case 11: fcb_path<T, LAYOUT, 11, SHW, WIDE>(P, w, e, numel, valid, M, c, ub, Gs, ys, zs, dw); break;
          default: fcb_path<T, LAYOUT, 13, SHW, WIDE>(P, w, e, numel, valid, M, c, ub, Gs, ys, zs, dw); break;
        }
      }
      // messages and harmonic-gradient partials (lane = input channel)
      for (int r = 0; r < nrows; ++r) {
        const FcvQK Q = qks[r];
        const T zv = zs[r * M + c];
        for (int en = Q.ent_begin; en < Q.ent_end; ++en) {
          const FcvEnt E = ents[en];
          const T cz = static_cast<T>(E.c) * zv;
          ms[E.a * M + c] = fmadd(cz, shs[E.b], ms[E.a * M + c]);
          hp[E.b * M + c] = fmadd(cz, xs[E.a * M + c], hp[E.b * M + c]);
        }
      }
      if (valid) {
        for (int bi = 0; bi < n_blocks; ++bi) {
          const FcvBlock B = blocks[bi];
          if (u < B.m)
            for (int a = 0; a < B.d; ++a) {
              const int64_t off = LAYOUT == kIrMul ? B.off + static_cast<int64_t>(a) * B.m + u
                                                   : B.off + static_cast<int64_t>(u) * B.d + a;
              msg[e * dim1 + off] = ms[(B.comp + a) * M + c];
            }
        }
      }
      fcb_wave_sync();
    }
    // dsh[e, b] = sum over the slot's lanes of hp[b] (every u tile added in)
    for (int b = 0; b < dim2; ++b) {
      T v = hp[b * M + c];
      for (int dd = 1; dd < M; dd <<= 1) v += __shfl_xor(v, dd);
      if (valid && c == 0) dsh[e * dim2 + b] = v;
    }
    fcb_wave_sync();
  }
}

// dx[s] = sum of the messages of the edges that read s, in permutation order.
template <typename T, typename Index>
__global__ void __launch_bounds__(64)
fcconv_bwd_src_kernel(const Index* __restrict__ src, const Index* __restrict__ perm, const T* __restrict__ msg,
                      int64_t n_edges, int64_t dim1, T* __restrict__ dx) {
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t i0 = lower_bound_perm(src, perm, n_edges, 0, n_edges, s);
  const int64_t i1 = lower_bound_perm(src, perm, n_edges, i0, n_edges, s + 1);
  for (int64_t j = lane; j < dim1; j += 64) {
    T acc = T(0);
    for (int64_t i = i0; i < i1; ++i) {
      const int64_t e = static_cast<int64_t>(perm[i]);
      if (e < 0 || e >= n_edges) continue;  // only an invalid permutation gets here
      acc += msg[e * dim1 + j];
    }
    dx[s * dim1 + j] = acc;
  }
}

template <typename T, typename Index, int LAYOUT, bool SHW>
void fcconv_bwd_edges(const FcvBwdArgs& a, T* dwe, hipStream_t st) {
  if (a.n_ut > 1) {
    hipLaunchKernelGGL((fcconv_bwd_edge_kernel<T, Index, LAYOUT, SHW, true>), dim3(static_cast<unsigned>(a.n_nodes)),
                       dim3(64), a.lds_bytes, st, static_cast<const T*>(a.x), static_cast<const T*>(a.sh),
                       static_cast<const T*>(a.w), static_cast<const T*>(a.g), static_cast<const Index*>(a.src),
                       static_cast<const Index*>(a.dst), a.n_src, a.n_edges, a.n_nodes, a.dim1, a.dim2, a.dimo,
                       a.numel, a.mean, static_cast<T*>(a.dsh), dwe, static_cast<T*>(a.msg), a.blocks, a.qks,
                       a.ents, a.bpaths, a.n_blocks, a.n_bpaths, a.nrows, a.ncomp, a.lane_bits, a.n_ut);
    return;
  }
  hipLaunchKernelGGL((fcconv_bwd_edge_kernel<T, Index, LAYOUT, SHW, false>), dim3(static_cast<unsigned>(a.n_nodes)), dim3(64),
                     a.lds_bytes, st, static_cast<const T*>(a.x), static_cast<const T*>(a.sh),
                     static_cast<const T*>(a.w), static_cast<const T*>(a.g), static_cast<const Index*>(a.src),
                     static_cast<const Index*>(a.dst), a.n_src, a.n_edges, a.n_nodes, a.dim1, a.dim2, a.dimo,
                     a.numel, a.mean, static_cast<T*>(a.dsh), dwe, static_cast<T*>(a.msg), a.blocks, a.qks, a.ents,
                     a.bpaths, a.n_blocks, a.n_bpaths, a.nrows, a.ncomp, a.lane_bits, a.n_ut);
}

template <typename T, typename Index, int LAYOUT>
int fcconv_bwd_launch(const FcvBwdArgs& a) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  // shared weights: per-edge gradient rows in the workspace, summed below
  T* const dwe = a.shared_w ? reinterpret_cast<T*>(static_cast<unsigned char*>(a.msg) + a.dw_ws_off)
                            : static_cast<T*>(a.dw);
  if (a.n_nodes > 0 && a.n_edges > 0) {
    if (a.shared_w)
      fcconv_bwd_edges<T, Index, LAYOUT, true>(a, dwe, st);
    else
      fcconv_bwd_edges<T, Index, LAYOUT, false>(a, dwe, st);
  } else if (a.n_edges > 0) {  // no destinations: every edge lies outside the output
    fill_zero(static_cast<T*>(a.dw), a.shared_w ? a.numel : a.n_edges * a.numel, st);
    fill_zero(static_cast<T*>(a.dsh), a.n_edges * a.dim2, st);
    fill_zero(static_cast<T*>(a.msg), a.n_edges * a.dim1, st);
  }
  int rc = static_cast<int>(hipGetLastError());
  if (rc) return rc;
  if (a.shared_w && a.n_nodes > 0 && a.n_edges > 0 && a.numel > 0) {
    const int64_t chunks = (a.n_edges + kTpDwChunk - 1) / kTpDwChunk;
    T* const dpart = reinterpret_cast<T*>(reinterpret_cast<unsigned char*>(dwe) +
                                          round_up_256(a.n_edges * a.numel * static_cast<int64_t>(sizeof(T))));
    hipLaunchKernelGGL((dw_edge_sum_kernel<T>), dim3(static_cast<unsigned>((a.numel + 255) / 256),
                                                     static_cast<unsigned>(chunks)),
                       dim3(256), 0, st, static_cast<const T*>(dwe), a.n_edges, a.numel, dpart);
    const int64_t blocks = (a.numel + 255) / 256;
    hipLaunchKernelGGL((fold_partials_kernel<T>), dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                       dim3(256), 0, st, static_cast<const T*>(dpart), static_cast<int>(chunks), a.numel,
                       static_cast<T*>(a.dw));
    rc = static_cast<int>(hipGetLastError());
    if (rc) return rc;
  }
  if (a.n_src == 0) return rc;
  hipLaunchKernelGGL((fcconv_bwd_src_kernel<T, Index>), dim3(static_cast<unsigned>(a.n_src)), dim3(64), 0, st,
                     static_cast<const Index*>(a.src), static_cast<const Index*>(a.perm),
                     static_cast<const T*>(a.msg), a.n_edges, a.dim1, static_cast<T*>(a.dx));
  return static_cast<int>(hipGetLastError());
}

template <typename T>
int fcconv_bwd_dispatch(const FcvBwdArgs& a) {
  if (a.idx == kI64)
    return a.layout == kMulIr ? fcconv_bwd_launch<T, int64_t, kMulIr>(a) : fcconv_bwd_launch<T, int64_t, kIrMul>(a);
  return a.layout == kMulIr ? fcconv_bwd_launch<T, int32_t, kMulIr>(a) : fcconv_bwd_launch<T, int32_t, kIrMul>(a);
}

}  // namespace kern

int launch_fcconv_bwd(const FcvBwdArgs& a) {
  return a.dtype == kF32 ? kern::fcconv_bwd_dispatch<float>(a) : kern::fcconv_bwd_dispatch<double>(a);
}

}  // namespace segpoly
