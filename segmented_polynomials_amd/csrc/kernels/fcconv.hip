// The fully connected product as a graph convolution with per-edge weights
// (cuequivariance-torch skill document, "Other operations and layers":
// FullyConnectedTensorProductConv takes source features, edge harmonics and
// one weight row per edge from its edge MLP, and sums or averages into the
// destinations).  For destination n and an output block o:
//   out[n, o, k, w] = s_n sum over edges e into n of sum over paths (i, j, o) of
//                     sum_u W_e[p][u, w] y[p, k, u],
//   y[p, k, u] = alpha_o sum_(a, b) C[a, b, k] x[src_e, i, a, u] sh[e, j, b],
// the weights W_e of a path being an mul1 x mul3 matrix (the harmonics have
// one channel per degree).
//
// One wave per (destination, tile); a tile is one output block o and up to 64
// of its channels, so every weight element is read by exactly one wave.  The
// wave works on S = 64 / M edges at once (M = the channel count rounded up
// to a power of two): lane (slot, c) first stages channel c of the slot's
// edge (x gathered by source, the harmonics row), then forms the coupled
// rows y[p, k, c] (lane = input channel u), and then accumulates for output
// channel w = c: acc[k] += W_e[p][u, w] y[p, k, u] over u, reading y as LDS
// broadcasts and the weight rows coalesced over w.  Destination edge ranges
// come from the wave-cooperative search of the channelwise convolution; the
// slots are summed with cross-lane shuffles at the end and each output value
// is written once (zero rows for destinations without edges).  Edges whose
// source is out of range contribute nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../fcconv_tables.hpp"
#include "../launch.hpp"
#include "common.hpp"
#include "tp_conv_spec.hpp"

namespace segpoly {
namespace kern {

// The block is one wave: LDS operations of a wave complete in issue order,
// so sharing staged rows between lanes needs only a compiler barrier (no
// s_barrier, and no wait for the weight loads still in flight).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The edge loop of one (destination, tile) for an output block of D
// components (compile-time, so the component loops carry no run-time
// guards).  With more than 64 input-1 channels each edge is taken one u tile
// (64 channels, one edge per wave) at a time: stage that tile of x[src],
// form its coupled rows, mix its weight elements.
template <typename T, typename Index, int LAYOUT, int D>
__device__ __forceinline__ void fcv_run(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
                                        const Index* __restrict__ src, int64_t n_src, int64_t e0, int64_t e1,
                                        int64_t dim1, int64_t dim2, int64_t w_stride, const FcvTile& tile,
                                        const FcvBlock* __restrict__ blocks, const FcvQK* __restrict__ qks,
                                        const FcvEnt* __restrict__ ents, const FcvQ* __restrict__ qs,
                                        const FcvChunk* __restrict__ chunks, const FcvUT* __restrict__ uts, int n_ut,
                                        int n_blocks, int M, int S, int slot, int c, T* xs, T* shs, T* ys,
                                        T (&acc)[D]) {
  constexpr int kB = sizeof(T) == 4 ? kFcvBatch : kFcvBatch / 2;  // chunks held in registers
  const bool wlane = c < tile.nw;
  auto source = [&](int64_t e) -> int64_t { return e < e1 ? static_cast<int64_t>(src[e]) : int64_t(-1); };
  // A batch of weight chunks b0 .. b0 + kB - 1 of u tile U, branch-free:
  // every load is issued before any is used (a guarded load per element
  // made each chunk wait for the previous one).  A chunk past the u tile's
  // last re-reads its last chunk and is never used; a lane past the tile's
  // channels reads channel 0; a slot past the edge range reads the range's
  // first edge.  Lanes whose edge has no valid source skip the mixing
  // (their weights are not used at all).
  T wr[kB][kFcvChunkU];
  auto fetch_w = [&](const FcvChunk* tc, int n_chunks, int b0, const T* wl) {
    int64_t off[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) off[i] = tc[b0 + i < n_chunks ? b0 + i : n_chunks - 1].off;
#pragma unroll
    for (int i = 0; i < kB; ++i)
#pragma unroll
      for (int uu = 0; uu < kFcvChunkU; ++uu) wr[i][uu] = wl[off[i] + uu * tile.m];
  };
  int64_t s_next = source(e0 + slot);
  for (int64_t eb = e0; eb < e1; eb += S) {
    const int64_t e = eb + slot;
    const int64_t s = s_next;
    const bool ok = s >= 0 && s < n_src;
    const bool wok = ok && wlane;
    const T* wl = w + (e < e1 ? e : e0) * w_stride + tile.w0 + (wlane ? c : 0);
    s_next = source(eb + S + slot);
    for (int b = c; b < dim2; b += M) shs[b] = ok ? sh[e * dim2 + b] : T(0);
    for (int ut = 0; ut < n_ut; ++ut) {
      const FcvUT U = uts[tile.ut_begin + ut];
      const FcvChunk* tc = chunks + U.chunk_begin;
      const FcvQ* tq = qs + U.q_begin;
      const int ub = ut * kFcvUTile;  // first channel of the u tile (0 with one u tile)
      const int u = ub + c;           // this lane's input channel
      // the first batch of weight chunks, issued before anything waits on memory
      if (U.n_chunks > 0) fetch_w(tc, U.n_chunks, 0, wl);
      // stage the slot's edge: x[src] (all input-1 blocks, this u tile)
      for (int bi = 0; bi < n_blocks; ++bi) {
        const FcvBlock B = blocks[bi];
        const bool on = ok && u < B.m;
        for (int a = 0; a < B.d; ++a) {
          const int64_t off = LAYOUT == kIrMul ? B.off + static_cast<int64_t>(a) * B.m + u
                                               : B.off + static_cast<int64_t>(u) * B.d + a;
          xs[(B.comp + a) * M + c] = on ? x[s * dim1 + off] : T(0);
        }
      }
      wave_sync();
      // coupled rows, lane = input channel
      for (int r = 0; r < tile.nqk; ++r) {
        const FcvQK Q = qks[tile.qk_begin + r];
        T t = T(0);
        for (int en = Q.ent_begin; en < Q.ent_end; ++en) {
          const FcvEnt E = ents[en];
          t = fmadd(static_cast<T>(E.c) * shs[E.b], xs[E.a * M + c], t);
        }
        ys[r * M + c] = t;
      }
      wave_sync();
      // mixing, lane = output channel: acc[k] += W[u, w] y[qk + k, u]
      for (int b0 = 0; b0 < U.n_chunks; b0 += kB) {
        if (b0 > 0) fetch_w(tc, U.n_chunks, b0, wl);
        if (wok) {
#pragma unroll
          for (int i = 0; i < kB; ++i)
            if (b0 + i < U.n_chunks) {
              const FcvChunk C = tc[b0 + i];
              const T* yq = ys + C.qk * M + (C.u0 - ub);
#pragma unroll
              for (int uu = 0; uu < kFcvChunkU; ++uu)
#pragma unroll
                for (int k = 0; k < D; ++k) acc[k] = fmadd(wr[i][uu], yq[k * M + uu], acc[k]);
            }
        }
      }
      for (int q = 0; q < U.nq; ++q) {  // channels past the last full chunk
        const FcvQ Q = tq[q];
        const T wv = wl[Q.off];
        const T* yq = ys + Q.qk * M + (Q.u - ub);
        if (wok) {
#pragma unroll
          for (int k = 0; k < D; ++k) acc[k] = fmadd(wv, yq[k * M], acc[k]);
        }
      }
      wave_sync();
    }
  }
}

template <typename T, int LAYOUT, int D>
__device__ __forceinline__ void fcv_store(T (&acc)[D], const FcvTile& tile, T* __restrict__ out, int64_t node,
                                          int64_t dimo, int M, int slot, int c, T scale) {
  // sum the slots (lanes c, c + M, c + 2M, ...)
  for (int dd = M; dd < 64; dd <<= 1) {
#pragma unroll
    for (int k = 0; k < D; ++k) acc[k] += __shfl_xor(acc[k], dd);
  }
  if (slot == 0 && c < tile.nw) {
    T* orow = out + node * dimo + tile.out_off;
    const int wc = tile.w0 + c;
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const int64_t off = LAYOUT == kIrMul ? static_cast<int64_t>(k) * tile.m + wc : static_cast<int64_t>(wc) * D + k;
      orow[off] = scale * acc[k];
    }
  }
}

// The float kernels are held to four waves per SIMD (their register
// allocation otherwise allows three; a few registers spill, and on the
// 600k-edge graph the four waves still win: 0.79 -> 0.76 ms mul_ir,
// 0.76 -> 0.72 ms ir_mul); double keeps the compiler's choice.
template <typename T, typename Index, int LAYOUT>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 4 : 1)))
fcconv_kernel(const T* __restrict__ x, const T* __restrict__ sh, const T* __restrict__ w,
              const Index* __restrict__ src, const Index* __restrict__ dst, int64_t n_src, int64_t n_edges,
              int64_t dim1, int64_t dim2, int64_t dimo, int64_t w_stride, int mean, T* __restrict__ out,
              const FcvBlock* __restrict__ blocks, const FcvQK* __restrict__ qks, const FcvEnt* __restrict__ ents,
              const FcvTile* __restrict__ tiles, const FcvQ* __restrict__ qs, const FcvChunk* __restrict__ chunks,
              const FcvUT* __restrict__ uts, int n_ut, int n_blocks, int ncomp, int max_nqk, int lane_bits) {
  extern __shared__ __align__(16) unsigned char fcv_smem[];
  T* lds = reinterpret_cast<T*>(fcv_smem);
  const int64_t node = blockIdx.x;
  const FcvTile tile = tiles[blockIdx.y];
  const int lane = threadIdx.x;
  const int M = 1 << lane_bits;
  const int S = 64 >> lane_bits;
  const int slot = lane >> lane_bits, c = lane & (M - 1);
  // per-slot LDS regions (strides padded by one so slots fall on different banks)
  const int XS = ncomp * M + 1, SH = static_cast<int>(dim2) + 1, YS = max_nqk * M + 1;
  T* xs = lds + slot * XS;
  T* shs = lds + S * XS + slot * SH;
  T* ys = lds + S * (XS + SH) + slot * YS;

  int64_t e0, e1;
  edge_range(dst, n_edges, 0, node, e0, e1);
  const T scale = (mean && e1 > e0) ? T(1) / static_cast<T>(e1 - e0) : T(1);

#define SEGPOLY_FCV_CASE(DD)                                                                                    \
  case DD: {                                                                                                    \
    T acc[DD];                                                                                                  \
    for (int k = 0; k < DD; ++k) acc[k] = T(0);                                                                 \
    fcv_run<T, Index, LAYOUT, DD>(x, sh, w, src, n_src, e0, e1, dim1, dim2, w_stride, tile, blocks, qks, ents, qs, \
                                  chunks, uts, n_ut, n_blocks, M, S, slot, c, xs, shs, ys, acc);                 \
    fcv_store<T, LAYOUT, DD>(acc, tile, out, node, dimo, M, slot, c, scale);                                    \
    break;                                                                                                      \
  }
  switch (tile.d) {
    SEGPOLY_FCV_CASE(1)
    SEGPOLY_FCV_CASE(3)
    SEGPOLY_FCV_CASE(5)
    SEGPOLY_FCV_CASE(7)
    SEGPOLY_FCV_CASE(9)
    SEGPOLY_FCV_CASE(11)
    SEGPOLY_FCV_CASE(13)
    default: break;
  }
#undef SEGPOLY_FCV_CASE
}

template <typename T, typename Index, int LAYOUT>
int fcconv_launch(const FcvArgs& a) {
  if (a.n_nodes == 0 || a.n_tiles == 0) return 0;
  const dim3 grid(static_cast<unsigned>(a.n_nodes), static_cast<unsigned>(a.n_tiles));
  hipLaunchKernelGGL((fcconv_kernel<T, Index, LAYOUT>), grid, dim3(64), a.lds_bytes,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x), static_cast<const T*>(a.sh),
                     static_cast<const T*>(a.w), static_cast<const Index*>(a.src), static_cast<const Index*>(a.dst),
                     a.n_src, a.n_edges, a.dim1, a.dim2, a.dimo, a.w_stride, a.mean, static_cast<T*>(a.out),
                     a.blocks, a.qks, a.ents, a.tiles, a.qs, a.chunks, a.uts, a.n_ut, a.n_blocks, a.ncomp, a.max_nqk,
                     a.lane_bits);
  return static_cast<int>(hipGetLastError());
}

template <typename T>
int fcconv_dispatch(const FcvArgs& a) {
  if (a.idx == kI64)
    return a.layout == kMulIr ? fcconv_launch<T, int64_t, kMulIr>(a) : fcconv_launch<T, int64_t, kIrMul>(a);
  return a.layout == kMulIr ? fcconv_launch<T, int32_t, kMulIr>(a) : fcconv_launch<T, int32_t, kIrMul>(a);
}

}  // namespace kern

int launch_fcconv(const FcvArgs& a) {
  return a.dtype == kF32 ? kern::fcconv_dispatch<float>(a) : kern::fcconv_dispatch<double>(a);
}

}  // namespace segpoly
