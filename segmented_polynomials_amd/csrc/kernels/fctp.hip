// Fully connected ("uvw") tensor product on the matrix cores (gfx950 MFMA).
//
// cuequivariance-torch skill document, "CPU tensor product and backward"
// (FullyConnectedTensorProduct with weights and gradients of both inputs)
// and e3nn-course Lesson 12a, exercise 1 (every input-1 channel u couples
// with every input-2 channel v into every output channel w, so a path holds
// mul1 * mul2 * mul3 weights).  For an output block o:
//   out[n, o, k, w] = sum over paths (i, j, o) of
//                     sum_(u, v) W_p[u, v, w] A_p[n, k, (u, v)],
//   A_p[n, k, (u, v)] = alpha_o sum_(a, b) C_p[a, b, k] x1[n, i, a, u] x2[n, j, b, v]:
// per output block a GEMM with rows (n, k), K = (u, v) and columns w.  The
// A operand never exists in memory: each lane builds its MFMA operand from
// the two input blocks staged in LDS (a handful of non-zero couplings per
// row), and the weight segment is the B operand.  The input gradients are
// the same GEMM with other operands (fctp_tables.hpp): dx1 rows (n, a),
// K = (v, w), A from x2 and the output gradient; dx2 likewise.
//
// fctp_kernel: a workgroup of 4 waves owns up to 128 rows (whole samples)
// and TN columns of one result block; each wave owns two 16-row MFMA tiles
// and all TN / 16 column tiles (v_mfma_*_16x16x4).  Per term the two
// operand blocks of the tile's samples are staged in LDS once, and the
// weight segment streams through a double-buffered LDS chunk of 32 K rows.
//
// fctp_dw_kernel: the weight gradient dW_p[(u, v), w] = sum over samples and
// output components (n, k) of A_p[n, k, (u, v)] g[n, o, k, w]: rows (u, v),
// K = (k, n) in staged groups of samples, A^T built per lane from the
// staged blocks (the K step keeps one k for all four lane groups, so the
// coupling entries are wave-uniform), B = the staged output gradient.
// Partial sums per chunk of samples, folded in chunk order.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../fctp_tables.hpp"
#include "../launch.hpp"
#include "mfma.hpp"

namespace segpoly {
namespace kern {

constexpr int kFcThreads = 256;
constexpr int kFcTK = 32;  // K rows per staged weight chunk (8 MFMA steps)

__device__ __forceinline__ int fc_div(int n, const FastDiv& f) {
  return static_cast<int>((static_cast<uint64_t>(__umulhi(static_cast<uint32_t>(n), f.magic)) +
                           static_cast<uint32_t>(n)) >> f.shift);
}

// B rows of TN + 16 elements (16 for TN = 16): the four K rows one MFMA
// step reads start 16 banks apart.
template <int TN>
struct FcB {
  static constexpr int stride = TN == 16 ? 16 : TN + 16;
};

// Stage `ns` samples (rows s0 ..) of one operand block into LDS as
// [sample][component][channel + kFcPad]; samples at or past n read as zero.
template <typename T, int LAYOUT>
__device__ __forceinline__ void fc_stage(const T* __restrict__ src, int64_t sdim, int64_t boff, int bd, int bm,
                                         int64_t s0, int ns, int64_t n, T* dst, int tid) {
  const int blk = bd * bm;
  const int cstride = bm + kFcPad, sstride = bd * cstride;
  if (blk <= kFcThreads) {
    const int spp = kFcThreads / blk;  // samples per pass
    const int sp = tid / blk, rem = tid - sp * blk;
    if (sp >= spp) return;
    int a, u;
    if (LAYOUT == kIrMul) {
      a = rem / bm;
      u = rem - a * bm;
    } else {
      u = rem / bd;
      a = rem - u * bd;
    }
    const int li = a * cstride + u;
    for (int s = sp; s < ns; s += spp) {
      const int64_t row = s0 + s;
      dst[s * sstride + li] = row < n ? src[row * sdim + boff + rem] : T(0);
    }
  } else {
    for (int rem = tid; rem < blk; rem += kFcThreads) {
      int a, u;
      if (LAYOUT == kIrMul) {
        a = rem / bm;
        u = rem - a * bm;
      } else {
        u = rem / bd;
        a = rem - u * bd;
      }
      const int li = a * cstride + u;
      for (int s = 0; s < ns; ++s) {
        const int64_t row = s0 + s;
        dst[s * sstride + li] = row < n ? src[row * sdim + boff + rem] : T(0);
      }
    }
  }
}

template <typename T, int LAYOUT, int TN>
__global__ void __launch_bounds__(kFcThreads)
fctp_kernel(const T* __restrict__ op0, const T* __restrict__ op1, const T* __restrict__ op2, int64_t dim0,
            int64_t dim1, int64_t dim2, const T* __restrict__ w, T* __restrict__ res, int64_t dim_res, int64_t n,
            const FcRes* __restrict__ rtab, const FcTerm* __restrict__ terms, const FcEnt* __restrict__ ents,
            FcTiles tiles) {
  using M = Mfma<T>;
  constexpr int kNT = TN / 16;
  constexpr int kBS = FcB<TN>::stride;
  constexpr int kBPer = kFcTK * TN / kFcThreads;  // weight elements staged per thread and chunk
  static_assert(kBPer >= 1 && (kFcTK * TN) % kFcThreads == 0, "weight chunk must split over the workgroup");
  extern __shared__ __align__(16) unsigned char fc_smem[];
  __shared__ T Bs[2][kFcTK][kBS];

  const int bid = blockIdx.x;
  int r = 0;
  while (r + 1 < tiles.n_res && tiles.tile_begin[r + 1] <= bid) ++r;
  const FcRes R = rtab[r];
  const int local = bid - tiles.tile_begin[r];
  const int trow = local / R.col_tiles, tcol = local - trow * R.col_tiles;
  const int64_t s0 = static_cast<int64_t>(trow) * R.ts;
  const int ts = static_cast<int>(n - s0 < R.ts ? n - s0 : R.ts);  // samples in this tile (>= 1)
  const int d = R.d;
  const int rows = ts * d;
  const int c0 = tcol * TN;

  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const bool has0 = wave * 16 < rows, has1 = (wave + 4) * 16 < rows;  // wave-uniform
  int sl[2], kc[2];
  bool rv[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = (wave + 4 * rt) * 16 + lane % 16;
    rv[rt] = row < rows;
    sl[rt] = rv[rt] ? row / d : 0;
    kc[rt] = rv[rt] ? row - sl[rt] * d : 0;
  }

  typename M::acc_t acc[2][kNT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[rt][j] = typename M::acc_t{0, 0, 0, 0};

  T* Ps = reinterpret_cast<T*>(fc_smem);
  for (int t = R.term_begin; t < R.term_end; ++t) {
    const FcTerm Tm = terms[t];
    const int pcs = Tm.p_m + kFcPad, qcs = Tm.q_m + kFcPad;
    const int pss = Tm.p_d * pcs, qss = Tm.q_d * qcs;
    T* Qs = Ps + R.ts * pss;
    const T* P = Tm.p_op == 0 ? op0 : (Tm.p_op == 1 ? op1 : op2);
    const T* Q = Tm.q_op == 0 ? op0 : (Tm.q_op == 1 ? op1 : op2);
    const int64_t pdim = Tm.p_op == 0 ? dim0 : (Tm.p_op == 1 ? dim1 : dim2);
    const int64_t qdim = Tm.q_op == 0 ? dim0 : (Tm.q_op == 1 ? dim1 : dim2);
    const int K = Tm.p_m * Tm.q_m;

    // this lane's coupling entries: LDS offsets of the P and Q components
    // of its rows' samples, and the coefficients (zero for padding and for
    // rows past the tile)
    int pa[2][kFcMaxT], qb[2][kFcMaxT];
    T ec[2][kFcMaxT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < kFcMaxT; ++e) {
        pa[rt][e] = 0;
        qb[rt][e] = 0;
        ec[rt][e] = T(0);
        if (e < Tm.T) {
          const FcEnt E = ents[Tm.ent + kc[rt] * Tm.T + e];
          pa[rt][e] = sl[rt] * pss + E.pa * pcs;
          qb[rt][e] = sl[rt] * qss + E.qb * qcs;
          ec[rt][e] = rv[rt] ? static_cast<T>(E.c) : T(0);
        }
      }

    // weight chunk staging: element e of the chunk is (kk, cc), cc fastest
    // when the result channel is the contiguous weight index, else kk
    const bool c_fast = Tm.s_r == 1;
    T rb[kBPer];
    auto fetch = [&](int k0) {
#pragma unroll
      for (int i = 0; i < kBPer; ++i) {
        const int e = i * kFcThreads + tid;
        const int kk = c_fast ? e / TN : e % kFcTK;
        const int cc = c_fast ? e % TN : e / kFcTK;
        const int kq = k0 + kk, col = c0 + cc;
        T v = T(0);
        if (kq < K && col < R.m) {
          const int pu = fc_div(kq, Tm.q_div), qv = kq - pu * Tm.q_m;
          v = w[Tm.w_off + pu * Tm.s_p + qv * Tm.s_q + col * Tm.s_r];
        }
        rb[i] = v;
      }
    };
    auto put = [&](int buf) {
#pragma unroll
      for (int i = 0; i < kBPer; ++i) {
        const int e = i * kFcThreads + tid;
        const int kk = c_fast ? e / TN : e % kFcTK;
        const int cc = c_fast ? e % TN : e / kFcTK;
        Bs[buf][kk][cc] = rb[i];
      }
    };

    __syncthreads();  // the previous term's LDS reads are done
    fc_stage<T, LAYOUT>(P, pdim, Tm.p_off, Tm.p_d, Tm.p_m, s0, ts, n, Ps, tid);
    fc_stage<T, LAYOUT>(Q, qdim, Tm.q_off, Tm.q_d, Tm.q_m, s0, ts, n, Qs, tid);
    fetch(0);
    put(0);
    __syncthreads();

    const int nch = (K + kFcTK - 1) / kFcTK;
    for (int ch = 0; ch < nch; ++ch) {
      const int k0 = ch * kFcTK;
      if (ch + 1 < nch) fetch(k0 + kFcTK);
      const int buf = ch & 1;
#pragma unroll
      for (int s = 0; s < kFcTK / 4; ++s) {
        const int kl = 4 * s + lane / 16;
        const int kq = k0 + kl;
        const bool kv = kq < K;
        const int pu0 = fc_div(kv ? kq : 0, Tm.q_div);
        const int qv = (kv ? kq : 0) - pu0 * Tm.q_m;
        T a[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          T acc_a = T(0);
#pragma unroll
          for (int e = 0; e < kFcMaxT; ++e)
            if (e < Tm.T) acc_a += ec[rt][e] * Ps[pa[rt][e] + pu0] * Qs[qb[rt][e] + qv];
          a[rt] = kv ? acc_a : T(0);
        }
        T b[kNT];
#pragma unroll
        for (int j = 0; j < kNT; ++j) b[j] = Bs[buf][kl][j * 16 + lane % 16];
        if (has0) {
#pragma unroll
          for (int j = 0; j < kNT; ++j) acc[0][j] = M::mma(a[0], b[j], acc[0][j]);
        }
        if (has1) {
#pragma unroll
          for (int j = 0; j < kNT; ++j) acc[1][j] = M::mma(a[1], b[j], acc[1][j]);
        }
      }
      if (ch + 1 < nch) put(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: rows (sample, component), columns c0 + ..
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    if (!(rt == 0 ? has0 : has1)) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (wave + 4 * rt) * 16 + M::row(lane, q);
      if (row >= rows) continue;
      const int s = row / d, k = row - s * d;
      T* orow = res + (s0 + s) * dim_res + R.off;
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int col = c0 + j * 16 + lane % 16;
        if (col < R.m) {
          const int64_t off = LAYOUT == kIrMul ? static_cast<int64_t>(k) * R.m + col : static_cast<int64_t>(col) * d + k;
          orow[off] = acc[rt][j][q];
        }
      }
    }
  }
}

// Weight gradient partials: part[chunk][w_off + (u q_m + v) g_m + w].
template <typename T, int LAYOUT>
__global__ void __launch_bounds__(kFcThreads)
fctp_dw_kernel(const T* __restrict__ x1, const T* __restrict__ x2, const T* __restrict__ g, int64_t dim1,
               int64_t dim2, int64_t dimo, T* __restrict__ part, int64_t numel, int64_t n,
               const FcDwPath* __restrict__ paths, const FcEnt* __restrict__ ents, FcDwTiles tiles) {
  using M = Mfma<T>;
  constexpr int kRT = kFcDwRows / 64;   // 16-row MFMA tiles per wave
  constexpr int kNT = kFcDwCols / 16;
  extern __shared__ __align__(16) unsigned char fc_smem[];

  const int bid = blockIdx.x;
  int pi = 0;
  while (pi + 1 < tiles.n_paths && tiles.tile_begin[pi + 1] <= bid) ++pi;
  const FcDwPath P = paths[pi];
  int local = bid - tiles.tile_begin[pi];
  const int per_chunk = P.m_tiles * P.col_tiles;
  const int chunk = local / per_chunk;
  local -= chunk * per_chunk;
  const int mt = local / P.col_tiles, ct = local - mt * P.col_tiles;
  const int K = P.p_m * P.q_m;
  const int row0 = mt * kFcDwRows, c0 = ct * kFcDwCols;
  const int64_t n_begin = static_cast<int64_t>(chunk) * kFcDwChunk;
  const int64_t n_end = n_begin + kFcDwChunk < n ? n_begin + kFcDwChunk : n;

  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int pcs = P.p_m + kFcPad, qcs = P.q_m + kFcPad, gcs = P.g_m + kFcPad;
  const int pss = P.p_d * pcs, qss = P.q_d * qcs, gss = P.g_d * gcs;
  T* Ps = reinterpret_cast<T*>(fc_smem);
  T* Qs = Ps + P.ts * pss;
  T* Gs = Qs + P.ts * qss;

  // this lane's rows (u, v) of its kRT tiles
  int ru[kRT], rq[kRT];
  bool rok[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int row = row0 + wave * (kFcDwRows / 4) + rt * 16 + lane % 16;
    rok[rt] = row < K;
    const int rr = rok[rt] ? row : 0;
    ru[rt] = fc_div(rr, P.q_div);
    rq[rt] = rr - ru[rt] * P.q_m;
  }
  const bool wave_any = row0 + wave * (kFcDwRows / 4) < K;
  const int col = c0 + lane % 16;

  typename M::acc_t acc[kRT][kNT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[rt][j] = typename M::acc_t{0, 0, 0, 0};

  for (int64_t sb = n_begin; sb < n_end; sb += P.ts) {
    const int ns = static_cast<int>(n_end - sb < P.ts ? n_end - sb : P.ts);
    const int nsp = (ns + 3) & ~3;  // staged samples (zero rows up to a multiple of 4)
    __syncthreads();
    fc_stage<T, LAYOUT>(x1, dim1, P.p_off, P.p_d, P.p_m, sb, nsp, n_end, Ps, tid);
    fc_stage<T, LAYOUT>(x2, dim2, P.q_off, P.q_d, P.q_m, sb, nsp, n_end, Qs, tid);
    fc_stage<T, LAYOUT>(g, dimo, P.g_off, P.g_d, P.g_m, sb, nsp, n_end, Gs, tid);
    __syncthreads();
    if (!wave_any) continue;
    for (int k = 0; k < P.g_d; ++k) {
      // the entries of output component k (wave-uniform)
      int ea[kFcMaxT], eb[kFcMaxT];
      T ecf[kFcMaxT];
#pragma unroll
      for (int e = 0; e < kFcMaxT; ++e) {
        ea[e] = 0;
        eb[e] = 0;
        ecf[e] = T(0);
        if (e < P.T) {
          const FcEnt E = ents[P.ent + k * P.T + e];
          ea[e] = E.pa * pcs;
          eb[e] = E.qb * qcs;
          ecf[e] = static_cast<T>(E.c);
        }
      }
      for (int s4 = 0; s4 < nsp; s4 += 4) {
        const int s = s4 + lane / 16;
        T bv[kNT];
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          const int cj = col + j * 16;
          bv[j] = cj < P.g_m ? Gs[s * gss + k * gcs + cj] : T(0);
        }
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          T av = T(0);
#pragma unroll
          for (int e = 0; e < kFcMaxT; ++e)
            if (e < P.T) av += ecf[e] * Ps[s * pss + ea[e] + ru[rt]] * Qs[s * qss + eb[e] + rq[rt]];
          av = rok[rt] ? av : T(0);
#pragma unroll
          for (int j = 0; j < kNT; ++j) acc[rt][j] = M::mma(av, bv[j], acc[rt][j]);
        }
      }
    }
  }
  if (!wave_any) return;
  T* prow = part + static_cast<int64_t>(chunk) * numel + P.w_off;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = row0 + wave * (kFcDwRows / 4) + rt * 16 + M::row(lane, q);
      if (row >= K) continue;
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int cj = col + j * 16;
        if (cj < P.g_m) prow[static_cast<int64_t>(row) * P.g_m + cj] = acc[rt][j][q];
      }
    }
}

// dw[e] = sum over chunks c (in order) of part[c][e].
template <typename T>
__global__ void __launch_bounds__(256)
fctp_dw_fold_kernel(const T* __restrict__ part, int chunks, int64_t numel, T* __restrict__ dw) {
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < numel;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    T acc = T(0);
    for (int c = 0; c < chunks; ++c) acc += part[c * numel + e];
    dw[e] = acc;
  }
}

template <typename T, int LAYOUT, int TN>
int fctp_launch_tn(const FcArgs& a, const FcTiles& t) {
  const int total = t.tile_begin[t.n_res];
  if (total == 0) return 0;
  hipLaunchKernelGGL((fctp_kernel<T, LAYOUT, TN>), dim3(static_cast<unsigned>(total)), dim3(kFcThreads),
                     a.lds_bytes, static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.op[0]),
                     static_cast<const T*>(a.op[1]), static_cast<const T*>(a.op[2]), a.dim[0], a.dim[1], a.dim[2],
                     static_cast<const T*>(a.w), static_cast<T*>(a.res), a.dim_res, a.n, a.res_tab, a.terms, a.ents,
                     t);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int LAYOUT>
int fctp_launch(const FcArgs& a, const FcTiles& t) {
  if (a.tn == 16) return fctp_launch_tn<T, LAYOUT, 16>(a, t);
  if (a.tn == 32) return fctp_launch_tn<T, LAYOUT, 32>(a, t);
  return fctp_launch_tn<T, LAYOUT, 64>(a, t);
}

template <typename T, int LAYOUT>
int fctp_dw_launch(const FcDwArgs& a, const FcDwTiles& t) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int total = t.tile_begin[t.n_paths];
  if (total > 0)
    hipLaunchKernelGGL((fctp_dw_kernel<T, LAYOUT>), dim3(static_cast<unsigned>(total)), dim3(kFcThreads),
                       a.lds_bytes, st, static_cast<const T*>(a.x1), static_cast<const T*>(a.x2),
                       static_cast<const T*>(a.g), a.dim1, a.dim2, a.dimo, static_cast<T*>(a.part), a.numel, a.n,
                       a.paths, a.ents, t);
  int rc = static_cast<int>(hipGetLastError());
  if (rc || a.numel == 0) return rc;
  const int64_t blocks = (a.numel + 255) / 256;
  hipLaunchKernelGGL((fctp_dw_fold_kernel<T>), dim3(static_cast<unsigned>(blocks < 2048 ? blocks : 2048)),
                     dim3(256), 0, st, static_cast<const T*>(a.part), t.chunks, a.numel, static_cast<T*>(a.dw));
  return static_cast<int>(hipGetLastError());
}

}  // namespace kern

int launch_fctp(const FcArgs& a, const FcTiles& t) {
  using namespace kern;
  if (a.dtype == kF32)
    return a.layout == kMulIr ? fctp_launch<float, kMulIr>(a, t) : fctp_launch<float, kIrMul>(a, t);
  return a.layout == kMulIr ? fctp_launch<double, kMulIr>(a, t) : fctp_launch<double, kIrMul>(a, t);
}

int launch_fctp_dw(const FcDwArgs& a, const FcDwTiles& t) {
  using namespace kern;
  if (a.dtype == kF32)
    return a.layout == kMulIr ? fctp_dw_launch<float, kMulIr>(a, t) : fctp_dw_launch<float, kIrMul>(a, t);
  return a.layout == kMulIr ? fctp_dw_launch<double, kMulIr>(a, t) : fctp_dw_launch<double, kIrMul>(a, t);
}

}  // namespace segpoly
