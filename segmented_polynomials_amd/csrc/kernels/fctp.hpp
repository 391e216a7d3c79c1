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
// and all TN / 16 column tiles (v_mfma_*_16x16x4).  Per term the operand
// block with fewer channels (P) of the tile's samples is staged in LDS; the
// one with more channels (Q) is held in registers a window of channels at a
// time (fc_term), and the weight segment streams through a double-buffered
// LDS chunk.
//
// fctp_dw_kernel: the weight gradient dW_p[(u, v), w] = sum over samples and
// output components (n, k) of A_p[n, k, (u, v)] g[n, o, k, w]: rows (u, v),
// K = (k, n) in staged groups of samples, A^T built per lane from the
// staged blocks (the K step keeps one k for all four lane groups, so the
// coupling entries are wave-uniform), B = the staged output gradient.
// Partial sums per chunk of samples, folded in chunk order.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../fctp_tables.hpp"
#include "../launch.hpp"
#include "mfma.hpp"

namespace segpoly {
namespace kern {

constexpr int kFcThreads = 256;
// s_waitcnt immediate that waits for every outstanding vector memory load
// (vmcnt 0) and leaves the export and LDS counters alone (gfx9 encoding).
constexpr unsigned kWaitVmcnt0 = 0x0F70;
constexpr int kFcTK = 32;  // K rows per staged weight chunk (8 MFMA steps)

// B rows of TN + 16 elements: the four K rows one MFMA
// step reads start 16 banks apart.
template <int TN>
struct FcB {
  static constexpr int stride = TN + 16;
};

// Stage `ns` samples (rows s0 ..) of one operand block into LDS as
// [sample (fc_sample_stride)][component][channel + kFcPad]; samples at or
// past n read as zero.  Row s0 must be < n.  Each thread issues its loads
// in batches of BATCH before writing any of them (a load followed by its
// own select and LDS write keeps one load in flight), with out-of-range
// rows reading row s0 and zeroed at the write.  The product kernel stages
// with batches of 8; the weight-gradient kernel, which relies on many
// small workgroups per CU to hide its staging, with 1 (more registers
// would cost it workgroups).
template <typename T, int LAYOUT, int BATCH>
__device__ __forceinline__ void fc_stage(const T* __restrict__ src, int64_t sdim, int64_t boff, int bd, int bm,
                                         int64_t s0, int ns, int64_t n, T* dst, int tid) {
  const int blk = bd * bm;
  const int cstride = bm + kFcPad, sstride = fc_sample_stride(bd, bm);
  // samples s0 + s for s = sfirst, sfirst + sstep, ... < ns of element rem
  auto column = [&](int rem, int sfirst, int sstep) {
    int a, u;
    if (LAYOUT == kIrMul) {
      a = rem / bm;
      u = rem - a * bm;
    } else {
      u = rem / bd;
      a = rem - u * bd;
    }
    const int li = a * cstride + u;
    const T* col = src + boff + rem;
    for (int s = sfirst; s < ns; s += sstep * BATCH) {
      T v[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const int64_t row = s0 + s + k * sstep;
        v[k] = col[(row < n ? row : s0) * sdim];
      }
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const int sk = s + k * sstep;
        if (sk < ns) dst[sk * sstride + li] = s0 + sk < n ? v[k] : T(0);
      }
    }
  };
  if (blk <= kFcThreads) {
    const int spp = kFcThreads / blk;  // samples per pass
    const int sp = tid / blk;
    if (sp < spp) column(tid - sp * blk, sp, spp);
  } else {
    for (int rem = tid; rem < blk; rem += kFcThreads) column(rem, 0, 1);
  }
}

// One term of a result tile: K runs over chunks (vc, u) -- vc outer, a
// window of VK = 4 VS channels v of the register operand Q, u one channel
// of the scalar operand P.  Per lane and row tile the window's Q values
// (Qreg[t][s] = Q[sample, qb_t, v0 + 4 s + lane / 16], read from global
// memory, where the tile's rows are L2-resident) stay in registers while u
// runs, so one MFMA step costs NT FMAs: A = sum_t y_t Qreg[t][s] with
// y_t = coef_t P[sample, pa_t, u] formed once per chunk from the P block
// staged in LDS.  The weight rows of the next chunk are fetched into
// registers while the current chunk multiplies, then written to the other
// LDS buffer.
template <typename T, int LAYOUT, int TN, int NT, bool DMA>
__device__ __forceinline__ void fc_term(const FcTerm& Tm, const FcEnt* __restrict__ ents, const T* __restrict__ w,
                                        const T* Ps, const T* __restrict__ Qt, int64_t qdim,
                                        T (*B0)[FcB<TN>::stride], T (*B1)[FcB<TN>::stride], int m_res, int c0,
                                        const int (&sl)[kFcRT],
                                        const int (&kc)[kFcRT], const bool (&rv)[kFcRT], int nrt, int tid,
                                        int lane, typename Mfma<T>::acc_t (&acc)[kFcRT][TN / 16]) {
  using M = Mfma<T>;
  constexpr int kNT = TN / 16;
  constexpr int VS = NT <= 4 ? 8 : 4;       // MFMA steps per chunk
  constexpr int VK = 4 * VS;                // K rows per chunk
  constexpr int kBPer = VK * TN / kFcThreads;
  static_assert(kBPer >= 1 && (VK * TN) % kFcThreads == 0, "weight chunk must split over the workgroup");
  const int pcs = Tm.p_m + kFcPad;
  const int pss = fc_sample_stride(Tm.p_d, Tm.p_m);
  // Q element (row, component b, channel v) at Qt + qo + v * qvs
  const int qvs = LAYOUT == kIrMul ? 1 : Tm.q_d;

  // entries of this lane's rows: P offset in LDS (without the channel) and
  // coefficient (zero for padding and rows past the tile)
  // (all entries read before any is used, and padding entries read the
  // row's first entry and are zeroed, so the reads are not serialised)
  int po[kFcRT][NT];
  int64_t qo[kFcRT][NT];  // Q offset of the entry's component, without the channel
  T cf[kFcRT][NT];
  FcEnt E[kFcRT][NT];
#pragma unroll
  for (int rt = 0; rt < kFcRT; ++rt)
#pragma unroll
    for (int e = 0; e < NT; ++e) E[rt][e] = ents[Tm.ent + kc[rt] * Tm.T + (e < Tm.T ? e : 0)];
#pragma unroll
  for (int rt = 0; rt < kFcRT; ++rt)
#pragma unroll
    for (int e = 0; e < NT; ++e) {
      const bool on = e < Tm.T;
      po[rt][e] = on ? sl[rt] * pss + E[rt][e].pa * pcs : 0;
      cf[rt][e] = on && rv[rt] ? static_cast<T>(E[rt][e].c) : T(0);
      const int qb = on ? E[rt][e].qb : 0;
      qo[rt][e] = sl[rt] * qdim + Tm.q_off + (LAYOUT == kIrMul ? qb * Tm.q_m : qb);
    }

  // the Q window: every load issued before any is zeroed (channels past q_m
  // read channel 0)
  T qreg[kFcRT][NT][VS];
  auto load_q = [&](int vc, int win) {
#pragma unroll
    for (int rt = 0; rt < kFcRT; ++rt)
#pragma unroll
      for (int e = 0; e < NT; ++e)
#pragma unroll
        for (int s = 0; s < VS; ++s) {
          const int v = vc * win + 4 * s + lane / 16;
          qreg[rt][e][s] = Qt[qo[rt][e] + static_cast<int64_t>(4 * s < win && v < Tm.q_m ? v : 0) * qvs];
        }
#pragma unroll
    for (int rt = 0; rt < kFcRT; ++rt)
#pragma unroll
      for (int e = 0; e < NT; ++e)
#pragma unroll
        for (int s = 0; s < VS; ++s) {
          const int v = vc * win + 4 * s + lane / 16;
          if (!(4 * s < win && v < Tm.q_m)) qreg[rt][e][s] = T(0);
        }
  };

  // window of the Q channels: VK, or q_m rounded up to 4 if smaller
  const int win = Tm.q_m + 3 < VK ? ((Tm.q_m + 3) & ~3) : VK;
  const int steps = win / 4;
  const int nvc = (Tm.q_m + win - 1) / win;
  const int nch = nvc * Tm.p_m;
  if (nch == 0) return;

  // weight chunk staging: element i of this thread is (kk, cc), cc fastest
  // when the result channel is the contiguous weight index, else kk; its
  // offset without the chunk's (u, vc) part is fixed for the term
  const bool c_fast = Tm.s_r == 1;
  auto kk_of = [&](int i) {
    const int e = i * kFcThreads + tid;
    return c_fast ? e / TN : e % VK;
  };
  auto cc_of = [&](int i) {
    const int e = i * kFcThreads + tid;
    return c_fast ? e % TN : e / VK;
  };
  int64_t wb[kBPer];
#pragma unroll
  for (int i = 0; i < kBPer; ++i)
    wb[i] = (kk_of(i) < win && c0 + cc_of(i) < m_res) ? Tm.w_off + kk_of(i) * Tm.s_q + (c0 + cc_of(i)) * Tm.s_r
                                                       : int64_t(-1);
  T rb[kBPer];
  // Branch-free: an element outside the window loads the segment's first
  // weight (a guarded load would split the chunk loop into branches), and
  // put() zeroes it; the select sits at put() so that nothing waits for the
  // prefetch before the steps have run.
  auto fetch = [&](int u, int vc) {
    const int64_t off = u * Tm.s_p + static_cast<int64_t>(vc) * win * Tm.s_q;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const bool ok = wb[i] >= 0 && vc * win + kk_of(i) < Tm.q_m;
      rb[i] = w[ok ? wb[i] + off : Tm.w_off];
    }
  };
  auto put = [&](int buf, int vc) {
    T (*B)[FcB<TN>::stride] = buf ? B1 : B0;
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const bool ok = wb[i] >= 0 && vc * win + kk_of(i) < Tm.q_m;
      B[kk_of(i)][cc_of(i)] = ok ? rb[i] : T(0);
    }
  };

  // B values of step s from a chunk buffer with rows of `rs` elements
  auto load_b = [&](const T* base, int rs, int s, T (&b)[kNT]) {
#pragma unroll
    for (int j = 0; j < kNT; ++j) b[j] = base[(4 * s + lane / 16) * rs + j * 16 + lane % 16];
  };
  // One MFMA step for the wave's row tiles: RT = 2 (both) or 1 (the second
  // starts past the tile's rows); chosen once per chunk, so the steps run
  // as straight-line code.
  auto step = [&](auto rt_count, int s, const T (&b)[kNT], const T (&y)[kFcRT][NT]) {
    constexpr int RT = decltype(rt_count)::value;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      T t = y[rt][0] * qreg[rt][0][s];
#pragma unroll
      for (int e = 1; e < NT; ++e) t += y[rt][e] * qreg[rt][e][s];
#pragma unroll
      for (int j = 0; j < kNT; ++j) acc[rt][j] = M::mma(t, b[j], acc[rt][j]);
    }
  };
  auto chunk = [&](auto rt_count, const T* base, int rs, const T (&y)[kFcRT][NT]) {
    if (steps == VS) {
      // the whole chunk's B values first: one LDS wait per chunk
      T b[VS][kNT];
#pragma unroll
      for (int s = 0; s < VS; ++s) load_b(base, rs, s, b[s]);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the steps
#pragma unroll
      for (int s = 0; s < VS; ++s) step(rt_count, s, b[s], y);
    } else {
      for (int s = 0; s < steps; ++s) {
        T b[kNT];
        load_b(base, rs, s, b);
        step(rt_count, s, b, y);
      }
    }
  };
  auto chunk_rows = [&](const T* base, int rs, int u) {
    T y[kFcRT][NT];
#pragma unroll
    for (int rt = 0; rt < kFcRT; ++rt)
#pragma unroll
      for (int e = 0; e < NT; ++e) y[rt][e] = cf[rt][e] * Ps[po[rt][e] + u];
    if (kFcRT == 2 && nrt == 2)
      chunk(std::integral_constant<int, kFcRT>{}, base, rs, y);
    else if (nrt >= 1)
      chunk(std::integral_constant<int, 1>{}, base, rs, y);
  };

  // DMA: LDS-direct weight chunks (the host launches this form only for
  // float, 32 columns, the result channel the contiguous weight index, full
  // windows and column tiles, 16-byte aligned rows): wave k copies rows
  // 8k .. 8k + 7 of the next chunk with one 16-byte-per-lane load straight
  // into LDS (rows of 32, no registers, no LDS write), into the buffer the
  // current chunk does not read; the two buffers are separate arrays, so
  // the reads of one never wait for the copy into the other.  Each wave
  // waits for its own copy before the chunk's barrier.
  if constexpr (DMA) {
    static_assert(sizeof(T) == 4 && TN == 32 && VK == 32, "LDS-direct chunks are float rows of 32");
    {
      const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
      T* D0 = &B0[0][0];
      T* D1 = &B1[0][0];
      auto copy = [&](T* dst, int c) {
        const int vc = c / Tm.p_m, u = c - vc * Tm.p_m;
        const int kk = 8 * wv + lane / 8, cc = 4 * (lane % 8);
        const T* gp = w + Tm.w_off + static_cast<int64_t>(u) * Tm.s_p +
                      static_cast<int64_t>(vc * win + kk) * Tm.s_q + c0 + cc;
        // (address-space casts: global source, LDS destination)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(gp),
                                         (__attribute__((address_space(3))) void*)(dst + 8 * wv * TN), 16, 0, 0);
      };
      auto body = [&](int c, const T* cur, T* nxt) {
        const int vc = c / Tm.p_m, u = c - vc * Tm.p_m;
        if (c + 1 < nch) copy(nxt, c + 1);
        chunk_rows(cur, TN, u);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (c + 1 < nch && (c + 1) / Tm.p_m != vc) {
          load_q((c + 1) / Tm.p_m, win);
          __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        }
      };
      copy(D0, 0);
      load_q(0, win);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      for (int c = 0; c < nch; c += 2) {
        body(c, D0, D1);
        if (c + 1 < nch) body(c + 1, D1, D0);
      }
      return;
    }
  }

  // Windows outer, P channels inner.  The Q window's loads are waited for
  // explicitly before the channel loop, so the loop's only outstanding
  // global loads are the weight prefetch, which the steps never wait for.
  fetch(0, 0);
  put(0, 0);
  int ch = 0;
  for (int vc = 0; vc < nvc; ++vc) {
    load_q(vc, win);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int u = 0; u < Tm.p_m; ++u, ++ch) {
      const bool more = ch + 1 < nch;
      if (more) {
        if (u + 1 < Tm.p_m)
          fetch(u + 1, vc);
        else
          fetch(0, vc + 1);
      }
      __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the steps
      const int buf = ch & 1;
      chunk_rows(&(buf ? B1 : B0)[0][0], FcB<TN>::stride, u);
      if (more) put(buf ^ 1, u + 1 < Tm.p_m ? vc : vc + 1);
      __syncthreads();
    }
  }
}

// Workgroups per CU the register allocation must allow: four for the
// float kernels with 32 columns and up to three couplings (the kernel is
// latency-bound, and four workgroups beat three even where the
// three-coupling class spills a few registers: 0.78 -> 0.74 ms on the
// 100k-sample product), otherwise what the allocation gives.
template <typename T, int TN, int NT>
constexpr int fc_min_blocks() {
  return (sizeof(T) == 4 && TN == 32 && NT <= 3) ? 4 : 1;
}

template <typename T, int LAYOUT, int TN, int NT, bool DMA>
__global__ void __launch_bounds__(kFcThreads, (fc_min_blocks<T, TN, NT>()))
fctp_kernel(const T* __restrict__ op0, const T* __restrict__ op1, const T* __restrict__ op2, int64_t dim0,
            int64_t dim1, int64_t dim2, const T* __restrict__ w, T* __restrict__ res, int64_t dim_res, int64_t n,
            const FcRes* __restrict__ rtab, const FcTerm* __restrict__ terms, const FcEnt* __restrict__ ents,
            FcTiles tiles) {
  using M = Mfma<T>;
  constexpr int kNT = TN / 16;
  extern __shared__ __align__(16) unsigned char fc_smem[];
  __shared__ T Bs0[kFcTK][FcB<TN>::stride];
  __shared__ T Bs1[kFcTK][FcB<TN>::stride];

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
  // row tiles of this wave that hold rows (wave-uniform; readfirstlane
  // tells the compiler so: scalar branches)
  int nrt = 0;
#pragma unroll
  for (int rt = 0; rt < kFcRT; ++rt) nrt += (wave + 4 * rt) * 16 < rows ? 1 : 0;
  nrt = __builtin_amdgcn_readfirstlane(nrt);
  int sl[kFcRT], kc[kFcRT];
  bool rv[kFcRT];
#pragma unroll
  for (int rt = 0; rt < kFcRT; ++rt) {
    const int row = (wave + 4 * rt) * 16 + lane % 16;
    rv[rt] = row < rows;
    sl[rt] = rv[rt] ? row / d : 0;
    kc[rt] = rv[rt] ? row - sl[rt] * d : 0;
  }

  typename M::acc_t acc[kFcRT][kNT];
#pragma unroll
  for (int rt = 0; rt < kFcRT; ++rt)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[rt][j] = typename M::acc_t{0, 0, 0, 0};

  T* Ps = reinterpret_cast<T*>(fc_smem);
  for (int t = R.term_begin; t < R.term_end; ++t) {
    const FcTerm Tm = terms[t];
    const T* P = Tm.p_op == 0 ? op0 : (Tm.p_op == 1 ? op1 : op2);
    const T* Q = Tm.q_op == 0 ? op0 : (Tm.q_op == 1 ? op1 : op2);
    const int64_t pdim = Tm.p_op == 0 ? dim0 : (Tm.p_op == 1 ? dim1 : dim2);
    const int64_t qdim = Tm.q_op == 0 ? dim0 : (Tm.q_op == 1 ? dim1 : dim2);
    __syncthreads();  // the previous term's LDS reads are done
    fc_stage<T, LAYOUT, 8>(P, pdim, Tm.p_off, Tm.p_d, Tm.p_m, s0, ts, n, Ps, tid);
    // (fc_term's first barrier publishes the staged block)
    fc_term<T, LAYOUT, TN, NT, DMA>(Tm, ents, w, Ps, Q + s0 * qdim, qdim, Bs0, Bs1, R.m, c0, sl, kc, rv, nrt, tid,
                               lane, acc);
  }

  // epilogue: rows (sample, component), columns c0 + ..
#pragma unroll
  for (int rt = 0; rt < kFcRT; ++rt) {
    if (rt >= nrt) continue;
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

// Weight-gradient partials of one tile: part[chunk][w_off + p s_p + q s_q + w].
// The wave's rows are 2 channels p (u0, u0 + 1) x 32 channels q; a lane
// owns q = v0 + lane % 16 and v0 + 16 + lane % 16, so its four row tiles
// need 2 NT values of P and 2 NT of Q per K step (one sample, one output
// component k: the entries of k are the same for the whole wave).
template <typename T, int NT>
__device__ __forceinline__ void fc_dw_tile(const FcDwPath& P, const FcEnt* __restrict__ ents, const T* Ps,
                                           const T* Qs, const T* Gs, int nsp, int k, int u0, int v0, int col,
                                           int lane, typename Mfma<T>::acc_t (&acc)[4][kFcDwCols / 16]) {
  using M = Mfma<T>;
  constexpr int kNT = kFcDwCols / 16;
  const int pcs = P.p_m + kFcPad, qcs = P.q_m + kFcPad, gcs = P.g_m + kFcPad;
  const int pss = fc_sample_stride(P.p_d, P.p_m), qss = fc_sample_stride(P.q_d, P.q_m),
            gss = fc_sample_stride(P.g_d, P.g_m);
  int pa[NT], qb[NT];
  T cf[NT];
#pragma unroll
  for (int e = 0; e < NT; ++e) {
    pa[e] = 0;
    qb[e] = 0;
    cf[e] = T(0);
    if (e < P.T) {
      const FcEnt E = ents[P.ent + k * P.T + e];
      pa[e] = E.pa * pcs;
      qb[e] = E.qb * qcs;
      cf[e] = static_cast<T>(E.c);
    }
  }
  // This lane's channels, clamped into the staged rows.  A channel p or q
  // past the block only feeds rows of the result, and a column w past it
  // only columns, that are never written, so the values need no zeroing.
  int pu[2], qv[2], gc[kNT];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    pu[i] = u0 + i < P.p_m ? u0 + i : 0;
    qv[i] = v0 + 16 * i + lane % 16 < P.q_m ? v0 + 16 * i + lane % 16 : 0;
  }
#pragma unroll
  for (int j = 0; j < kNT; ++j) gc[j] = k * gcs + (col + 16 * j < P.g_m ? col + 16 * j : 0);
  for (int s4 = 0; s4 < nsp; s4 += 4) {
    const int s = s4 + lane / 16;
    T y[2][NT], z[2][NT];
#pragma unroll
    for (int e = 0; e < NT; ++e) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        y[i][e] = cf[e] * Ps[s * pss + pa[e] + pu[i]];
        z[i][e] = Qs[s * qss + qb[e] + qv[i]];
      }
    }
    T b[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) b[j] = Gs[s * gss + gc[j]];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        T a = y[i][0] * z[h][0];
#pragma unroll
        for (int e = 1; e < NT; ++e) a += y[i][e] * z[h][e];
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[2 * i + h][j] = M::mma(a, b[j], acc[2 * i + h][j]);
      }
  }
}

// Weight-gradient staging straight into LDS (float): a lane's slots of
// one staged sample of a block are r = 64 j + lane (j < kFcDwDmaJ), at
// component r / (m + kFcPad) and channel r % (m + kFcPad); off[j] is the
// element's offset in the block, 0 for pad slots (which are never read)
// and -1 past the sample's stride (the lane copies nothing).
template <int LAYOUT>
__device__ __forceinline__ void fc_dw_dma_lanes(int bd, int bm, int lane, int (&off)[kFcDwDmaJ]) {
  const int cstride = bm + kFcPad, sstride = fc_sample_stride(bd, bm);
#pragma unroll
  for (int j = 0; j < kFcDwDmaJ; ++j) {
    const int r = 64 * j + lane;
    const int a = r / cstride, u = r - a * cstride;
    const int e = LAYOUT == kIrMul ? a * bm + u : u * bd + a;
    off[j] = r >= sstride ? -1 : (a < bd && u < bm ? e : 0);
  }
}

// Copy samples sb + s (s = wave, wave + 4, ... < nsp) of one block to
// dst + s sstride with one dword global_load_lds per slot group; samples
// at or past the chunk end are written as zeros.
__device__ __forceinline__ void fc_dw_dma_issue(const float* __restrict__ src, int64_t sdim, int64_t boff,
                                                int sstride, const int (&off)[kFcDwDmaJ], int64_t sb, int nsp,
                                                int64_t n_end, float* dst, int wave, int lane) {
  for (int s = wave; s < nsp; s += 4) {
    float* d = dst + s * sstride;
    if (sb + s < n_end) {
      const float* g = src + (sb + s) * sdim + boff;
#pragma unroll
      for (int j = 0; j < kFcDwDmaJ; ++j)
        if (off[j] >= 0)
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g + off[j]),
                                           (__attribute__((address_space(3))) void*)(d + 64 * j), 4, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < kFcDwDmaJ; ++j)
        if (off[j] >= 0) d[64 * j + lane] = 0.0f;
    }
  }
}

// Five weight-gradient workgroups per CU for the float kernels of up to
// three couplings per component that stage through registers (they hide
// each other's staging loads; four couplings would spill); four for those
// that stage straight into LDS, so that nothing spills (a scratch reload
// waits for every outstanding load, the copies of the next group too).
template <typename T, int NT, bool DMA>
constexpr int fc_dw_min_blocks() {
  return (sizeof(T) == 4 && NT <= 3) ? (DMA ? 4 : 5) : 1;
}

template <typename T, int LAYOUT, int NT, bool DMA>
__global__ void __launch_bounds__(kFcThreads, (fc_dw_min_blocks<T, NT, DMA>()))
fctp_dw_kernel(const T* __restrict__ x1, const T* __restrict__ x2, const T* __restrict__ g, int64_t dim1,
               int64_t dim2, int64_t dimo, T* __restrict__ part, int64_t numel, int64_t n,
               const FcDwPath* __restrict__ paths, const FcEnt* __restrict__ ents, FcDwTiles tiles) {
  using M = Mfma<T>;
  constexpr int kNT = kFcDwCols / 16;
  extern __shared__ __align__(16) unsigned char fc_smem[];

  const int bid = blockIdx.x;
  int pi = 0;
  while (pi + 1 < tiles.n_paths && tiles.tile_begin[pi + 1] <= bid) ++pi;
  const FcDwPath P = paths[pi];
  int local = bid - tiles.tile_begin[pi];
  const int per_chunk = P.u_tiles * P.v_tiles * P.col_tiles;
  const int chunk = local / per_chunk;
  local -= chunk * per_chunk;
  const int ut = local / (P.v_tiles * P.col_tiles);
  local -= ut * (P.v_tiles * P.col_tiles);
  const int vt = local / P.col_tiles, ct = local - vt * P.col_tiles;
  const int64_t n_begin = static_cast<int64_t>(chunk) * kFcDwChunk;
  const int64_t n_end = n_begin + kFcDwChunk < n ? n_begin + kFcDwChunk : n;

  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int u0 = ut * kFcDwU + 2 * wave, v0 = vt * kFcDwV, c0 = ct * kFcDwCols;
  const int col = c0 + lane % 16;
  T* Ps = reinterpret_cast<T*>(fc_smem);
  T* Qs = Ps + P.ts * fc_sample_stride(P.p_d, P.p_m);
  T* Gs = Qs + P.ts * fc_sample_stride(P.q_d, P.q_m);
  const T* Pg = P.p_op == 0 ? x1 : x2;
  const T* Qg = P.q_op == 0 ? x1 : x2;
  const int64_t pdim = P.p_op == 0 ? dim1 : dim2, qdim = P.q_op == 0 ? dim1 : dim2;
  const bool wave_any = u0 < P.p_m;  // wave-uniform

  typename M::acc_t acc[4][kNT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[r][j] = typename M::acc_t{0, 0, 0, 0};

  if constexpr (DMA) {
    // Double-buffered: the next group of samples is copied into the other
    // static buffer while this one multiplies (two distinct LDS objects, so
    // reads of one never wait for copies into the other).
    __shared__ __align__(16) float Sb0[kFcDwDmaElems];
    __shared__ __align__(16) float Sb1[kFcDwDmaElems];
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int pss = fc_sample_stride(P.p_d, P.p_m), qss = fc_sample_stride(P.q_d, P.q_m),
              gss = fc_sample_stride(P.g_d, P.g_m);
    const int qbase = P.ts * pss, gbase = qbase + P.ts * qss;
    int offp[kFcDwDmaJ], offq[kFcDwDmaJ], offg[kFcDwDmaJ];
    fc_dw_dma_lanes<LAYOUT>(P.p_d, P.p_m, lane, offp);
    fc_dw_dma_lanes<LAYOUT>(P.q_d, P.q_m, lane, offq);
    fc_dw_dma_lanes<LAYOUT>(P.g_d, P.g_m, lane, offg);
    auto group = [&](int64_t sb) {
      const int ns = static_cast<int>(n_end - sb < P.ts ? n_end - sb : P.ts);
      return (ns + 3) & ~3;  // staged samples (zero rows up to a multiple of 4)
    };
    auto issue = [&](int64_t sb, float* buf) {
      const int nsp = group(sb);
      fc_dw_dma_issue(Pg, pdim, P.p_off, pss, offp, sb, nsp, n_end, buf, wv, lane);
      fc_dw_dma_issue(Qg, qdim, P.q_off, qss, offq, sb, nsp, n_end, buf + qbase, wv, lane);
      fc_dw_dma_issue(g, dimo, P.g_off, gss, offg, sb, nsp, n_end, buf + gbase, wv, lane);
    };
    auto step = [&](int64_t sb, const float* cur, float* nxt) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();  // cur has landed; nxt is no longer read
      if (sb + P.ts < n_end) issue(sb + P.ts, nxt);
      if (wave_any) {
        const int nsp = group(sb);
        for (int k = 0; k < P.g_d; ++k)
          fc_dw_tile<T, NT>(P, ents, cur, cur + qbase, cur + gbase, nsp, k, u0, v0, col, lane, acc);
      }
    };
    issue(n_begin, Sb0);
    for (int64_t sb = n_begin; sb < n_end; sb += 2 * P.ts) {
      step(sb, Sb0, Sb1);
      if (sb + P.ts < n_end) step(sb + P.ts, Sb1, Sb0);
    }
  } else {
  for (int64_t sb = n_begin; sb < n_end; sb += P.ts) {
    const int ns = static_cast<int>(n_end - sb < P.ts ? n_end - sb : P.ts);
    const int nsp = (ns + 3) & ~3;  // staged samples (zero rows up to a multiple of 4)
    __syncthreads();
    fc_stage<T, LAYOUT, 1>(Pg, pdim, P.p_off, P.p_d, P.p_m, sb, nsp, n_end, Ps, tid);
    fc_stage<T, LAYOUT, 1>(Qg, qdim, P.q_off, P.q_d, P.q_m, sb, nsp, n_end, Qs, tid);
    fc_stage<T, LAYOUT, 1>(g, dimo, P.g_off, P.g_d, P.g_m, sb, nsp, n_end, Gs, tid);
    __syncthreads();
    if (!wave_any) continue;
    for (int k = 0; k < P.g_d; ++k) {
      fc_dw_tile<T, NT>(P, ents, Ps, Qs, Gs, nsp, k, u0, v0, col, lane, acc);
    }
  }
  }
  if (!wave_any) return;
  // accumulator j of row tile (i, h): rows = the 16 q of half h for channel
  // p = u0 + i (M::row gives the q within the half), column col + 16 j
  T* prow = part + static_cast<int64_t>(chunk) * numel + P.w_off;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (u0 + i >= P.p_m) continue;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qq = v0 + 16 * h + M::row(lane, q);
        if (qq >= P.q_m) continue;
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
          const int cj = col + 16 * j;
          if (cj < P.g_m) prow[(u0 + i) * P.s_p + qq * P.s_q + cj] = acc[2 * i + h][j][q];
        }
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

// W[u][v][w] -> W1[v][w][u], W2[u][w][v] per path segment (one thread per
// weight; the segment of weight i is the last path whose offset is <= i).
template <typename T>
__global__ void __launch_bounds__(256)
fctp_transpose_kernel(const T* __restrict__ w, T* __restrict__ w1, T* __restrict__ w2,
                      const FcTrPath* __restrict__ paths, int n_paths, int64_t numel) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < numel;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    int lo = 0, hi = n_paths - 1;
    while (lo < hi) {  // last path with w_off <= i
      const int mid = (lo + hi + 1) / 2;
      if (paths[mid].w_off <= i)
        lo = mid;
      else
        hi = mid - 1;
    }
    const FcTrPath P = paths[lo];
    const int64_t r = i - P.w_off;
    const int64_t c = r % P.m3, t = r / P.m3;
    const int64_t v = t % P.m2, u = t / P.m2;
    const T x = w[i];
    w1[P.w_off + (v * P.m3 + c) * P.m1 + u] = x;
    w2[P.w_off + (u * P.m3 + c) * P.m2 + v] = x;
  }
}

template <typename T>
int fctp_transpose_launch(const FcTrArgs& a) {
  if (a.numel == 0 || a.n_paths == 0) return 0;
  const int64_t blocks = (a.numel + 255) / 256;
  hipLaunchKernelGGL((fctp_transpose_kernel<T>), dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.w),
                     static_cast<T*>(a.w1), static_cast<T*>(a.w2), a.paths, a.n_paths, a.numel);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int LAYOUT, int TN, int NT, bool DMA = false>
int fctp_launch_k(const FcArgs& a, const FcTiles& t) {
  const int total = t.tile_begin[t.n_res];
  if (total == 0) return 0;
  hipLaunchKernelGGL((fctp_kernel<T, LAYOUT, TN, NT, DMA>), dim3(static_cast<unsigned>(total)), dim3(kFcThreads),
                     a.lds_bytes, static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.op[0]),
                     static_cast<const T*>(a.op[1]), static_cast<const T*>(a.op[2]), a.dim[0], a.dim[1], a.dim[2],
                     static_cast<const T*>(a.w), static_cast<T*>(a.res), a.dim_res, a.n, a.res_tab, a.terms, a.ents,
                     t);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int LAYOUT, int TN>
int fctp_launch_tn(const FcArgs& a, const FcTiles& t) {
  if constexpr (sizeof(T) == 4 && TN == 32) {
    if (a.lds_direct) {  // (the host checked the pass's terms and the weight alignment)
      switch (a.nt) {
        case 1: return fctp_launch_k<T, LAYOUT, TN, 1, true>(a, t);
        case 2: return fctp_launch_k<T, LAYOUT, TN, 2, true>(a, t);
        case 3: return fctp_launch_k<T, LAYOUT, TN, 3, true>(a, t);
        case 4: return fctp_launch_k<T, LAYOUT, TN, 4, true>(a, t);
        default: break;
      }
    }
  }
  switch (a.nt) {
    case 1: return fctp_launch_k<T, LAYOUT, TN, 1>(a, t);
    case 2: return fctp_launch_k<T, LAYOUT, TN, 2>(a, t);
    case 3: return fctp_launch_k<T, LAYOUT, TN, 3>(a, t);
    case 4: return fctp_launch_k<T, LAYOUT, TN, 4>(a, t);
    case 6: return fctp_launch_k<T, LAYOUT, TN, 6>(a, t);
    case 8: return fctp_launch_k<T, LAYOUT, TN, 8>(a, t);
    default: return fctp_launch_k<T, LAYOUT, TN, 16>(a, t);
  }
}

template <typename T, int LAYOUT>
int fctp_launch(const FcArgs& a, const FcTiles& t) {
  return a.tn == 32 ? fctp_launch_tn<T, LAYOUT, 32>(a, t) : fctp_launch_tn<T, LAYOUT, 64>(a, t);
}

template <typename T, int LAYOUT, int NT, bool DMA>
int fctp_dw_launch_d(const FcDwArgs& a, const FcDwTiles& t) {
  const int total = t.tile_begin[t.n_paths];
  if (total == 0) return 0;
  hipLaunchKernelGGL((fctp_dw_kernel<T, LAYOUT, NT, DMA>), dim3(static_cast<unsigned>(total)), dim3(kFcThreads),
                     a.lds_bytes, static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.x1),
                     static_cast<const T*>(a.x2), static_cast<const T*>(a.g), a.dim1, a.dim2, a.dimo,
                     static_cast<T*>(a.part), a.numel, a.n, a.paths, a.ents, t);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int LAYOUT, int NT>
int fctp_dw_launch_k(const FcDwArgs& a, const FcDwTiles& t) {
  if constexpr (std::is_same_v<T, float>) {
    if (a.dma) return fctp_dw_launch_d<T, LAYOUT, NT, true>(a, t);
  }
  return fctp_dw_launch_d<T, LAYOUT, NT, false>(a, t);
}

template <typename T, int LAYOUT>
int fctp_dw_launch(const FcDwArgs& a, const FcDwTiles& t) {
  int rc = 0;
  switch (a.nt) {
    case 1: rc = fctp_dw_launch_k<T, LAYOUT, 1>(a, t); break;
    case 2: rc = fctp_dw_launch_k<T, LAYOUT, 2>(a, t); break;
    case 3: rc = fctp_dw_launch_k<T, LAYOUT, 3>(a, t); break;
    case 4: rc = fctp_dw_launch_k<T, LAYOUT, 4>(a, t); break;
    case 6: rc = fctp_dw_launch_k<T, LAYOUT, 6>(a, t); break;
    case 8: rc = fctp_dw_launch_k<T, LAYOUT, 8>(a, t); break;
    default: rc = fctp_dw_launch_k<T, LAYOUT, 16>(a, t); break;
  }
  if (rc || a.numel == 0) return rc;
  const int64_t blocks = (a.numel + 255) / 256;
  hipLaunchKernelGGL((fctp_dw_fold_kernel<T>), dim3(static_cast<unsigned>(blocks < 2048 ? blocks : 2048)),
                     dim3(256), 0, static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.part), t.chunks,
                     a.numel, static_cast<T*>(a.dw));
  return static_cast<int>(hipGetLastError());
}

}  // namespace kern
}  // namespace segpoly
