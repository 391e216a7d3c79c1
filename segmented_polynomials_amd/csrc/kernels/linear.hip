// Equivariant linear layer on the matrix cores (gfx950 MFMA).
//
// cuequivariance-torch skill document, "Linear: layout conversion and
// rotations" and "Other operations and layers" (species-indexed Linear):
// only blocks of one irrep type mix, channel by channel, with the same matrix
// for every component m.  For an output block o of type t (d = 2l + 1
// components, alpha_t = 1 / sqrt(sum of the input multiplicities of type t)):
//   out[n, o, m, v] = alpha_t * sum over input blocks i of type t of
//                     sum_u W_io[u, v] * x[n, i, m, u].
// Per output block this is a dense GEMM with rows r = (n, m) (n * d rows),
// K = the concatenated input channels of its type, columns v.  The same
// kernel computes the backward's dx = alpha G W^T (TRANSW: the weight
// segment is read transposed).
//
// Tiling: a workgroup of 4 waves owns a 128 x 128 tile of one output block's
// GEMM; the K loop stages 128 x 32 of A (rows of x) and 32 x 128 of B (the
// weight segment) in LDS; each wave computes 64 x 64 with sixteen
// v_mfma_*_16x16x4 per 4 k.  Class-indexed weights (one row of weights per
// sample picked by an index, sorted in practice): the tile runs one masked
// pass per class present among its rows (rows of other classes read as
// zero), so a tile inside one class costs one pass.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../launch.hpp"
#include "../linear_tables.hpp"
#include "bufload.hpp"
#include "mfma.hpp"

namespace segpoly {
namespace kern {

constexpr int kLinTM = kLinTileRows, kLinTN = kLinTileCols, kLinTK = 32, kLinThreads = 256;
// 4 waves as 2 x 2; each wave owns (kLinTM / 2) x (kLinTN / 2) = kMT x kNT
// MFMA tiles of 16 x 16
constexpr int kMT = kLinTM / 32, kNT = kLinTN / 32;
static_assert(kLinTM % 32 == 0 && kLinTN % 32 == 0, "tiles are multiples of two 16-wide MFMA tiles");

// LDS row padding: A rows of 36 and B rows of 144 elements keep the MFMA
// operand reads free of bank conflicts (64 banks).
constexpr int kLinPadA = 4, kLinPadB = 16;
constexpr int kARows = kLinTM * kLinTK / kLinThreads;   // A rows staged per thread
constexpr int kBElems = kLinTK * kLinTN / kLinThreads;  // B elements staged per thread

template <typename T, typename Index, int LAYOUT, bool TRANSW, bool CLASSES>
__global__ void __launch_bounds__(kLinThreads)
linear_kernel(const T* __restrict__ x, const T* __restrict__ w, const Index* __restrict__ cls,
              T* __restrict__ out, int64_t n, int64_t dim_in, int64_t dim_out, int64_t numel, int num_classes,
              LinTable tab) {
  using M = Mfma<T>;
  __shared__ T As[kLinTM][kLinTK + kLinPadA];
  // B as [k][column]; with TRANSW as [column][k]: the transposed segment is
  // read k-contiguous, and writing it k-major into [k][column] rows of 144
  // put 8 lanes of a wave on each bank
  constexpr int kBRows = TRANSW ? kLinTN : kLinTK, kBCols = TRANSW ? kLinTK + kLinPadA : kLinTN + kLinPadB;
  __shared__ T Bs[kBRows][kBCols];
  __shared__ int cls_range[kLinThreads / 64][2];

  // which output block and tile
  const int bid = blockIdx.x;
  int ob = 0;
  while (ob + 1 < tab.n_out && tab.outs[ob + 1].tile_begin <= bid) ++ob;
  const LinOut O = tab.outs[ob];
  const int tile = bid - O.tile_begin;
  const int row0 = (tile / O.col_tiles) * kLinTM;  // rows n * d < 2^31 (checked on the host)
  const int col0 = (tile % O.col_tiles) * kLinTN;
  const int d = O.d;
  const int R = static_cast<int>(n) * d;

  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = tid / 64;
  const int wr = wave / 2, wc = wave % 2;  // wave tile: rows 32 wr.., cols 64 wc..

  // the A rows this thread stages: r = e * 8 + tid / 32, channel tid % 32
  // (decomposed once: element offset from the tile's first sample s0,
  // component, class).  Offsets stay below 2^31 bytes: a tile spans at most
  // kLinTM + 1 samples and the host bounds dim_in.
  const int kk_a = tid % kLinTK;
  const int s0 = row0 / d;
  int a_rel[kARows];
  int a_m[kARows];
  bool a_ok[kARows];
  int a_cls[CLASSES ? kARows : 1];
#pragma unroll
  for (int e = 0; e < kARows; ++e) {
    const int row = row0 + e * (kLinThreads / kLinTK) + tid / kLinTK;
    a_ok[e] = row < R;
    const int nn = a_ok[e] ? row / d : s0;
    a_m[e] = a_ok[e] ? row - nn * d : 0;
    a_rel[e] = (nn - s0) * static_cast<int>(dim_in);
    if constexpr (CLASSES) {
      const int64_t c = a_ok[e] ? static_cast<int64_t>(cls[nn]) : -1;
      a_cls[e] = (c >= 0 && c < num_classes) ? static_cast<int>(c) : -1;
    }
  }
  const __amdgpu_buffer_rsrc_t x_rsrc =
      buf_rsrc(x + static_cast<int64_t>(s0) * dim_in, (n - s0) * dim_in * static_cast<int64_t>(sizeof(T)));

  typename M::acc_t acc[kMT][kNT];
#pragma unroll
  for (int a = 0; a < kMT; ++a)
#pragma unroll
    for (int b = 0; b < kNT; ++b) acc[a][b] = typename M::acc_t{0, 0, 0, 0};

  // The K loop runs over the flattened sequence (class, pair, chunk of
  // kLinTK channels); the next chunk's global loads are issued into
  // registers before the current chunk's MFMAs, so their latency hides
  // behind the matrix work.
  // Staging loads go through buffer resources: a masked element (a row past
  // the end, a channel past the block's K, a column past its N) gets an
  // offset beyond the resource and reads zero, so no load waits on a branch
  // or a select of its value.  The class mask is applied when the chunk is
  // written to LDS: the loads of a tile's first chunk then wait for no class
  // of its rows, only for the (scalar) class of its first sample.
  T ra[kARows], rb[kBElems];
  auto fetch = [&](int c, int p, int k0) {
    const LinPair P = tab.pairs[p];
    const __amdgpu_buffer_rsrc_t w_rsrc =
        buf_rsrc(CLASSES ? w + static_cast<int64_t>(c) * numel : w, numel * static_cast<int64_t>(sizeof(T)));
    const int u = k0 + kk_a;
    const bool u_in = u < P.k_ext;
    const int in_off = static_cast<int>(P.in_off), k_ext = P.k_ext;
#pragma unroll
    for (int e = 0; e < kARows; ++e) {
      const bool take = a_ok[e] && u_in;
      const int off = a_rel[e] + in_off + (LAYOUT == kIrMul ? a_m[e] * k_ext + u : u * d + a_m[e]);
      ra[e] = buf_load<T>(x_rsrc, take ? static_cast<uint32_t>(off) * sizeof(T) : kBufMasked);
    }
    const int w_off = static_cast<int>(P.w_off), n_ext = O.n_ext;
#pragma unroll
    for (int e = 0; e < kBElems; ++e) {
      const int idx = e * kLinThreads + tid;
      const int kk = TRANSW ? idx % kLinTK : idx / kLinTN;
      const int cc = TRANSW ? idx / kLinTK : idx % kLinTN;
      const int uu = k0 + kk, v = col0 + cc;
      const bool in = uu < k_ext && v < n_ext;
      const int off = w_off + (TRANSW ? v * k_ext + uu : uu * n_ext + v);
      rb[e] = buf_load<T>(w_rsrc, in ? static_cast<uint32_t>(off) * sizeof(T) : kBufMasked);
    }
  };

  // Classes: the tile makes one pass per class between the lowest (cmin)
  // and highest (cmax) class among its rows, starting with the class of its
  // first sample (`first`) when that is in range, so that the first chunk's
  // loads go out before the class range is known.
  int cmin = 0, cmax = 0, first = 0;
  int c = 0, p = O.pair_begin, k0 = 0;
  bool have = O.pair_begin < O.pair_end;
  if constexpr (CLASSES) {
    const int64_t c0 = static_cast<int64_t>(cls[s0]);
    first = (c0 >= 0 && c0 < num_classes) ? static_cast<int>(c0) : -1;
    if (have && first >= 0) fetch(first, p, k0);
    // range over the wave's rows, then over the four waves through LDS
    int lo = num_classes, hi = -1;
#pragma unroll
    for (int e = 0; e < kARows; ++e)
      if (a_cls[e] >= 0) {
        lo = a_cls[e] < lo ? a_cls[e] : lo;
        hi = a_cls[e] > hi ? a_cls[e] : hi;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
      lo = l2 < lo ? l2 : lo;
      hi = h2 > hi ? h2 : hi;
    }
    if (lane == 0) {
      cls_range[wave][0] = lo;
      cls_range[wave][1] = hi;
    }
    __syncthreads();
    cmin = num_classes;
    cmax = -1;
#pragma unroll
    for (int q = 0; q < kLinThreads / 64; ++q) {
      cmin = cls_range[q][0] < cmin ? cls_range[q][0] : cmin;
      cmax = cls_range[q][1] > cmax ? cls_range[q][1] : cmax;
    }
    cmin = __builtin_amdgcn_readfirstlane(cmin);
    cmax = __builtin_amdgcn_readfirstlane(cmax);
    if (first < 0) {
      first = cmin;
      have = have && cmin <= cmax;
      if (have) fetch(first, p, k0);
    }
    c = first;
  } else {
    if (have) fetch(c, p, k0);
  }
  // advance (c, p, k0) to the next chunk; false at the end.  After the
  // first class the passes run from cmin up, skipping `first`.
  auto next = [&](int& c, int& p, int& k0) -> bool {
    k0 += kLinTK;
    if (k0 < tab.pairs[p].k_ext) return true;
    k0 = 0;
    if (++p < O.pair_end) return true;
    p = O.pair_begin;
    if constexpr (!CLASSES) return false;
    c = c == first ? cmin : c + 1;
    if (c == first) ++c;
    return c <= cmax;
  };
  while (have) {
    __syncthreads();  // the previous chunk's operands are no longer read
#pragma unroll
    for (int e = 0; e < kARows; ++e) {
      bool keep = true;
      if constexpr (CLASSES) keep = a_cls[e] == c;
      As[e * (kLinThreads / kLinTK) + tid / kLinTK][kk_a] = keep ? ra[e] : T(0);
    }
#pragma unroll
    for (int e = 0; e < kBElems; ++e) {
      const int idx = e * kLinThreads + tid;
      const int kk = TRANSW ? idx % kLinTK : idx / kLinTN;
      const int cc = TRANSW ? idx / kLinTK : idx % kLinTN;
      if constexpr (TRANSW)
        Bs[cc][kk] = rb[e];
      else
        Bs[kk][cc] = rb[e];
    }
    __syncthreads();
    have = next(c, p, k0);
    if (have) fetch(c, p, k0);
#pragma unroll
    for (int s = 0; s < kLinTK / 4; ++s) {
      const int kq = s * 4 + lane / 16;
      T a[kMT], b[kNT];
#pragma unroll
      for (int i = 0; i < kMT; ++i) a[i] = As[wr * (kLinTM / 2) + i * 16 + lane % 16][kq];
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int col = wc * (kLinTN / 2) + j * 16 + lane % 16;
        b[j] = TRANSW ? Bs[col][kq] : Bs[kq][col];
      }
#pragma unroll
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = M::mma(a[i], b[j], acc[i][j]);
    }
  }

  // epilogue: scale and store (rows of no class in range stay zero)
  const T alpha = static_cast<T>(O.alpha);
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = row0 + wr * (kLinTM / 2) + i * 16 + M::row(lane, q);
      if (row >= R) continue;
      const int nn = row / d, m = row - nn * d;
      T* orow = out + static_cast<int64_t>(nn) * dim_out + O.out_off;
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int v = col0 + wc * (kLinTN / 2) + j * 16 + lane % 16;
        if (v < O.n_ext) {
          const int64_t off = LAYOUT == kIrMul ? static_cast<int64_t>(m) * O.n_ext + v : static_cast<int64_t>(v) * d + m;
          orow[off] = alpha * acc[i][j][q];
        }
      }
    }
}

// Weight gradient of one pair, one (64 u x 128 v) tile and one chunk of
// kLinDwRows rows: part[chunk][u][v] = sum over the chunk's rows (n, m) of
// x[n, i, m, u] g[n, o, m, v] (A = x^T staged as [u][row], B = g as [row][v]).
// With class-indexed weights (CLS) the workgroup first finds the lowest and
// highest class among the chunk's samples (recorded in `ranges` by the
// chunk's first tile) and makes one pass per class in that range, rows of
// other classes (and classes outside [0, num_classes)) masked to zero:
// part[c][chunk][u][v], part_class elements apart.  Sorted classes give one
// or two passes per chunk; any order is correct.
template <typename T, int LAYOUT, bool CLS, typename Index>
__global__ void __launch_bounds__(kLinThreads)
linear_dw_kernel(const T* __restrict__ x, const T* __restrict__ g, T* __restrict__ part, int64_t n, int64_t dim_in,
                 int64_t dim_out, LinDwTable tab, const Index* __restrict__ cls, int num_classes,
                 int64_t part_class, int* __restrict__ ranges) {
  using M = Mfma<T>;
  __shared__ T As[kLinTM][kLinTK + kLinPadA];   // [u][row]
  __shared__ T Bs[kLinTK][kLinTN + kLinPadB];   // [row][v]
  const int bid = blockIdx.x;
  int pi = 0;
  while (pi + 1 < tab.n_pairs && tab.pairs[pi + 1].tile_begin <= bid) ++pi;
  const LinDwPair P = tab.pairs[pi];
  int t = bid - P.tile_begin;
  const int chunk = t / (P.u_tiles * P.v_tiles);
  t %= P.u_tiles * P.v_tiles;
  const int u0 = (t / P.v_tiles) * kLinTM, v0 = (t % P.v_tiles) * kLinTN;
  const int d = P.d;
  const int R = static_cast<int>(n) * d;
  const int r_begin = chunk * kLinDwRows;
  const int r_end = r_begin + kLinDwRows < R ? r_begin + kLinDwRows : R;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wr = wave / 2, wc = wave % 2;
  // rows staged by this thread: A row rk_a + 4 e' ... as (sample, component),
  // advanced by kLinTK rows per step without dividing
  constexpr int kAStep = kLinThreads / kLinTM;   // rows of A per pass (4)
  constexpr int kBStep = kLinThreads / kLinTN;   // rows of B per pass (2)
  const int uu_a = tid % kLinTM, rk_a = tid / kLinTM;
  const int vv_b = tid % kLinTN, rk_b = tid / kLinTN;
  int c_lo = 0, c_hi = 0;
  bool sorted = false;
  const int s_begin = r_begin / d, s_end = (r_end - 1) / d + 1;  // the chunk's samples
  // the chunk's classes in LDS for the masked passes (-1: outside [0, num_classes))
  __shared__ int cls_s[CLS ? kLinDwRows : 1];
  if constexpr (CLS) {
    int lo = num_classes, hi = -1, unsorted = 0;
    for (int sm = s_begin + tid; sm < s_end; sm += kLinThreads) {
      const int64_t c = static_cast<int64_t>(cls[sm]);
      if (sm + 1 < s_end && c > static_cast<int64_t>(cls[sm + 1])) unsorted = 1;
      cls_s[sm - s_begin] = c >= 0 && c < num_classes ? static_cast<int>(c) : -1;
      if (c >= 0 && c < num_classes) {
        lo = static_cast<int>(c) < lo ? static_cast<int>(c) : lo;
        hi = static_cast<int>(c) > hi ? static_cast<int>(c) : hi;
      }
    }
    sorted = __syncthreads_or(unsorted) == 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
      lo = l2 < lo ? l2 : lo;
      hi = h2 > hi ? h2 : hi;
    }
    __shared__ int red[2][kLinThreads / 64];
    if (lane == 0) {
      red[0][wave] = lo;
      red[1][wave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kLinThreads / 64; ++k) {
      lo = red[0][k] < lo ? red[0][k] : lo;
      hi = red[1][k] > hi ? red[1][k] : hi;
    }
    c_lo = lo;
    c_hi = hi;
    if (t == 0 && tid == 0) {
      ranges[2 * (P.range_off + chunk)] = lo;
      ranges[2 * (P.range_off + chunk) + 1] = hi;
    }
  }
  const int step_n = kLinTK / d, step_m = kLinTK - step_n * d;      // divmod(kLinTK, d)
  const int sa_n = kAStep / d, sa_m = kAStep - sa_n * d;            // divmod(kAStep, d)
  const int sb_n = kBStep / d, sb_m = kBStep - sb_n * d;            // divmod(kBStep, d)
  const int u = u0 + uu_a, v = v0 + vv_b;
  const bool u_in = u < P.mul_in, v_in = v < P.mul_out;
  const int x_off = static_cast<int>(P.x_off), g_off = static_cast<int>(P.g_off);
  // the chunk's rows through buffer resources based at its first sample:
  // 32-bit offsets, as a chunk spans at most kLinDwRows samples and the host
  // bounds dim_in and dim_out
  const __amdgpu_buffer_rsrc_t x_rsrc = buf_rsrc(x + static_cast<int64_t>(s_begin) * dim_in,
                                                 (n - s_begin) * dim_in * static_cast<int64_t>(sizeof(T)));
  const __amdgpu_buffer_rsrc_t g_rsrc = buf_rsrc(g + static_cast<int64_t>(s_begin) * dim_out,
                                                 (n - s_begin) * dim_out * static_cast<int64_t>(sizeof(T)));
  for (int cc = c_lo; cc <= c_hi; ++cc) {
  // rows [kb, ke) of the pass; when the chunk's classes are sorted, class
  // cc is one run of samples (found by binary search) and the pass covers
  // exactly its rows, else every row of the chunk with the others masked
  int kb = r_begin, ke = r_end;
  bool mask = CLS;
  if constexpr (CLS) {
    if (sorted) {
      auto first_at_least = [&](int64_t c) {  // first sample of the chunk with class >= c
        int lo = s_begin, hi = s_end;
        while (lo < hi) {
          const int mid = (lo + hi) / 2;
          if (static_cast<int64_t>(cls[mid]) < c) lo = mid + 1;
          else hi = mid;
        }
        return lo;
      };
      const int sa = first_at_least(cc), sb = first_at_least(static_cast<int64_t>(cc) + 1);
      kb = sa * d > r_begin ? sa * d : r_begin;
      ke = sb * d < r_end ? sb * d : r_end;
      mask = false;
    }
  }
  int a_n = (kb + rk_a) / d, a_m = (kb + rk_a) - a_n * d;
  int b_n = (kb + rk_b) / d, b_m = (kb + rk_b) - b_n * d;
  // rows of another class than cc contribute nothing (the index is clamped
  // so that the read stays in cls_s for rows past the pass)
  auto in_class = [&](int nn) {
    const int i = nn - s_begin < kLinDwRows - 1 ? nn - s_begin : kLinDwRows - 1;
    return !mask || cls_s[i] == cc;
  };
  typename M::acc_t acc[kMT][kNT];
#pragma unroll
  for (int a = 0; a < kMT; ++a)
#pragma unroll
    for (int b = 0; b < kNT; ++b) acc[a][b] = typename M::acc_t{0, 0, 0, 0};
  // the next chunk of rows is loaded into registers while the current one
  // is multiplied; masked elements read zero through the buffer range check
  T ra[kLinTK / kAStep], rb[kLinTK / kBStep];
  auto fetch = [&](int k0) {
    int nn = a_n, m = a_m;
#pragma unroll
    for (int e = 0; e < kLinTK / kAStep; ++e) {
      const int row = k0 + rk_a + e * kAStep;
      const bool take = row < ke && u_in && in_class(nn);
      const int off = (nn - s_begin) * static_cast<int>(dim_in) + x_off +
                      (LAYOUT == kIrMul ? m * P.mul_in + u : u * d + m);
      ra[e] = buf_load<T>(x_rsrc, take ? static_cast<uint32_t>(off) * sizeof(T) : kBufMasked);
      nn += sa_n;
      m += sa_m;
      if (m >= d) {
        m -= d;
        ++nn;
      }
    }
    nn = b_n;
    m = b_m;
#pragma unroll
    for (int e = 0; e < kLinTK / kBStep; ++e) {
      const int row = k0 + rk_b + e * kBStep;
      const bool take = row < ke && v_in && in_class(nn);
      const int off = (nn - s_begin) * static_cast<int>(dim_out) + g_off +
                      (LAYOUT == kIrMul ? m * P.mul_out + v : v * d + m);
      rb[e] = buf_load<T>(g_rsrc, take ? static_cast<uint32_t>(off) * sizeof(T) : kBufMasked);
      nn += sb_n;
      m += sb_m;
      if (m >= d) {
        m -= d;
        ++nn;
      }
    }
    // advance the staged rows by kLinTK for the next fetch
    a_n += step_n;
    a_m += step_m;
    if (a_m >= d) {
      a_m -= d;
      ++a_n;
    }
    b_n += step_n;
    b_m += step_m;
    if (b_m >= d) {
      b_m -= d;
      ++b_n;
    }
  };
  int k0 = kb;
  if (k0 < ke) fetch(k0);
  while (k0 < ke) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kLinTK / kAStep; ++e) As[uu_a][rk_a + e * kAStep] = ra[e];
#pragma unroll
    for (int e = 0; e < kLinTK / kBStep; ++e) Bs[rk_b + e * kBStep][vv_b] = rb[e];
    __syncthreads();
    k0 += kLinTK;
    if (k0 < ke) fetch(k0);
#pragma unroll
    for (int s = 0; s < kLinTK / 4; ++s) {
      const int kq = s * 4 + lane / 16;
      T a[kMT], b[kNT];
#pragma unroll
      for (int i = 0; i < kMT; ++i) a[i] = As[wr * (kLinTM / 2) + i * 16 + lane % 16][kq];
#pragma unroll
      for (int j = 0; j < kNT; ++j) b[j] = Bs[kq][wc * (kLinTN / 2) + j * 16 + lane % 16];
#pragma unroll
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = M::mma(a[i], b[j], acc[i][j]);
    }
  }
  T* prow = part + (CLS ? cc * part_class : 0) + P.part_off + static_cast<int64_t>(chunk) * P.mul_in * P.mul_out;
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int j = 0; j < kNT; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int uo = u0 + wr * (kLinTM / 2) + i * 16 + M::row(lane, q);
        const int vo = v0 + wc * (kLinTN / 2) + j * 16 + lane % 16;
        if (uo < P.mul_in && vo < P.mul_out) prow[static_cast<int64_t>(uo) * P.mul_out + vo] = acc[i][j][q];
      }
  }
}

// dw[c][w_off + e] = alpha * sum over the pair's chunks (in order) of
// part[c][chunk][e]; with classes (CLS, class c = blockIdx.z) only the
// chunks whose class range holds c have written that partial.
template <typename T, bool CLS>
__global__ void __launch_bounds__(256)
linear_dw_fold_kernel(const T* __restrict__ part, LinDwTable tab, T* __restrict__ dw, int64_t part_class,
                      int64_t numel, const int* __restrict__ ranges) {
  const int pi = blockIdx.y, c = blockIdx.z;
  const LinDwPair P = tab.pairs[pi];
  const int64_t sz = static_cast<int64_t>(P.mul_in) * P.mul_out;
  const T* pc = part + c * part_class + P.part_off;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < sz;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    T acc = T(0);
    for (int k = 0; k < P.chunks; ++k) {
      if constexpr (CLS) {
        const int lo = ranges[2 * (P.range_off + k)], hi = ranges[2 * (P.range_off + k) + 1];
        if (c < lo || c > hi) continue;
      }
      acc += pc[k * sz + e];
    }
    dw[c * numel + P.w_off + e] = static_cast<T>(P.alpha) * acc;
  }
}

template <typename T, int LAYOUT, bool CLS, typename Index>
int linear_dw_launch_c(const LinearDwArgs& a, const LinDwTable& tab) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  T* part = static_cast<T*>(a.workspace);
  const int nc = CLS ? a.num_classes : 1;
  int* ranges = CLS ? reinterpret_cast<int*>(part + a.part * nc) : nullptr;
  if (tab.total_tiles > 0)
    hipLaunchKernelGGL((linear_dw_kernel<T, LAYOUT, CLS, Index>), dim3(static_cast<unsigned>(tab.total_tiles)),
                       dim3(kLinThreads), 0, st, static_cast<const T*>(a.x), static_cast<const T*>(a.g), part, a.n,
                       a.dim_in, a.dim_out, tab, static_cast<const Index*>(a.cls), nc, a.part, ranges);
  int rc = static_cast<int>(hipGetLastError());
  if (rc || tab.n_pairs == 0) return rc;
  hipLaunchKernelGGL((linear_dw_fold_kernel<T, CLS>), dim3(64, static_cast<unsigned>(tab.n_pairs), nc), dim3(256), 0,
                     st, static_cast<const T*>(part), tab, static_cast<T*>(a.dw), a.part, a.numel, ranges);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int LAYOUT>
int linear_dw_launch(const LinearDwArgs& a, const LinDwTable& tab) {
  if (!a.cls) return linear_dw_launch_c<T, LAYOUT, false, int32_t>(a, tab);
  return a.idx == kI32 ? linear_dw_launch_c<T, LAYOUT, true, int32_t>(a, tab)
                       : linear_dw_launch_c<T, LAYOUT, true, int64_t>(a, tab);
}

template <typename T, typename Index, int LAYOUT, bool TRANSW>
int linear_launch(const LinearArgs& a, const LinTable& tab) {
  if (tab.total_tiles == 0 || a.n == 0) return 0;
  const dim3 grid(static_cast<unsigned>(tab.total_tiles));
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  if (a.classes)
    hipLaunchKernelGGL((linear_kernel<T, Index, LAYOUT, TRANSW, true>), grid, dim3(kLinThreads), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.w), static_cast<const Index*>(a.cls),
                       static_cast<T*>(a.out), a.n, a.dim_in, a.dim_out, a.numel, a.num_classes, tab);
  else
    hipLaunchKernelGGL((linear_kernel<T, Index, LAYOUT, TRANSW, false>), grid, dim3(kLinThreads), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.w), static_cast<const Index*>(a.cls),
                       static_cast<T*>(a.out), a.n, a.dim_in, a.dim_out, a.numel, a.num_classes, tab);
  return static_cast<int>(hipGetLastError());
}

template <typename T, bool TRANSW>
int linear_dispatch(const LinearArgs& a, const LinTable& tab) {
  if (a.idx == kI64) {
    if (a.layout == kMulIr) return linear_launch<T, int64_t, kMulIr, TRANSW>(a, tab);
    return linear_launch<T, int64_t, kIrMul, TRANSW>(a, tab);
  }
  if (a.layout == kMulIr) return linear_launch<T, int32_t, kMulIr, TRANSW>(a, tab);
  return linear_launch<T, int32_t, kIrMul, TRANSW>(a, tab);
}

}  // namespace kern

namespace kern {
template <typename T>
__global__ void __launch_bounds__(256) lin_fill_zero_kernel(T* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = T(0);
}
}  // namespace kern

int launch_fill_zero(void* p, int64_t n, int dtype, void* stream) {
  using namespace kern;
  if (n <= 0) return 0;
  const int64_t blocks = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 1024 ? blocks : 1024));
  if (dtype == kF32)
    hipLaunchKernelGGL((lin_fill_zero_kernel<float>), grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<float*>(p), n);
  else
    hipLaunchKernelGGL((lin_fill_zero_kernel<double>), grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<double*>(p), n);
  return static_cast<int>(hipGetLastError());
}

int launch_linear_dw(const LinearDwArgs& a, const LinDwTable& tab) {
  using namespace kern;
  if (a.dtype == kF32)
    return a.layout == kMulIr ? linear_dw_launch<float, kMulIr>(a, tab) : linear_dw_launch<float, kIrMul>(a, tab);
  return a.layout == kMulIr ? linear_dw_launch<double, kMulIr>(a, tab) : linear_dw_launch<double, kIrMul>(a, tab);
}

int launch_linear(const LinearArgs& a, const LinTable& tab, bool transw) {
  using namespace kern;
  if (a.dtype == kF32) return transw ? linear_dispatch<float, true>(a, tab) : linear_dispatch<float, false>(a, tab);
  return transw ? linear_dispatch<double, true>(a, tab) : linear_dispatch<double, false>(a, tab);
}

}  // namespace segpoly
