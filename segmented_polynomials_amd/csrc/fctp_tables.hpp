// Tables of the fully connected tensor product kernels (plain structs,
// built on the host from the descriptor, uploaded once per device).
//
// Every pass of the product (forward, input-1 gradient, input-2 gradient)
// is the same computation seen from a different "result" operand:
//   res[n, R, r, c] = sum over the terms t of R of
//                     sum over (p, q) of B_t[(p, q), c] A_t[n, r, (p, q)],
//   A_t[n, r, (p, q)] = sum over the entries e of (t, r) of
//                       coef_e P[n, Pblk_t, pa_e, p] Q[n, Qblk_t, qb_e, q],
// a GEMM per result block with rows (n, r), K = (p, q) and columns c, whose
// A operand is generated from two per-sample operands and whose B operand
// is the weight segment read with the term's strides.  The path
// normalisation is folded into coef.
#pragma once
#include <cstdint>

#include "launch.hpp"

namespace segpoly {

// Entries per (term, result component) rounded up to a compiled class: a
// launch runs one class, the largest among its terms (smaller terms are
// zero-padded).
constexpr int fc_t_class(int t) {
  return t <= 1 ? 1 : t <= 2 ? 2 : t <= 3 ? 3 : t <= 4 ? 4 : t <= 6 ? 6 : t <= 8 ? 8 : 16;
}

constexpr int kFcMaxT = 16;      // coupling entries per (term, result component): every l <= 6
constexpr int kFcMaxRes = 32;    // result blocks per pass
constexpr int kFcRT = 2;         // 16-row MFMA tiles per wave (4 waves per workgroup)
constexpr int kFcRowsMax = 64 * kFcRT;  // rows (sample, component) per tile
constexpr int kFcPad = 1;        // LDS padding of each staged channel row
constexpr int kFcDwChunk = 1024; // samples per weight-gradient partial sum
constexpr int kFcDwSamples = 16; // samples a weight-gradient workgroup stages at a time (few: several
                                 // workgroups then share a CU and hide each other's staging loads)

// LDS stride of one staged sample ([component][channel + kFcPad]), rounded up
// to 16 mod 32 elements: the four samples one MFMA step reads (lane / 16)
// then start 16 banks apart in float (32 in double), so a 16-lane row of
// consecutive channels never shares a bank with another sample's.
constexpr int fc_sample_stride(int d, int m) {
  const int base = d * (m + kFcPad);
  return base + ((16 - base % 32) + 32) % 32;
}

// P is the operand with fewer channels (one channel per K chunk), Q the one
// with more (a window of channels per K chunk, held in registers).
struct FcTerm {
  int p_op, q_op;           // operand of P and Q: 0 = input 1, 1 = input 2, 2 = output gradient
  int p_d, p_m, q_d, q_m;   // components and channels of the two blocks
  int64_t p_off, q_off;     // block offsets within an operand row
  int64_t w_off;            // weight segment of the path
  int64_t s_p, s_q, s_r;    // weight strides of channel p, channel q, result channel
  int T;                    // entries per result component (zero-padded)
  int ent;                  // first entry: [result component][T]
};

struct FcEnt {
  int pa, qb;               // P component, Q component
  double c;                 // coefficient, normalisation included
};

struct FcRes {
  int64_t off;              // block offset within a result row
  int d, m;                 // components and channels
  int term_begin, term_end;
  int ts;                   // samples per tile (ts * d <= kFcRowsMax)
  int col_tiles;
};

// Per-call tile map of one pass: result block r owns tiles
// [tile_begin[r], tile_begin[r + 1]), row tile major.
struct FcTiles {
  int n_res;
  int tile_begin[kFcMaxRes + 1];
};

// Weight gradient: one term per path seen as a GEMM with rows (p, q) (a
// channel of P and one of Q: input 1 and input 2, Q the one with more
// channels), K = (output component, sample) and columns w (output channel):
//   dW[w_off + p s_p + q s_q + w] = sum over samples n and components k of
//       sum over the entries e of k of coef_e P[n, pa_e, p] Q[n, qb_e, q] g[n, o, k, w].
// A workgroup tile is kFcDwU channels p x kFcDwV channels q x kFcDwCols
// columns; each wave owns 2 p x 32 q.
struct FcDwPath {
  int p_op, q_op;           // 0 = input 1, 1 = input 2
  int p_d, p_m, q_d, q_m, g_d, g_m;
  int64_t p_off, q_off, g_off, w_off;
  int64_t s_p, s_q;         // weight strides of channel p and channel q
  int T, ent;               // entries [output component][T]
  int ts;                   // samples staged at a time (a multiple of 4)
  int u_tiles, v_tiles;     // tiles of kFcDwU channels p and kFcDwV channels q
  int col_tiles;            // tiles of kFcDwCols columns w
};

// Float weight-gradient staging straight into LDS: two static buffers of
// kFcDwDmaElems floats per workgroup (the group being multiplied and the
// next), and at most kFcDwDmaJ dword copies per lane for one staged sample
// of a block (sample strides up to 64 kFcDwDmaJ floats).
constexpr int kFcDwDmaElems = 4096;
constexpr int kFcDwDmaJ = 2;

constexpr int kFcDwU = 8;        // P channels per weight-gradient tile (2 per wave)
constexpr int kFcDwV = 32;       // Q channels per weight-gradient tile
constexpr int kFcDwCols = 32;    // output channels per weight-gradient tile
constexpr int kFcMaxPaths = 64;

// Per call: path p owns tiles [tile_begin[p], tile_begin[p + 1]), ordered
// (sample chunk, u tile, v tile, column tile).
struct FcDwTiles {
  int n_paths;
  int chunks;                    // sample chunks of kFcDwChunk
  int tile_begin[kFcMaxPaths + 1];
};

struct FcArgs {
  const void* op[3];        // input 1, input 2, output gradient (unused ones NULL)
  int64_t dim[3];           // their row widths
  const void* w;            // [1, weight_numel]
  void* res;                // result rows
  int64_t dim_res;
  int64_t n;
  const FcRes* res_tab;     // device tables
  const FcTerm* terms;
  const FcEnt* ents;
  int tn;                   // column tile width: 32 or 64
  int nt;                   // entry class (fc_t_class)
  int lds_direct;           // weight chunks copied straight into LDS (see fc_term)
  size_t lds_bytes;
  int dtype, layout;
  void* stream;
};

struct FcDwArgs {
  const void* x1;
  const void* x2;
  const void* g;
  int64_t dim1, dim2, dimo;
  void* part;               // [chunks][weight_numel]
  void* dw;                 // [weight_numel]
  int64_t numel;
  int64_t n;
  const FcDwPath* paths;    // device
  const FcEnt* ents;
  int nt;                   // entry class (fc_t_class)
  size_t lds_bytes;
  int dma;                  // stage through the static LDS-direct buffers (float only)
  int dtype, layout;
  void* stream;
};

// The input-gradient passes read the weights transposed, so that their
// result channel is the contiguous weight index (the form whose chunks go
// straight into LDS): per path W[u][v][w] -> W1[v][w][u] (for dx1) and
// W2[u][w][v] (for dx2), at the same segment offsets.
struct FcTrPath {
  int64_t w_off;
  int m1, m2, m3;
};

struct FcTrArgs {
  const void* w;
  void* w1;
  void* w2;
  const FcTrPath* paths;    // device, in segment order
  int n_paths;
  int64_t numel;
  int dtype;
  void* stream;
};

int launch_fctp_transpose_f32(const FcTrArgs& a);
int launch_fctp_transpose_f64(const FcTrArgs& a);

inline int launch_fctp_transpose(const FcTrArgs& a) {
  return a.dtype == kF32 ? launch_fctp_transpose_f32(a) : launch_fctp_transpose_f64(a);
}

int launch_fctp_f32(const FcArgs& a, const FcTiles& t);
int launch_fctp_f64(const FcArgs& a, const FcTiles& t);
int launch_fctp_dw_f32(const FcDwArgs& a, const FcDwTiles& t);
int launch_fctp_dw_f64(const FcDwArgs& a, const FcDwTiles& t);

inline int launch_fctp(const FcArgs& a, const FcTiles& t) {
  return a.dtype == kF32 ? launch_fctp_f32(a, t) : launch_fctp_f64(a, t);
}
inline int launch_fctp_dw(const FcDwArgs& a, const FcDwTiles& t) {
  return a.dtype == kF32 ? launch_fctp_dw_f32(a, t) : launch_fctp_dw_f64(a, t);
}

}  // namespace segpoly
