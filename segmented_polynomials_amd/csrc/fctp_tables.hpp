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

// Division of a non-negative 31-bit integer by an invariant divisor d >= 1
// with one high multiply, an add and a shift (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994, round-up
// variant): shift = ceil(log2 d), magic = floor(2^32 (2^shift - d) / d) + 1,
// n / d = (umulhi(n, magic) + n) >> shift.
struct FastDiv {
  uint32_t magic;
  int shift;
  int d;
};

inline FastDiv make_fast_div(int d) {
  FastDiv f{};
  f.d = d;
  f.shift = 0;
  while ((1ll << f.shift) < d) ++f.shift;
  f.magic = static_cast<uint32_t>(((uint64_t(1) << 32) * ((uint64_t(1) << f.shift) - uint64_t(d))) / uint64_t(d) + 1);
  return f;
}

constexpr int kFcMaxT = 8;       // coupling entries per (term, result component)
constexpr int kFcMaxRes = 32;    // result blocks per pass
constexpr int kFcRowsMax = 128;  // rows (sample, component) per tile
constexpr int kFcPad = 1;        // LDS padding of each staged channel row
constexpr int kFcDwChunk = 2048; // samples per weight-gradient partial sum

struct FcTerm {
  int p_op, q_op;           // operand of P and Q: 0 = input 1, 1 = input 2, 2 = output gradient
  int p_d, p_m, q_d, q_m;   // components and channels of the two blocks
  int64_t p_off, q_off;     // block offsets within an operand row
  int64_t w_off;            // weight segment of the path
  int64_t s_p, s_q, s_r;    // weight strides of channel p, channel q, result channel
  int T;                    // entries per result component (zero-padded)
  int ent;                  // first entry: [result component][T]
  FastDiv q_div;            // division by q_m (K index -> (p, q))
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

// Weight gradient: one term per path seen as a GEMM with rows (u, v) =
// (input-1 channel, input-2 channel), K = (sample, output component) and
// columns w (output channel); P = input 1, Q = input 2, G = output gradient.
struct FcDwPath {
  int p_d, p_m, q_d, q_m, g_d, g_m;
  int64_t p_off, q_off, g_off, w_off;
  int T, ent;               // entries [output component][T] (the forward's)
  int ts;                   // samples staged at a time (a multiple of 4)
  int m_tiles;              // tiles of kFcDwRows rows (u, v)
  int col_tiles;            // tiles of kFcDwCols columns w
  FastDiv q_div;            // division by q_m (row -> (u, v))
};

constexpr int kFcDwRows = 256;   // (u, v) rows per weight-gradient tile
constexpr int kFcDwCols = 32;    // output channels per weight-gradient tile
constexpr int kFcMaxPaths = 64;

// Per call: path p owns tiles [tile_begin[p], tile_begin[p + 1]), ordered
// (sample chunk, row tile, column tile).
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
  int tn;                   // column tile width: 16, 32 or 64
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
  size_t lds_bytes;
  int dtype, layout;
  void* stream;
};

int launch_fctp(const FcArgs& a, const FcTiles& t);
int launch_fctp_dw(const FcDwArgs& a, const FcDwTiles& t);

}  // namespace segpoly
