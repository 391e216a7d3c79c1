// Tables of the fully connected product as a graph convolution (per-edge
// weights): built on the host from the descriptor, uploaded once per device.
//
// A tile is one output block o and a range of its channels w.  Per edge the
// tile needs, for each path (i, j, o) into o, the coupled rows
//   y[p, k, u] = alpha_o sum over the entries (a, b) of k of C[a, b, k] x[src, i, a, u] sh[e, j, b]
// ("qk rows", one per path and output component) and then
//   acc[k, w] += sum_u W_e[p][u, w] y[p, k, u].
#pragma once
#include <cstdint>

#include "launch.hpp"

namespace segpoly {

constexpr int kFcvMaxD = 13;       // components of an output block (l <= 6)
constexpr int kFcvMaxLanesPerEdge = 64;

struct FcvBlock {                  // an input-1 block as staged per edge
  int64_t off;                     // offset in an x row
  int d, m, comp;                  // components, channels, first staged component
};

struct FcvPath {
  int64_t w_off;                   // weight segment in a weight row: [m1][m3], w fastest
  int m1;                          // input-1 channels (u runs over them)
  int qk;                          // first qk row of the path in its tile
};

struct FcvQK {
  int ent_begin, ent_end;          // entries of this (path, component)
};

struct FcvEnt {
  int a, b;                        // staged x component, harmonic component
  double c;                        // coefficient, alpha_o included
};

// One weight column element of a tile per (path, u): the lane's weight
// W_e[p][u, w0 + c] sits at w_off + u m + w0 + c of the edge's row, and
// multiplies the qk rows starting at qk (tile-local) for channel u.
struct FcvQ {
  int64_t off;                     // w_off + u * m
  int qk, u;
};

// Sixteen consecutive channels u0 .. u0 + 15 of one path: the weights
// W_e[p][u0 + uu, w0 + c] at off + uu m, multiplying qk rows from qk.
struct FcvChunk {
  int64_t off;                     // w_off + u0 * m
  int qk, u0;
};

constexpr int kFcvChunkU = 16;     // channels per chunk
constexpr int kFcvBatch = 4;       // chunks whose weights a lane holds in registers at a time (half in double)

// Input-1 channels are taken 64 at a time when a block has more than 64
// (a "u tile"; one u tile otherwise): the weight elements of one output
// block and one u tile, the full 16-channel chunks of its paths that lie in
// the u tile and then the remaining (path, u) elements one by one.
constexpr int kFcvUTile = 64;

struct FcvUT {
  int chunk_begin, n_chunks;       // full 16-channel chunks
  int q_begin, nq;                 // the remaining (path, u) weight elements
};

struct FcvTile {
  int64_t out_off;                 // block offset in an output row
  int d, m, w0, nw;                // components, channels, channel range of the tile
  int path_begin, path_end;        // paths into the block
  int qk_begin, nqk;               // qk rows of the tile
  int ut_begin;                    // its u tiles' weight elements (n_ut entries of FcvUT)
  int pad;
};

// Backward: every path with its rows in the global list of coupled rows
// (the tiles' rows, output block by block).
struct FcvBPath {
  int64_t w_off;                   // weight segment [m1][m3]
  int64_t g_off;                   // output block offset in a row of the output gradient
  int m1, m3, d3;
  int row;                         // first of its d3 rows
};

struct FcvBwdArgs {
  const void* x;
  const void* sh;
  const void* w;
  const void* g;
  const void* src;
  const void* dst;
  const void* perm;                // edges ordered by source (stable argsort of src)
  int64_t n_src, n_edges, n_nodes;
  int64_t dim1, dim2, dimo, numel;
  int mean;
  void* dx;
  void* dsh;
  void* dw;
  void* msg;                       // workspace: per-edge source messages [n_edges][dim1]
  int shared_w;                    // one weight row for every edge: dw [1, numel] sums over the edges
  int64_t dw_ws_off;               // shared: byte offset of the per-edge dw rows in the workspace
  const FcvBlock* blocks;          // device tables
  const FcvQK* qks;
  const FcvEnt* ents;
  const FcvBPath* bpaths;
  int n_blocks, n_bpaths, nrows, ncomp, lane_bits;
  int n_ut;                        // u tiles of kFcvUTile input channels (1 when no block has more)
  size_t lds_bytes;
  int dtype, layout, idx;
  void* stream;
};

int launch_fcconv_bwd(const FcvBwdArgs& a);

struct FcvArgs {
  const void* x;
  const void* sh;
  const void* w;
  const void* src;
  const void* dst;
  int64_t n_src, n_edges, n_nodes;
  int64_t dim1, dim2, dimo;
  int64_t w_stride;                // weight row stride: weight_numel, or 0 for one shared row
  void* out;
  int mean;
  const FcvBlock* blocks;          // device tables
  const FcvPath* paths;
  const FcvQK* qks;
  const FcvEnt* ents;
  const FcvTile* tiles;
  const FcvUT* uts;
  const FcvQ* qs;
  const FcvChunk* chunks;
  int n_blocks, n_tiles;
  int n_ut;                        // u tiles of kFcvUTile input channels (1 when no block has more)
  int ncomp;                       // staged x components per edge (sum of 2l + 1)
  int max_nqk;                     // qk rows of the largest tile
  int lane_bits;                   // log2 of the lanes per edge (channels rounded up to a power of two)
  size_t lds_bytes;
  int dtype, layout, idx;
  void* stream;
};

int launch_fcconv(const FcvArgs& a);

}  // namespace segpoly
