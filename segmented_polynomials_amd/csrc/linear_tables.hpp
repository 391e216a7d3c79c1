// Tables of the equivariant linear layer shared by the C ABI (host, built
// from the descriptor) and the MFMA kernels (passed by value as a kernel
// argument).  One GEMM per output block: rows (sample, component), K the
// concatenated input channels of its irrep type, columns its channels.
#pragma once
#include <cstdint>

namespace segpoly {

struct LinPair {
  int64_t in_off;  // offset of the input block in a row
  int64_t w_off;   // offset of the weight segment in a weight row
  int k_ext;       // channels of the input block (the pair's share of K)
  int pad;
};

struct LinOut {
  int64_t out_off;  // offset of the output block in a row
  double alpha;     // 1 / sqrt(fan-in of the block's irrep type)
  int n_ext;        // channels of the output block
  int d;            // 2l + 1
  int pair_begin, pair_end;  // its pairs in LinTable::pairs
  int tile_begin, col_tiles;  // first workgroup of its GEMM; column tiles
};

// GEMM tile of one workgroup: rows x columns (the weight-gradient GEMM:
// input channels x output channels), shared by the launchers' grid sizes
// and the kernels.
constexpr int kLinTileRows = 128;
constexpr int kLinTileCols = 128;

constexpr int kLinMaxOut = 32;
constexpr int kLinMaxPairs = 64;

// The kernels address operands through buffer resources with 32-bit byte
// offsets from a tile's (or a row chunk's) first sample.  A row chunk of the
// weight gradient spans at most kLinDwRows (2048) samples, so rows of at most
// 2^16 elements of 8 bytes keep every offset below 2^30 bytes; a class's
// weight row of at most 2^27 elements likewise.
constexpr int64_t kLinMaxDim = int64_t(1) << 16;
constexpr int64_t kLinMaxNumel = int64_t(1) << 27;

struct LinTable {
  int n_out;
  int total_tiles;
  LinOut outs[kLinMaxOut];
  LinPair pairs[kLinMaxPairs];
};

// Weight-gradient GEMMs of the backward: one per (input block, output
// block) pair, split over chunks of kLinDwRows rows.
struct LinDwPair {
  int64_t x_off, g_off, w_off;
  int mul_in, mul_out, d;
  int chunks;            // row chunks of this pair
  int64_t part_off;      // first element of its partials in the workspace
  int64_t range_off;     // first chunk of its class ranges (class-indexed weights)
  int tile_begin;        // first workgroup
  int u_tiles, v_tiles;  // tiles of mul_in x mul_out
  double alpha;
};

constexpr int kLinDwRows = 2048;

struct LinDwTable {
  int n_pairs;
  int total_tiles;
  LinDwPair pairs[kLinMaxPairs / 2];
};

struct LinearArgs {
  const void* x;    // [n, dim_in] (backward dx: the output gradient)
  const void* w;    // [1 or num_classes, numel]
  const void* cls;  // [n] class of each sample, or null
  void* out;        // [n, dim_out]
  int64_t n, dim_in, dim_out, numel;
  int num_classes;
  int classes;      // 1: class-indexed weights
  int dtype, idx, layout;
  void* stream;
};

struct LinearDwArgs {
  const void* x;    // [n, dim_in] forward input
  const void* g;    // [n, dim_out] output gradient
  const void* cls;  // [n] class of each sample, or null (shared weights)
  void* dw;         // [num_classes, numel]
  void* workspace;  // partials [num_classes][part], then the chunks' class ranges
  int64_t n, dim_in, dim_out, numel;
  int64_t part;     // partial elements of one class (fill_dw_tiles)
  int num_classes;  // 1 without classes
  int dtype, idx, layout;
  void* stream;
};

int launch_linear(const LinearArgs& a, const LinTable& tab, bool transw);
int launch_linear_dw(const LinearDwArgs& a, const LinDwTable& tab);
// p[0..n) = 0 with a kernel (stream-ordered, safe under graph capture)
int launch_fill_zero(void* p, int64_t n, int dtype, void* stream);

}  // namespace segpoly
