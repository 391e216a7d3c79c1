// Launch arguments shared by the C ABI and the kernel translation units.
// Plain pointers and sizes; the stream is a hipStream_t passed as void*.
#pragma once
#include <cstdint>

namespace segpoly {

enum Layout : int { kMulIr = 0, kIrMul = 1 };
enum DType : int { kF32 = 0, kF64 = 1 };
enum IdxType : int { kI32 = 0, kI64 = 1 };

struct TPArgs {
  const void* x;      // [n_src, dim1]
  const void* sh;     // [n_edges, dim2]
  const void* w;      // [n_edges or 1, numel]
  const void* src;    // [n_edges] or null (batch mode)
  const void* dst;    // [n_edges], sorted ascending, or null (batch mode)
  const void* row_ptr;  // [n_nodes + 1] first edge of each destination (index dtype), or null: search dst
  void* out;          // [n_nodes, dim_out]
  int64_t n_src, n_edges, n_nodes;
  int64_t w_stride;   // numel, or 0 for shared weights
  int mul;            // channels of every input-1 block (specialised kernels)
  int batch;          // 1: batch mode, edge e feeds row e (src, dst unused)
  int mean;           // 1: each output row divided by its number of edges
  int dtype, idx, layout;
  void* stream;
  // fused harmonics: with `vec` ([n_edges, 3]) set, sh is computed in the
  // kernel from the edge vectors (degrees 0..L, D2 = (L+1)^2) instead of read
  const void* vec;
  int sh_normalize;
  const struct ShConsts* sh_consts;
};

// Backward of the TP-conv (per-edge weights, specialised kernels only).
struct TPBwdArgs {
  const void* x;      // [n_src, dim1]
  const void* sh;     // [n_edges, dim2]
  const void* w;      // [n_edges, numel]
  const void* src;    // [n_edges] or null (batch mode)
  const void* dst;    // [n_edges], sorted ascending, or null (batch mode)
  const void* perm;   // [n_edges] edge ids ordered by src, or null (batch mode)
  const void* row_ptr;      // [n_nodes + 1] destination row pointers, or null (ranges searched in dst)
  const void* src_row_ptr;  // [n_src + 1] source row pointers over perm order, or null (searched)
  const void* g;      // [n_nodes, dim_out] gradient of the output
  void* dx;           // [n_src, dim1]
  void* dsh;          // [n_edges, dim2]
  void* dw;           // [n_edges, numel], or [1, numel] with shared weights
  void* workspace;    // [n_edges, dim1] per-edge source messages (unused in batch mode), ...
  int64_t n_src, n_edges, n_nodes;
  int mul;
  int batch;
  int mean;           // 1: the forward divided each row by its number of edges
  int shared_w;       // 1: w is one row shared by every edge (dw sums over the edges)
  int64_t dw_ws_off;  // shared weights: byte offset of the per-edge dw rows in the workspace
  int64_t keys_ws_off;  // indexed mode: byte offset of the sorted source keys [n_edges] int32
  int dtype, idx, layout;
  void* stream;
};

struct SymconArgs {
  const void* x;        // [n_atoms, dim_in]
  const void* species;  // [n_atoms]
  const void* w;        // [num_elements, numel]
  void* out;            // [n_atoms, dim_out]
  int64_t n_atoms;
  int num_elements;
  int mul;
  int dtype, idx, layout;
  void* stream;
};

// Backward of the symmetric contraction (specialised kernels only).
struct SymconBwdArgs {
  const void* x;        // [n_atoms, dim_in]
  const void* species;  // [n_atoms]
  const void* perm;     // [n_atoms] atom ids ordered by species
  const void* w;        // [num_elements, numel]
  const void* g;        // [n_atoms, dim_out] gradient of the output
  void* dx;             // [n_atoms, dim_in]
  void* dw;             // [num_elements, numel]
  void* workspace;      // segment table, then per-chunk weight-gradient partials
  int64_t n_atoms;
  int num_elements;
  int mul;
  int dtype, idx, layout;
  void* stream;
};

constexpr int kShMaxL = 6;

// N_l0 and sqrt2 N_lm (m > 0) of the real harmonics at index l (l + 1) / 2 + m,
// computed on the host in extended precision.
struct ShConsts {
  double c[(kShMaxL + 1) * (kShMaxL + 2) / 2];
};

// Spherical harmonics of vectors: forward (grad null: out = Y [n, (lmax+1)^2])
// or vector-Jacobian product (out = dL/dv [n, 3] for grad = dL/dY).
struct ShArgs {
  const void* vec;   // [n, 3]
  const void* grad;  // [n, (lmax + 1)^2] or null
  void* out;
  int64_t n;
  int lmax;
  int normalize;
  int dtype;
  const ShConsts* consts;
  void* stream;
};
int launch_sh(const ShArgs& a);

// Workspace layouts of the backward calls, shared by the C ABI (sizes) and
// the launchers (offsets).
inline int64_t round_up_256(int64_t n) { return (n + 255) / 256 * 256; }
// Edges per partial sum of a shared weight gradient (then the partials in order).
constexpr int64_t kTpDwChunk = 1024;

// Symmetric contraction: a segment table of 2 * (E + 3) int64, then one
// partial weight-gradient row per chunk of kSymconBwdChunk atoms (each
// element segment adds at most one partial chunk, so E + 2 extra rows).
constexpr int kSymconBwdChunk = 8;
inline int64_t symcon_bwd_table_bytes(int num_elements) { return round_up_256(16 * (num_elements + 3)); }
inline int64_t symcon_bwd_max_chunks(int64_t n_atoms, int num_elements) {
  return (n_atoms + kSymconBwdChunk - 1) / kSymconBwdChunk + num_elements + 2;
}

// Returns 0 or a hipError_t value of the launch.
using TPLaunchFn = int (*)(const TPArgs&);
using SymconLaunchFn = int (*)(const SymconArgs&);
using TPBwdLaunchFn = int (*)(const TPBwdArgs&);
using SymconBwdLaunchFn = int (*)(const SymconBwdArgs&);

struct TPSpecEntry {
  const char* key;
  const char* name;
  unsigned dtypes;  // bit 0: f32, bit 1: f64
  TPLaunchFn launch;
  TPBwdLaunchFn launch_bwd;
};

struct SymconSpecEntry {
  const char* key;
  const char* name;
  unsigned dtypes;
  SymconLaunchFn launch;
  SymconBwdLaunchFn launch_bwd;
};

// generated registry
extern const TPSpecEntry kTPSpecs[];
extern const int kNumTPSpecs;
extern const SymconSpecEntry kSymconSpecs[];
extern const int kNumSymconSpecs;

}  // namespace segpoly
