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
  void* out;          // [n_nodes, dim_out]
  int64_t n_src, n_edges, n_nodes;
  int64_t w_stride;   // numel, or 0 for shared weights
  int mul;            // channels of every input-1 block (specialised kernels)
  int batch;          // 1: batch mode, edge e feeds row e (src, dst unused)
  int dtype, idx, layout;
  void* stream;
};

// Backward of the TP-conv (per-edge weights, specialised kernels only).
struct TPBwdArgs {
  const void* x;      // [n_src, dim1]
  const void* sh;     // [n_edges, dim2]
  const void* w;      // [n_edges, numel]
  const void* src;    // [n_edges] or null (batch mode)
  const void* dst;    // [n_edges], sorted ascending, or null (batch mode)
  const void* perm;   // [n_edges] edge ids ordered by src, or null (batch mode)
  const void* g;      // [n_nodes, dim_out] gradient of the output
  void* dx;           // [n_src, dim1]
  void* dsh;          // [n_edges, dim2]
  void* dw;           // [n_edges, numel]
  void* workspace;    // [n_edges, dim1] per-edge source messages (unused in batch mode)
  int64_t n_src, n_edges, n_nodes;
  int mul;
  int batch;
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

// Returns 0 or a hipError_t value of the launch.
using TPLaunchFn = int (*)(const TPArgs&);
using SymconLaunchFn = int (*)(const SymconArgs&);
using TPBwdLaunchFn = int (*)(const TPBwdArgs&);

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
};

// generated registry
extern const TPSpecEntry kTPSpecs[];
extern const int kNumTPSpecs;
extern const SymconSpecEntry kSymconSpecs[];
extern const int kNumSymconSpecs;

}  // namespace segpoly
