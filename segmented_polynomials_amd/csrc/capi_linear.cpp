// C ABI of the equivariant linear layer: descriptor tables, validation,
// launches.  Host code.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <map>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "capi_util.hpp"
#include "irreps.hpp"
#include "launch.hpp"
#include "linear_tables.hpp"
#include "segpoly.h"

using namespace segpoly;

namespace {

constexpr int kLinTM = kLinTileRows, kLinTN = kLinTileCols, kLinDwTM = kLinTileRows;

template <typename Index>
int check_classes(const void* dcls, int64_t n, int num_classes, void* stream) {
  std::vector<Index> c(n);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess && n) e = hipMemcpy(c.data(), dcls, n * sizeof(Index), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SEGPOLY_E_HIP, std::string("validate copy: ") + hipGetErrorString(e));
  for (int64_t i = 0; i < n; ++i)
    if (c[i] < 0 || static_cast<int64_t>(c[i]) >= num_classes)
      return fail(SEGPOLY_E_RANGE, "classes[" + std::to_string(i) + "] outside [0, num_classes)");
  return ok();
}

}  // namespace

struct segpoly_linear {
  std::vector<Irrep> in, out;
  std::vector<int64_t> in_off, out_off;
  int layout = 0, dtype = 0;
  unsigned flags = 0;
  int64_t dim_in = 0, dim_out = 0, numel = 0;
  LinTable fwd{}, bwd{};  // tile fields filled per call
  LinDwTable dw{};
};

namespace {

// Per-call tiles of a GEMM table for n samples.
void fill_tiles(LinTable& t, const std::vector<Irrep>& blocks, int64_t n) {
  int64_t acc = 0;
  for (int o = 0; o < t.n_out; ++o) {
    LinOut& O = t.outs[o];
    const int64_t rows = n * O.d;
    const int64_t row_tiles = (rows + kLinTM - 1) / kLinTM;
    O.col_tiles = (O.n_ext + kLinTN - 1) / kLinTN;
    O.tile_begin = static_cast<int>(acc);
    acc += row_tiles * O.col_tiles;
  }
  (void)blocks;
  t.total_tiles = static_cast<int>(acc);
}

int64_t fill_dw_tiles(LinDwTable& t, int64_t n, int64_t* n_chunks = nullptr) {
  int64_t tiles = 0, part = 0, chunks = 0;
  for (int p = 0; p < t.n_pairs; ++p) {
    LinDwPair& P = t.pairs[p];
    const int64_t rows = n * P.d;
    P.chunks = static_cast<int>((rows + kLinDwRows - 1) / kLinDwRows);
    P.u_tiles = (P.mul_in + kLinDwTM - 1) / kLinDwTM;
    P.v_tiles = (P.mul_out + kLinTN - 1) / kLinTN;
    P.tile_begin = static_cast<int>(tiles);
    P.part_off = part;
    P.range_off = chunks;
    tiles += static_cast<int64_t>(P.chunks) * P.u_tiles * P.v_tiles;
    part += static_cast<int64_t>(P.chunks) * P.mul_in * P.mul_out;
    chunks += P.chunks;
  }
  t.total_tiles = static_cast<int>(tiles);
  if (n_chunks) *n_chunks = chunks;
  return part;  // elements of partials (of one class)
}

// Workspace of the weight gradient: the partials of every class, then two
// int32 (first and last class present) per row chunk with classes.
size_t dw_workspace_bytes(const segpoly_linear* h, int64_t n, int num_classes) {
  LinDwTable t = h->dw;
  int64_t chunks = 0;
  const int64_t part = fill_dw_tiles(t, n, &chunks);
  if (part == 0) return 0;
  const size_t elt = h->dtype == SEGPOLY_F32 ? 4 : 8;
  if (num_classes <= 0) return static_cast<size_t>(part) * elt;
  return static_cast<size_t>(part) * num_classes * elt + static_cast<size_t>(chunks) * 2 * sizeof(int32_t);
}

bool tiles_fit(int64_t n, const segpoly_linear* h) {
  // rows (sample, component) are 32-bit in the kernels, and the flattened
  // grids must stay below 2^31 workgroups
  int lmax = 0;
  for (const auto& b : h->in) lmax = b.l > lmax ? b.l : lmax;
  for (const auto& b : h->out) lmax = b.l > lmax ? b.l : lmax;
  if (static_cast<double>(n) * (2 * lmax + 1) >= 2.0e9) return false;
  double t = 0, u = 0;
  for (const auto& b : h->out) t += std::ceil(double(n) * (2 * b.l + 1) / kLinTM) * std::ceil(double(b.mul) / kLinTN);
  for (const auto& b : h->in) u += std::ceil(double(n) * (2 * b.l + 1) / kLinTM) * std::ceil(double(b.mul) / kLinTN);
  return t < 2.0e9 && u < 2.0e9;
}

}  // namespace

extern "C" {

int linear_create(const char* irreps_in, const char* irreps_out, int layout, int dtype, unsigned flags,
                  linear_handle* out) {
  if (!out) return fail(SEGPOLY_E_INVALID, "null handle pointer");
  *out = nullptr;
  if (!irreps_in || !irreps_out) return fail(SEGPOLY_E_INVALID, "null irreps string");
  if (layout != SEGPOLY_MUL_IR && layout != SEGPOLY_IR_MUL) return fail(SEGPOLY_E_INVALID, "bad layout");
  if (dtype != SEGPOLY_F32 && dtype != SEGPOLY_F64) return fail(SEGPOLY_E_INVALID, "bad dtype");
  if (flags & ~SEGPOLY_VALIDATE) return fail(SEGPOLY_E_INVALID, "unknown flag bits");
  segpoly_linear* h = nullptr;
  try {
    h = new segpoly_linear();
    h->in = parse_irreps(irreps_in);
    h->out = parse_irreps(irreps_out);
  } catch (const ParseError& e) {
    delete h;
    return fail(SEGPOLY_E_PARSE, e.what());
  } catch (const std::bad_alloc&) {
    delete h;
    return fail(SEGPOLY_E_OOM, "out of host memory");
  } catch (const std::exception& e) {
    delete h;
    return fail(SEGPOLY_E_INVALID, e.what());
  }
  h->layout = layout;
  h->dtype = dtype;
  h->flags = flags;
  for (const auto& b : h->in) {
    h->in_off.push_back(h->dim_in);
    h->dim_in += static_cast<int64_t>(b.mul) * (2 * b.l + 1);
  }
  for (const auto& b : h->out) {
    h->out_off.push_back(h->dim_out);
    h->dim_out += static_cast<int64_t>(b.mul) * (2 * b.l + 1);
  }
  // weight segments: (input block, output block) pairs of equal type, i then o
  std::map<std::pair<int, int>, int64_t> woff;
  std::map<std::pair<int, int>, int> fan_in;
  for (size_t i = 0; i < h->in.size(); ++i) {
    fan_in[{h->in[i].l, h->in[i].p}] += h->in[i].mul;
    for (size_t o = 0; o < h->out.size(); ++o)
      if (h->in[i].l == h->out[o].l && h->in[i].p == h->out[o].p) {
        woff[{static_cast<int>(i), static_cast<int>(o)}] = h->numel;
        h->numel += static_cast<int64_t>(h->in[i].mul) * h->out[o].mul;
      }
  }
  if (h->dim_in > kLinMaxDim || h->dim_out > kLinMaxDim || h->numel > kLinMaxNumel) {
    delete h;
    return fail(SEGPOLY_E_UNSUPPORTED, "rows wider than 65536 elements or more than 2^27 weights");
  }
  const int n_pairs = static_cast<int>(woff.size());
  if (h->out.size() > static_cast<size_t>(kLinMaxOut) || h->in.size() > static_cast<size_t>(kLinMaxOut) ||
      n_pairs > kLinMaxPairs / 2) {
    delete h;
    return fail(SEGPOLY_E_UNSUPPORTED, "too many blocks or block pairs for the linear kernels");
  }
  auto alpha = [&](int l, int p) {
    auto it = fan_in.find({l, p});
    return it == fan_in.end() ? 0.0 : 1.0 / std::sqrt(static_cast<double>(it->second));
  };
  // forward: one GEMM per output block over its same-type input blocks
  LinTable& F = h->fwd;
  F.n_out = static_cast<int>(h->out.size());
  int np = 0;
  for (size_t o = 0; o < h->out.size(); ++o) {
    LinOut& O = F.outs[o];
    O.out_off = h->out_off[o];
    O.alpha = alpha(h->out[o].l, h->out[o].p);
    O.n_ext = h->out[o].mul;
    O.d = 2 * h->out[o].l + 1;
    O.pair_begin = np;
    for (size_t i = 0; i < h->in.size(); ++i) {
      auto it = woff.find({static_cast<int>(i), static_cast<int>(o)});
      if (it == woff.end()) continue;
      F.pairs[np++] = LinPair{h->in_off[i], it->second, h->in[i].mul, 0};
    }
    O.pair_end = np;
  }
  // backward dx: one GEMM per input block over the same-type output blocks,
  // the weight segment read transposed
  LinTable& B = h->bwd;
  B.n_out = static_cast<int>(h->in.size());
  np = 0;
  for (size_t i = 0; i < h->in.size(); ++i) {
    LinOut& O = B.outs[i];
    O.out_off = h->in_off[i];
    O.alpha = alpha(h->in[i].l, h->in[i].p);
    O.n_ext = h->in[i].mul;
    O.d = 2 * h->in[i].l + 1;
    O.pair_begin = np;
    for (size_t o = 0; o < h->out.size(); ++o) {
      auto it = woff.find({static_cast<int>(i), static_cast<int>(o)});
      if (it == woff.end()) continue;
      B.pairs[np++] = LinPair{h->out_off[o], it->second, h->out[o].mul, 0};
    }
    O.pair_end = np;
  }
  // backward dw: one split-K GEMM per pair
  LinDwTable& D = h->dw;
  D.n_pairs = n_pairs;
  int k = 0;
  for (const auto& kv : woff) {
    const int i = kv.first.first, o = kv.first.second;
    LinDwPair& P = D.pairs[k++];
    P.x_off = h->in_off[i];
    P.g_off = h->out_off[o];
    P.w_off = kv.second;
    P.mul_in = h->in[i].mul;
    P.mul_out = h->out[o].mul;
    P.d = 2 * h->in[i].l + 1;
    P.alpha = alpha(h->in[i].l, h->in[i].p);
  }
  *out = h;
  return ok();
}

int linear_query(linear_handle h, int key, int64_t* value) {
  if (!h || !value) return fail(SEGPOLY_E_INVALID, "null argument");
  switch (key) {
    case SEGPOLY_Q_DIM_IN: *value = h->dim_in; break;
    case SEGPOLY_Q_DIM_OUT: *value = h->dim_out; break;
    case SEGPOLY_Q_WEIGHT_NUMEL: *value = h->numel; break;
    case SEGPOLY_Q_NUM_PATHS: *value = h->dw.n_pairs; break;
    default: return fail(SEGPOLY_E_INVALID, "unknown query key");
  }
  return ok();
}

int linear_fwd(linear_handle h, const void* x, const void* w, const void* classes, int idx_dtype, int num_classes,
               int64_t n, void* out, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (classes && num_classes < 1) return fail(SEGPOLY_E_INVALID, "num_classes must be >= 1 with classes");
  if (!tiles_fit(n, h)) return fail(SEGPOLY_E_UNSUPPORTED, "too many rows for one launch");
  if (n == 0 || h->dim_out == 0) return ok();
  if (!out || (h->dim_in > 0 && !x) || (h->numel > 0 && !w)) return fail(SEGPOLY_E_INVALID, "null pointer");
  if (classes && (h->flags & SEGPOLY_VALIDATE)) {
    int st = idx_dtype == SEGPOLY_I32 ? check_classes<int32_t>(classes, n, num_classes, stream)
                                      : check_classes<int64_t>(classes, n, num_classes, stream);
    if (st != SEGPOLY_OK) return st;
  }
  LinTable t = h->fwd;
  fill_tiles(t, h->out, n);
  LinearArgs a{};
  a.x = x;
  a.w = w;
  a.cls = classes;
  a.out = out;
  a.n = n;
  a.dim_in = h->dim_in;
  a.dim_out = h->dim_out;
  a.numel = h->numel;
  a.num_classes = classes ? num_classes : 1;
  a.classes = classes ? 1 : 0;
  a.dtype = h->dtype;
  a.idx = idx_dtype;
  a.layout = h->layout;
  a.stream = stream;
  const int rc = launch_linear(a, t, false);
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int linear_bwd_workspace(linear_handle h, int64_t n, int num_classes, size_t* bytes) {
  if (!h || !bytes) return fail(SEGPOLY_E_INVALID, "null argument");
  if (n < 0 || num_classes < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  *bytes = dw_workspace_bytes(h, n, num_classes);
  return ok();
}

int linear_bwd(linear_handle h, const void* x, const void* w, const void* grad_out, const void* classes,
               int idx_dtype, int num_classes, int64_t n, void* grad_x, void* grad_w, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (classes && num_classes < 1) return fail(SEGPOLY_E_INVALID, "num_classes must be >= 1 with classes");
  if (classes && grad_w && num_classes > 65535)
    return fail(SEGPOLY_E_UNSUPPORTED, "more than 65535 classes for the weight gradient");
  if (!tiles_fit(n, h)) return fail(SEGPOLY_E_UNSUPPORTED, "too many rows for one launch");
  if (n > 0 && (!grad_x || !grad_out || (h->numel > 0 && !w) || (grad_w && h->dim_in > 0 && !x)))
    return fail(SEGPOLY_E_INVALID, "null pointer");
  LinDwTable dt = h->dw;
  const int64_t part = fill_dw_tiles(dt, n);
  const size_t need = dw_workspace_bytes(h, n, classes ? num_classes : 0);
  if (grad_w && need > 0 && (!workspace || workspace_bytes < need))
    return fail(SEGPOLY_E_INVALID, "workspace missing or smaller than linear_bwd_workspace()");
  if (classes && (h->flags & SEGPOLY_VALIDATE) && n > 0) {
    int st = idx_dtype == SEGPOLY_I32 ? check_classes<int32_t>(classes, n, num_classes, stream)
                                      : check_classes<int64_t>(classes, n, num_classes, stream);
    if (st != SEGPOLY_OK) return st;
  }
  int rc = 0;
  if (n > 0 && h->dim_in > 0) {
    LinTable t = h->bwd;
    fill_tiles(t, h->in, n);
    LinearArgs a{};
    a.x = grad_out;
    a.w = w;
    a.cls = classes;
    a.out = grad_x;
    a.n = n;
    a.dim_in = h->dim_out;
    a.dim_out = h->dim_in;
    a.numel = h->numel;
    a.num_classes = classes ? num_classes : 1;
    a.classes = classes ? 1 : 0;
    a.dtype = h->dtype;
    a.idx = idx_dtype;
    a.layout = h->layout;
    a.stream = stream;
    rc = launch_linear(a, t, true);
  }
  if (rc == 0 && grad_w && h->numel > 0) {
    const int nc = classes ? num_classes : 1;
    if (n == 0) {
      rc = launch_fill_zero(grad_w, h->numel * nc, h->dtype, stream);
    } else {
      LinearDwArgs d{};
      d.x = x;
      d.g = grad_out;
      d.cls = classes;
      d.dw = grad_w;
      d.workspace = workspace;
      d.n = n;
      d.dim_in = h->dim_in;
      d.dim_out = h->dim_out;
      d.numel = h->numel;
      d.part = part;
      d.num_classes = nc;
      d.dtype = h->dtype;
      d.idx = idx_dtype;
      d.layout = h->layout;
      d.stream = stream;
      rc = launch_linear_dw(d, dt);
    }
  }
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int linear_destroy(linear_handle h) {
  delete h;
  return ok();
}

}  // extern "C"
