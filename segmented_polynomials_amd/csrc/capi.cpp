// C ABI of the library: handles, validation, kernel selection.  Host code.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "capi_util.hpp"
#include "cg.hpp"
#include "generic_tables.hpp"
#include "linear_tables.hpp"
#include "launch.hpp"
#include "segpoly.h"
#include "symcon_descriptor.hpp"
#include "tp_descriptor.hpp"

using namespace segpoly;

namespace segpoly {
thread_local std::string g_last_error;
}  // namespace segpoly

namespace {

constexpr size_t kGenericLdsLimit = 64 * 1024;
constexpr int64_t kMaxGrid = 2147483647;

int copy_str(const std::string& s, char* buf, size_t cap) {
  if (!buf) return fail(SEGPOLY_E_INVALID, "null buffer");
  if (cap < s.size() + 1) return fail(SEGPOLY_E_INVALID, "buffer too small: need " + std::to_string(s.size() + 1));
  std::memcpy(buf, s.c_str(), s.size() + 1);
  return ok();
}


// VALIDATE for the symmetric-contraction backward: perm is a permutation
// of the atoms with species[perm[.]] ascending.
template <typename Index>
int check_species_perm(const void* dsp, const void* dperm, int64_t n, void* stream) {
  std::vector<Index> s(n), p(n);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess && n) e = hipMemcpy(s.data(), dsp, n * sizeof(Index), hipMemcpyDeviceToHost);
  if (e == hipSuccess && n) e = hipMemcpy(p.data(), dperm, n * sizeof(Index), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SEGPOLY_E_HIP, std::string("validate copy: ") + hipGetErrorString(e));
  std::vector<char> seen(n, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t q = static_cast<int64_t>(p[i]);
    if (q < 0 || q >= n || seen[q])
      return fail(SEGPOLY_E_RANGE, "species_perm is not a permutation of the atoms (entry " + std::to_string(i) + ")");
    seen[q] = 1;
    if (i && s[q] < s[p[i - 1]])
      return fail(SEGPOLY_E_UNSORTED, "species[species_perm[.]] is not ascending at entry " + std::to_string(i));
  }
  return ok();
}

template <typename Index>
int check_species(const void* dsp, int64_t n, int num_elements, void* stream) {
  std::vector<Index> s(n);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess && n) e = hipMemcpy(s.data(), dsp, n * sizeof(Index), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SEGPOLY_E_HIP, std::string("validate copy: ") + hipGetErrorString(e));
  for (int64_t i = 0; i < n; ++i)
    if (s[i] < 0 || static_cast<int64_t>(s[i]) >= num_elements)
      return fail(SEGPOLY_E_RANGE, "species[" + std::to_string(i) + "] outside [0, num_elements)");
  return ok();
}

}  // namespace

struct segpoly_tp {
  TPDescriptor d;
  int layout = 0, dtype = 0;
  unsigned flags = 0;
  const TPSpecEntry* spec = nullptr;
  std::string kernel_name;
  std::vector<GPath> gpaths;
  std::vector<GNz> gnz;
  std::vector<GIn> gin;
  std::vector<unsigned char> blob;  // gpaths, gnz, then gin, uploaded once per device
  int max_mul = 0;
  std::mutex mu;
  std::map<int, DeviceBuffer> dev;
};

struct segpoly_symcon {
  SymconDescriptor d;
  int layout = 0, dtype = 0, num_elements = 0;
  unsigned flags = 0;
  const SymconSpecEntry* spec = nullptr;
  std::string kernel_name;
  std::vector<GTerm> gterms;
  std::vector<GBlock> gin, gout;
  std::vector<unsigned char> blob;  // gterms, gin, gout
  std::mutex mu;
  std::map<int, DeviceBuffer> dev;
};

namespace {
// Device view of a handle's uploaded tables (gpaths, gnz, gin in one blob).
GenericTPInfo generic_tp_info(const segpoly_tp* h, void* dp) {
  const size_t bp = h->gpaths.size() * sizeof(GPath), bz = h->gnz.size() * sizeof(GNz);
  unsigned char* base = static_cast<unsigned char*>(dp);
  GenericTPInfo g{};
  g.paths = reinterpret_cast<const GPath*>(base);
  g.nz = reinterpret_cast<const GNz*>(base + bp);
  g.in = reinterpret_cast<const GIn*>(base + bp + bz);
  g.np = static_cast<int>(h->gpaths.size());
  g.nk = h->d.nk;
  g.max_mul = h->max_mul;
  g.n_in = static_cast<int>(h->gin.size());
  g.nx = h->d.nx;
  g.dim1 = h->d.dim1;
  g.dim2 = h->d.dim2;
  g.dimo = h->d.dimo;
  g.numel = h->d.numel;
  return g;
}

// Device view of a symmetric contraction's uploaded tables (terms, input
// blocks, output blocks in one blob).
GenericSymconInfo generic_symcon_info(const segpoly_symcon* h, void* dp) {
  const size_t bt = h->gterms.size() * sizeof(GTerm), bi = h->gin.size() * sizeof(GBlock);
  unsigned char* base = static_cast<unsigned char*>(dp);
  GenericSymconInfo g{};
  g.terms = reinterpret_cast<const GTerm*>(base);
  g.in_blocks = reinterpret_cast<const GBlock*>(base + bt);
  g.out_blocks = reinterpret_cast<const GBlock*>(base + bt + bi);
  g.n_terms = static_cast<int>(h->gterms.size());
  g.n_in_blocks = static_cast<int>(h->gin.size());
  g.n_out_blocks = static_cast<int>(h->gout.size());
  g.nv = h->d.n;
  g.no = h->d.nout;
  g.numel = h->d.numel;
  return g;
}

int tp_conv_fwd_impl(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* vec, int normalize,
                     const void* w, const void* src, const void* dst, const void* row_ptr, int idx_dtype,
                     int64_t n_edges, int64_t n_nodes, void* out, void* stream);
}  // namespace

namespace segpoly {
// the creation flags of a handle (for the allocation-free backward in noalloc.hip)
unsigned symcon_handle_flags(symcon_handle h) { return h ? h->flags : 0u; }
}  // namespace segpoly

extern "C" {

const char* segpoly_last_error(void) { return g_last_error.c_str(); }

const char* segpoly_version(void) { return "segpoly 0.1.0 (gfx950)"; }

int segpoly_real_cg(int l1, int l2, int l3, double* out) {
  if (!out) return fail(SEGPOLY_E_INVALID, "null output");
  if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > kMaxL || l2 > kMaxL || l3 > kMaxL)
    return fail(SEGPOLY_E_UNSUPPORTED, "l outside the supported range");
  const auto& t = real_cg(l1, l2, l3);
  std::memcpy(out, t.data(), t.size() * sizeof(double));
  return ok();
}

// ------------------------------------------------------------------ TP

int tp_create(const char* in1, const char* in2, const char* outs, int layout, int dtype, unsigned flags,
              tp_handle* out) {
  if (!out) return fail(SEGPOLY_E_INVALID, "null handle pointer");
  *out = nullptr;
  if (!in1 || !in2 || !outs) return fail(SEGPOLY_E_INVALID, "null irreps string");
  if (layout != SEGPOLY_MUL_IR && layout != SEGPOLY_IR_MUL) return fail(SEGPOLY_E_INVALID, "bad layout");
  if (dtype != SEGPOLY_F32 && dtype != SEGPOLY_F64) return fail(SEGPOLY_E_INVALID, "bad dtype");
  if (flags & ~(SEGPOLY_SHARED_WEIGHTS | SEGPOLY_VALIDATE | SEGPOLY_FORCE_GENERIC | SEGPOLY_REDUCE_MEAN |
                SEGPOLY_MERGE_PATHS))
    return fail(SEGPOLY_E_INVALID, "unknown flag bits");
  segpoly_tp* h = nullptr;
  try {
    h = new segpoly_tp();
    h->d = build_tp(in1, in2, outs, (flags & SEGPOLY_MERGE_PATHS) != 0);
  } catch (const ParseError& e) {
    delete h;
    return fail(SEGPOLY_E_PARSE, e.what());
  } catch (const std::invalid_argument& e) {
    delete h;
    return fail(SEGPOLY_E_UNSUPPORTED, e.what());
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
  const unsigned bit = dtype == SEGPOLY_F32 ? 1u : 2u;
  if (!(flags & SEGPOLY_FORCE_GENERIC) && h->d.uniform_mul && h->d.mul > 0) {
    for (int i = 0; i < kNumTPSpecs; ++i)
      if ((kTPSpecs[i].dtypes & bit) && h->d.key == kTPSpecs[i].key) {
        h->spec = &kTPSpecs[i];
        break;
      }
  }
  // generic tables (merged paths share their output components)
  for (const auto& p : h->d.paths) {
    GPath g{};
    g.l1 = p.l1;
    g.lo = p.lo;
    g.mul = p.mul;
    g.nz_begin = static_cast<int>(h->gnz.size());
    for (const auto& z : p.nz) h->gnz.push_back({z.i, z.j, z.k, 0, z.c});
    g.nz_end = static_cast<int>(h->gnz.size());
    g.kcomp = p.kcomp;
    g.xcomp = p.xcomp;
    g.off1 = p.off1;
    g.off2 = p.off2;
    g.offo = p.offo;
    g.woff = p.woff;
    h->gpaths.push_back(g);
    h->max_mul = std::max(h->max_mul, p.mul);
  }
  {  // input-1 blocks (the table-driven backward writes dx block by block)
    int64_t off = 0;
    int comp = 0;
    for (const auto& r : h->d.in1) {
      h->gin.push_back({r.l, comp, r.mul, 0, off});
      off += static_cast<int64_t>(r.mul) * (2 * r.l + 1);
      comp += 2 * r.l + 1;
      h->max_mul = std::max(h->max_mul, r.mul);
    }
  }
  {
    const size_t bp = h->gpaths.size() * sizeof(GPath), bz = h->gnz.size() * sizeof(GNz),
                 bi = h->gin.size() * sizeof(GIn);
    h->blob.resize(bp + bz + bi);
    if (bp) std::memcpy(h->blob.data(), h->gpaths.data(), bp);
    if (bz) std::memcpy(h->blob.data() + bp, h->gnz.data(), bz);
    if (bi) std::memcpy(h->blob.data() + bp + bz, h->gin.data(), bi);
  }
  const size_t esz = dtype == SEGPOLY_F32 ? 4 : 8;
  if (!h->spec && static_cast<size_t>(h->d.nk) * 64 * esz > kGenericLdsLimit) {
    delete h;
    return fail(SEGPOLY_E_UNSUPPORTED, "too many output components per channel for the generic kernel");
  }
  h->kernel_name = h->spec ? std::string("tp_conv_spec_") + h->spec->name : "tp_conv_generic";
  *out = h;
  return ok();
}

int tp_query(tp_handle h, int key, int64_t* value) {
  if (!h || !value) return fail(SEGPOLY_E_INVALID, "null argument");
  const auto& d = h->d;
  switch (key) {
    case SEGPOLY_Q_DIM_IN1: *value = d.dim1; break;
    case SEGPOLY_Q_DIM_IN2: *value = d.dim2; break;
    case SEGPOLY_Q_DIM_OUT: *value = d.dimo; break;
    case SEGPOLY_Q_WEIGHT_NUMEL: *value = d.numel; break;
    case SEGPOLY_Q_NUM_PATHS: *value = static_cast<int64_t>(d.paths.size()); break;
    case SEGPOLY_Q_CG_NNZ: *value = d.cg_nnz(); break;
    case SEGPOLY_Q_SPECIALIZED: *value = h->spec ? 1 : 0; break;
    case SEGPOLY_Q_MUL: *value = d.uniform_mul ? d.mul : 0; break;
    default: return fail(SEGPOLY_E_INVALID, "unknown query key");
  }
  return ok();
}

int tp_irreps_out(tp_handle h, char* buf, size_t cap) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  return copy_str(irreps_str(h->d.out), buf, cap);
}

int tp_kernel_name(tp_handle h, char* buf, size_t cap) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  return copy_str(h->kernel_name, buf, cap);
}

int tp_path_info(tp_handle h, int p, int64_t* info) {
  if (!h || !info) return fail(SEGPOLY_E_INVALID, "null argument");
  if (p < 0 || p >= static_cast<int>(h->d.paths.size())) return fail(SEGPOLY_E_INVALID, "path index out of range");
  const auto& q = h->d.paths[p];
  int64_t v[10] = {q.b1, q.b2, q.l1, q.l2, q.lo, q.po, q.mul, q.offo, q.woff, static_cast<int64_t>(q.nz.size())};
  std::memcpy(info, v, sizeof v);
  return ok();
}

int tp_path_cg(tp_handle h, int p, double* out) {
  if (!h || !out) return fail(SEGPOLY_E_INVALID, "null argument");
  if (p < 0 || p >= static_cast<int>(h->d.paths.size())) return fail(SEGPOLY_E_INVALID, "path index out of range");
  const auto& q = h->d.paths[p];
  const int d2 = 2 * q.l2 + 1, d3 = 2 * q.lo + 1;
  std::memset(out, 0, sizeof(double) * (2 * q.l1 + 1) * d2 * d3);
  for (const auto& z : q.nz) out[(static_cast<size_t>(z.i) * d2 + z.j) * d3 + z.k] = z.c;
  return ok();
}

int tp_conv_fwd(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, const void* src,
                const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* out, void* stream) {
  return tp_conv_fwd_impl(h, x, n_src, sh, nullptr, 0, w, src, dst, nullptr, idx_dtype, n_edges, n_nodes, out,
                          stream);
}

int tp_conv_fwd_rowptr(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, const void* src,
                       const void* row_ptr, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* out,
                       void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n_nodes > 0 && !row_ptr) return fail(SEGPOLY_E_INVALID, "null row_ptr");
  if (n_edges > 0 && !src) return fail(SEGPOLY_E_INVALID, "null src");
  return tp_conv_fwd_impl(h, x, n_src, sh, nullptr, 0, w, src, nullptr, row_ptr, idx_dtype, n_edges, n_nodes, out,
                          stream);
}

int tp_rowptr_build(const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* row_ptr,
                    void* stream) {
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (n_edges < 0 || n_nodes < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (!row_ptr || (n_edges > 0 && !dst)) return fail(SEGPOLY_E_INVALID, "null buffer");
  if (idx_dtype == SEGPOLY_I32 && (n_edges > 2147483647 || n_nodes > 2147483646))
    return fail(SEGPOLY_E_UNSUPPORTED, "int32 row pointers need n_edges and n_nodes below 2^31");
  if ((n_nodes + 1 + 255) / 256 > kMaxGrid) return fail(SEGPOLY_E_UNSUPPORTED, "too many nodes for one launch");
  const int rc = launch_rowptr_build(dst, nullptr, idx_dtype, n_edges, n_nodes, row_ptr, stream);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("row pointer launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int tp_src_rowptr_build(const void* src, const void* src_perm, int idx_dtype, int64_t n_edges, int64_t n_src,
                        void* row_ptr, void* stream) {
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (n_edges < 0 || n_src < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (!row_ptr || (n_edges > 0 && (!src || !src_perm))) return fail(SEGPOLY_E_INVALID, "null buffer");
  if (idx_dtype == SEGPOLY_I32 && (n_edges > 2147483647 || n_src > 2147483646))
    return fail(SEGPOLY_E_UNSUPPORTED, "int32 row pointers need n_edges and n_src below 2^31");
  if ((n_src + 1 + 255) / 256 > kMaxGrid) return fail(SEGPOLY_E_UNSUPPORTED, "too many sources for one launch");
  const int rc = launch_rowptr_build(src, n_edges > 0 ? src_perm : nullptr, idx_dtype, n_edges, n_src, row_ptr, stream);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("row pointer launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int tp_conv_fwd_vec(tp_handle h, const void* x, int64_t n_src, const void* vec, int normalize, const void* w,
                    const void* src, const void* dst, int idx_dtype, int64_t n_edges, int64_t n_nodes, void* out,
                    void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (!h->spec) return fail(SEGPOLY_E_UNSUPPORTED, "fused harmonics need a specialised kernel for this descriptor");
  const auto& in2 = h->d.in2;
  for (size_t i = 0; i < in2.size(); ++i)
    if (in2[i].mul != 1 || in2[i].l != static_cast<int>(i) || in2[i].p != ((i % 2) ? -1 : 1))
      return fail(SEGPOLY_E_UNSUPPORTED, "input 2 is not the harmonics 0e + 1o + 2e + ... (one copy each)");
  if (in2.empty() || static_cast<int>(in2.size()) - 1 > kShMaxL)
    return fail(SEGPOLY_E_UNSUPPORTED, "harmonics degree outside [0, 6]");
  if (n_edges > 0 && !vec) return fail(SEGPOLY_E_INVALID, "null vec");
  return tp_conv_fwd_impl(h, x, n_src, nullptr, vec ? vec : reinterpret_cast<const void*>(16), normalize, w, src,
                          dst, nullptr, idx_dtype, n_edges, n_nodes, out, stream);
}

}  // extern "C"

namespace {
int tp_conv_fwd_impl(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* vec, int normalize,
                     const void* w, const void* src, const void* dst, const void* row_ptr, int idx_dtype,
                     int64_t n_edges, int64_t n_nodes, void* out, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n_src < 0 || n_edges < 0 || n_nodes < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (!row_ptr && (src == nullptr) != (dst == nullptr))
    return fail(SEGPOLY_E_INVALID, "src and dst must both be given or both be NULL");
  const auto& d = h->d;
  // NULL indices select batch mode, except that an empty edge list (whose
  // index arrays may well be NULL) always means "no edges, all rows zero"
  const bool batch = src == nullptr && n_edges > 0;
  if (batch && (n_edges != n_nodes || n_src < n_edges))
    return fail(SEGPOLY_E_INVALID, "batch mode needs n_edges == n_nodes <= n_src");
  if (n_nodes > kMaxGrid) return fail(SEGPOLY_E_UNSUPPORTED, "n_nodes must be below 2^31");
  if (n_nodes == 0 || d.dimo == 0) return ok();
  if (!out) return fail(SEGPOLY_E_INVALID, "null out");
  if (n_edges > 0) {
    if (!sh && !vec && d.dim2 > 0) return fail(SEGPOLY_E_INVALID, "null sh");
    if (!w) return fail(SEGPOLY_E_INVALID, "null w");
    if (!x && n_src > 0) return fail(SEGPOLY_E_INVALID, "null x");
  }
  if ((h->flags & SEGPOLY_VALIDATE) && !batch) {
    int st;
    if (row_ptr)
      st = idx_dtype == SEGPOLY_I32 ? check_rowptr<int32_t>(src, row_ptr, n_edges, n_src, n_nodes, stream)
                                    : check_rowptr<int64_t>(src, row_ptr, n_edges, n_src, n_nodes, stream);
    else
      st = idx_dtype == SEGPOLY_I32 ? check_indices<int32_t>(src, dst, n_edges, n_src, n_nodes, stream)
                                    : check_indices<int64_t>(src, dst, n_edges, n_src, n_nodes, stream);
    if (st != SEGPOLY_OK) return st;
  }
  TPArgs a{};
  a.x = x;
  a.sh = sh;
  a.w = w;
  a.src = src;
  a.dst = dst;
  a.row_ptr = batch ? nullptr : row_ptr;
  a.out = out;
  a.n_src = n_src;
  // without source rows no edge contributes (and x may be NULL): every
  // output row is zero, as with no edges
  a.n_edges = (!batch && n_src == 0) ? 0 : n_edges;
  a.n_nodes = n_nodes;
  a.w_stride = (h->flags & SEGPOLY_SHARED_WEIGHTS) ? 0 : d.numel;
  a.mul = d.uniform_mul ? d.mul : 0;
  a.batch = batch ? 1 : 0;
  a.mean = (h->flags & SEGPOLY_REDUCE_MEAN) ? 1 : 0;
  a.dtype = h->dtype;
  a.idx = idx_dtype;
  a.layout = h->layout;
  a.stream = stream;
  a.vec = vec;
  a.sh_normalize = normalize ? 1 : 0;
  a.sh_consts = &sh_consts();
  int rc;
  if (h->spec) {
    rc = h->spec->launch(a);
    if (rc == -2) return fail(SEGPOLY_E_UNSUPPORTED, "input 2 of this descriptor is not a harmonics set");
  } else {
    int st = SEGPOLY_OK;
    void* dp = upload(h->dev, h->mu, h->blob.data(), h->blob.size(), &st);
    if (!dp) return st;
    rc = launch_tp_generic(a, generic_tp_info(h, dp));
  }
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

}  // namespace

extern "C" {

// Messages [n_edges][DIM_IN1] (indexed mode), then 256-byte aligned the
// harmonic-gradient partials [tiles][n_edges][DIM_IN2] when one wave of
// single channels does not cover the multiplicity (tiles = ceil(mul / 64),
// the most any launch uses); in indexed mode then, 256-byte aligned, the
// sources in src_perm order [n_edges] int32; with shared weights then,
// 256-byte aligned, the per-edge weight-gradient rows [n_edges][numel] and,
// again aligned, their partial sums [ceil(n_edges / kTpDwChunk)][numel].
// `dw_off` and `keys_off` receive the offsets of the per-edge rows and keys.
static size_t tp_bwd_ws(const segpoly_tp* h, int64_t n_edges, bool batch, int64_t* dw_off,
                        int64_t* keys_off = nullptr) {
  const size_t esz = h->dtype == SEGPOLY_F32 ? 4 : 8;
  const size_t e = static_cast<size_t>(n_edges);
  if (!h->spec) {  // table-driven backward: only the shared-weight rows and their chunk sums
    if (dw_off) *dw_off = 0;
    if (!(h->flags & SEGPOLY_SHARED_WEIGHTS) || n_edges == 0) return 0;
    const size_t numel = static_cast<size_t>(h->d.numel);
    const size_t chunks = (e + kTpDwChunk - 1) / kTpDwChunk;
    return static_cast<size_t>(round_up_256(static_cast<int64_t>(e * numel * esz))) + chunks * numel * esz;
  }
  const size_t msg = static_cast<size_t>(round_up_256(static_cast<int64_t>(batch ? 0 : e * h->d.dim1 * esz)));
  const int mul = h->d.uniform_mul ? h->d.mul : 0;
  const size_t tiles = static_cast<size_t>((mul + 63) / 64);
  size_t bytes = msg + (tiles > 1 ? tiles * e * static_cast<size_t>(h->d.dim2) * esz : 0);
  if (!batch && n_edges > 0) {
    bytes = static_cast<size_t>(round_up_256(static_cast<int64_t>(bytes)));
    if (keys_off) *keys_off = static_cast<int64_t>(bytes);
    bytes += e * sizeof(int32_t);
  }
  if ((h->flags & SEGPOLY_SHARED_WEIGHTS) && n_edges > 0) {
    bytes = static_cast<size_t>(round_up_256(static_cast<int64_t>(bytes)));
    if (dw_off) *dw_off = static_cast<int64_t>(bytes);
    const size_t numel = static_cast<size_t>(h->d.numel);
    const size_t chunks = (e + kTpDwChunk - 1) / kTpDwChunk;
    bytes += static_cast<size_t>(round_up_256(static_cast<int64_t>(e * numel * esz))) + chunks * numel * esz;
  }
  return bytes;
}

int tp_conv_bwd_workspace(tp_handle h, int64_t n_edges, int batch, size_t* bytes) {
  if (!h || !bytes) return fail(SEGPOLY_E_INVALID, "null argument");
  if (n_edges < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  *bytes = tp_bwd_ws(h, n_edges, batch != 0, nullptr);
  return ok();
}

static int tp_conv_bwd_impl(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w,
                            const void* src, const void* dst, const void* src_perm, const void* row_ptr,
                            const void* src_row_ptr, int idx_dtype, int64_t n_edges, int64_t n_nodes,
                            const void* grad_out, void* grad_x, void* grad_sh, void* grad_w, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n_src < 0 || n_edges < 0 || n_nodes < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if ((src == nullptr) != (dst == nullptr) || (src == nullptr) != (src_perm == nullptr))
    return fail(SEGPOLY_E_INVALID, "src, dst and src_perm must all be given or all be NULL");
  const auto& d = h->d;
  const bool shared = (h->flags & SEGPOLY_SHARED_WEIGHTS) != 0;
  if (h->spec && !h->spec->launch_bwd)
    return fail(SEGPOLY_E_UNSUPPORTED, "backward needs a specialised kernel for this descriptor");
  if (!h->spec && tp_generic_bwd_lds(d.nx, d.dim2, h->dtype) > kGenericLdsLimit)
    return fail(SEGPOLY_E_UNSUPPORTED, "too many input-1 or input-2 components per channel for the generic backward");
  const bool batch = src == nullptr && n_edges > 0;
  if (batch && (n_edges != n_nodes || n_src < n_edges))
    return fail(SEGPOLY_E_INVALID, "batch mode needs n_edges == n_nodes <= n_src");
  if (n_nodes > kMaxGrid || n_src > kMaxGrid) return fail(SEGPOLY_E_UNSUPPORTED, "n_nodes and n_src must be below 2^31");
  if (n_src > 0 && !grad_x) return fail(SEGPOLY_E_INVALID, "null grad_x");
  if (shared && !grad_w && d.numel > 0) return fail(SEGPOLY_E_INVALID, "null grad_w");
  int64_t dw_off = 0, keys_off = 0;
  if (n_edges > 0) {
    if (!grad_w || (!grad_sh && d.dim2 > 0)) return fail(SEGPOLY_E_INVALID, "null grad_sh or grad_w");
    if (n_nodes > 0) {
      if (!sh && d.dim2 > 0) return fail(SEGPOLY_E_INVALID, "null sh");
      if (!w) return fail(SEGPOLY_E_INVALID, "null w");
      if (!x && n_src > 0) return fail(SEGPOLY_E_INVALID, "null x");
      if (!grad_out) return fail(SEGPOLY_E_INVALID, "null grad_out");
    }
    const size_t need = tp_bwd_ws(h, n_edges, batch, &dw_off, &keys_off);
    if (need && (!workspace || workspace_bytes < need))
      return fail(SEGPOLY_E_INVALID, "workspace missing or smaller than tp_conv_bwd_workspace()");
    if (need && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(SEGPOLY_E_INVALID, "workspace must be 256-byte aligned");
  }
  if ((h->flags & SEGPOLY_VALIDATE) && !batch) {
    int st = idx_dtype == SEGPOLY_I32 ? check_indices<int32_t>(src, dst, n_edges, n_src, n_nodes, stream)
                                      : check_indices<int64_t>(src, dst, n_edges, n_src, n_nodes, stream);
    if (st == SEGPOLY_OK)
      st = idx_dtype == SEGPOLY_I32 ? check_perm<int32_t>(src, src_perm, n_edges, stream)
                                    : check_perm<int64_t>(src, src_perm, n_edges, stream);
    if (st == SEGPOLY_OK && row_ptr)
      st = idx_dtype == SEGPOLY_I32
               ? check_rowptr_matches<int32_t>(dst, nullptr, row_ptr, n_edges, n_nodes, "row_ptr", stream)
               : check_rowptr_matches<int64_t>(dst, nullptr, row_ptr, n_edges, n_nodes, "row_ptr", stream);
    if (st == SEGPOLY_OK && src_row_ptr)
      st = idx_dtype == SEGPOLY_I32
               ? check_rowptr_matches<int32_t>(src, src_perm, src_row_ptr, n_edges, n_src, "src_row_ptr", stream)
               : check_rowptr_matches<int64_t>(src, src_perm, src_row_ptr, n_edges, n_src, "src_row_ptr", stream);
    if (st != SEGPOLY_OK) return st;
  }
  if (n_src == 0 && n_edges == 0 && !(shared && d.numel > 0)) return ok();
  if (!batch && n_src == 0 && n_edges > 0) {
    // no edge has a source row (x may be NULL): nothing reached the output,
    // so every weight and harmonics gradient is zero
    int rc = launch_fill_zero(grad_w, shared ? d.numel : n_edges * d.numel, h->dtype, stream);
    if (rc == 0 && d.dim2 > 0) rc = launch_fill_zero(grad_sh, n_edges * d.dim2, h->dtype, stream);
    if (rc != 0)
      return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
    return ok();
  }
  TPBwdArgs a{};
  a.x = x;
  a.sh = sh;
  a.w = w;
  a.src = src;
  a.dst = dst;
  a.perm = src_perm;
  a.row_ptr = batch ? nullptr : row_ptr;
  a.src_row_ptr = batch ? nullptr : src_row_ptr;
  a.g = grad_out;
  a.dx = grad_x;
  a.dsh = grad_sh;
  a.dw = grad_w;
  a.workspace = workspace;
  a.n_src = n_src;
  a.n_edges = n_edges;
  a.n_nodes = n_nodes;
  a.mul = d.mul;
  a.batch = batch ? 1 : 0;
  a.mean = (h->flags & SEGPOLY_REDUCE_MEAN) ? 1 : 0;
  a.shared_w = shared ? 1 : 0;
  a.dw_ws_off = dw_off;
  a.keys_ws_off = keys_off;
  a.dtype = h->dtype;
  a.idx = idx_dtype;
  a.layout = h->layout;
  a.stream = stream;
  int rc;
  if (h->spec) {
    rc = h->spec->launch_bwd(a);
  } else {
    int st = SEGPOLY_OK;
    void* dp = upload(h->dev, h->mu, h->blob.data(), h->blob.size(), &st);
    if (!dp) return st;
    rc = launch_tp_generic_bwd(a, generic_tp_info(h, dp));
  }
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int tp_conv_bwd(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, const void* src,
                const void* dst, const void* src_perm, int idx_dtype, int64_t n_edges, int64_t n_nodes,
                const void* grad_out, void* grad_x, void* grad_sh, void* grad_w, void* workspace,
                size_t workspace_bytes, void* stream) {
  return tp_conv_bwd_impl(h, x, n_src, sh, w, src, dst, src_perm, nullptr, nullptr, idx_dtype, n_edges, n_nodes,
                          grad_out, grad_x, grad_sh, grad_w, workspace, workspace_bytes, stream);
}

int tp_conv_bwd_rowptr(tp_handle h, const void* x, int64_t n_src, const void* sh, const void* w, const void* src,
                       const void* dst, const void* src_perm, const void* row_ptr, const void* src_row_ptr,
                       int idx_dtype, int64_t n_edges, int64_t n_nodes, const void* grad_out, void* grad_x,
                       void* grad_sh, void* grad_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n_edges > 0 && (!src || !dst || !src_perm))
    return fail(SEGPOLY_E_INVALID, "the row-pointer backward needs src, dst and src_perm");
  if (!row_ptr || !src_row_ptr) return fail(SEGPOLY_E_INVALID, "null row_ptr or src_row_ptr");
  return tp_conv_bwd_impl(h, x, n_src, sh, w, src, dst, src_perm, row_ptr, src_row_ptr, idx_dtype, n_edges, n_nodes,
                          grad_out, grad_x, grad_sh, grad_w, workspace, workspace_bytes, stream);
}

int tp_destroy(tp_handle h) {
  if (!h) return ok();
  free_all(h->dev);
  delete h;
  return ok();
}

// ------------------------------------------------------------------ symcon

int symcon_create(const char* s_in, const char* s_out, int max_degree, int num_elements, int layout, int dtype,
                  unsigned flags, symcon_handle* out) {
  if (!out) return fail(SEGPOLY_E_INVALID, "null handle pointer");
  *out = nullptr;
  if (!s_in || !s_out) return fail(SEGPOLY_E_INVALID, "null irreps string");
  if (layout != SEGPOLY_MUL_IR && layout != SEGPOLY_IR_MUL) return fail(SEGPOLY_E_INVALID, "bad layout");
  if (dtype != SEGPOLY_F32 && dtype != SEGPOLY_F64) return fail(SEGPOLY_E_INVALID, "bad dtype");
  if (num_elements < 1) return fail(SEGPOLY_E_INVALID, "num_elements must be >= 1");
  if (max_degree < 1 || max_degree > 3) return fail(SEGPOLY_E_UNSUPPORTED, "max_degree must be 1, 2 or 3");
  if (flags & ~(SEGPOLY_VALIDATE | SEGPOLY_FORCE_GENERIC)) return fail(SEGPOLY_E_INVALID, "unknown flag bits");
  std::vector<int> deg;
  for (int i = 1; i <= max_degree; ++i) deg.push_back(i);
  segpoly_symcon* h = nullptr;
  try {
    h = new segpoly_symcon();
    h->d = build_symcon(s_in, s_out, deg);
  } catch (const ParseError& e) {
    delete h;
    return fail(SEGPOLY_E_PARSE, e.what());
  } catch (const std::invalid_argument& e) {
    delete h;
    return fail(SEGPOLY_E_UNSUPPORTED, e.what());
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
  h->num_elements = num_elements;
  const unsigned bit = dtype == SEGPOLY_F32 ? 1u : 2u;
  // the specialised forward addresses one atom's rows (x, w, out) through
  // 32-bit buffer offsets: rows below 2 GiB
  const int64_t widest = std::max<int64_t>({static_cast<int64_t>(h->d.n), static_cast<int64_t>(h->d.nout),
                                            static_cast<int64_t>(h->d.couplings.size())});
  const bool rows_fit = static_cast<int64_t>(h->d.mul) * widest * (dtype == SEGPOLY_F32 ? 4 : 8) <= 0x7fffffff;
  if (!(flags & SEGPOLY_FORCE_GENERIC) && rows_fit)
    for (int i = 0; i < kNumSymconSpecs; ++i)
      if ((kSymconSpecs[i].dtypes & bit) && h->d.key == kSymconSpecs[i].key) {
        h->spec = &kSymconSpecs[i];
        break;
      }
  for (size_t s = 0; s < h->d.couplings.size(); ++s) {
    const auto& cp = h->d.couplings[s];
    for (const auto& t : cp.terms)
      h->gterms.push_back({t.m[0], t.m[1], t.m[2], h->d.out_comp[cp.ob] + t.M, static_cast<int>(s), 0, t.c});
  }
  for (size_t b = 0; b < h->d.in.size(); ++b) h->gin.push_back({h->d.in[b].l, h->d.in_comp[b]});
  for (size_t b = 0; b < h->d.out.size(); ++b) h->gout.push_back({h->d.out[b].l, h->d.out_comp[b]});
  {
    const size_t bt = h->gterms.size() * sizeof(GTerm), bi = h->gin.size() * sizeof(GBlock),
                 bo = h->gout.size() * sizeof(GBlock);
    h->blob.resize(bt + bi + bo);
    if (bt) std::memcpy(h->blob.data(), h->gterms.data(), bt);
    std::memcpy(h->blob.data() + bt, h->gin.data(), bi);
    std::memcpy(h->blob.data() + bt + bi, h->gout.data(), bo);
  }
  const size_t esz = dtype == SEGPOLY_F32 ? 4 : 8;
  if (!h->spec && static_cast<size_t>(h->d.n + h->d.nout) * 64 * esz > kGenericLdsLimit) {
    delete h;
    return fail(SEGPOLY_E_UNSUPPORTED, "too many components per channel for the generic kernel");
  }
  h->kernel_name = h->spec ? std::string("symcon_spec_") + h->spec->name : "symcon_generic";
  *out = h;
  return ok();
}

int symcon_query(symcon_handle h, int key, int64_t* value) {
  if (!h || !value) return fail(SEGPOLY_E_INVALID, "null argument");
  const auto& d = h->d;
  switch (key) {
    case SEGPOLY_Q_DIM_IN: *value = d.dim_in; break;
    case SEGPOLY_Q_DIM_OUT: *value = d.dim_out; break;
    case SEGPOLY_Q_WEIGHT_NUMEL: *value = d.numel; break;
    case SEGPOLY_Q_NUM_COUPLINGS: *value = static_cast<int64_t>(d.couplings.size()); break;
    case SEGPOLY_Q_NUM_TERMS: *value = d.num_terms(); break;
    case SEGPOLY_Q_SPECIALIZED: *value = h->spec ? 1 : 0; break;
    case SEGPOLY_Q_MUL: *value = d.mul; break;
    case SEGPOLY_Q_NUM_ELEMENTS: *value = h->num_elements; break;
    case SEGPOLY_Q_NUM_MONOMIALS: *value = d.num_monomial_products(); break;
    default: return fail(SEGPOLY_E_INVALID, "unknown query key");
  }
  return ok();
}

int symcon_coupling_info(symcon_handle h, int c, int64_t* info) {
  if (!h || !info) return fail(SEGPOLY_E_INVALID, "null argument");
  if (c < 0 || c >= static_cast<int>(h->d.couplings.size())) return fail(SEGPOLY_E_INVALID, "coupling index out of range");
  const auto& cp = h->d.couplings[c];
  int64_t v[4] = {cp.nu, cp.ob, cp.k, cp.L};
  std::memcpy(info, v, sizeof v);
  return ok();
}

int symcon_coupling_dense(symcon_handle h, int c, double* out) {
  if (!h || !out) return fail(SEGPOLY_E_INVALID, "null argument");
  if (c < 0 || c >= static_cast<int>(h->d.couplings.size())) return fail(SEGPOLY_E_INVALID, "coupling index out of range");
  const auto& cp = h->d.couplings[c];
  std::memcpy(out, cp.dense.data(), cp.dense.size() * sizeof(double));
  return ok();
}

int symcon_fwd(symcon_handle h, const void* x, const void* species, int idx_dtype, const void* w, int64_t n_atoms,
               void* out, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n_atoms < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (n_atoms > kMaxGrid) return fail(SEGPOLY_E_UNSUPPORTED, "n_atoms must be below 2^31");
  if (n_atoms == 0 || h->d.dim_out == 0) return ok();
  if (!x || !species || !w || !out) return fail(SEGPOLY_E_INVALID, "null pointer");
  if (h->flags & SEGPOLY_VALIDATE) {
    int st = idx_dtype == SEGPOLY_I32 ? check_species<int32_t>(species, n_atoms, h->num_elements, stream)
                                      : check_species<int64_t>(species, n_atoms, h->num_elements, stream);
    if (st != SEGPOLY_OK) return st;
  }
  SymconArgs a{};
  a.x = x;
  a.species = species;
  a.w = w;
  a.out = out;
  a.n_atoms = n_atoms;
  a.num_elements = h->num_elements;
  a.mul = h->d.mul;
  a.dtype = h->dtype;
  a.idx = idx_dtype;
  a.layout = h->layout;
  a.stream = stream;
  int rc;
  if (h->spec) {
    rc = h->spec->launch(a);
  } else {
    int st = SEGPOLY_OK;
    void* dp = upload(h->dev, h->mu, h->blob.data(), h->blob.size(), &st);
    if (!dp) return st;
    rc = launch_symcon_generic(a, generic_symcon_info(h, dp));
  }
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int symcon_bwd_workspace(symcon_handle h, int64_t n_atoms, size_t* bytes) {
  if (!h || !bytes) return fail(SEGPOLY_E_INVALID, "null argument");
  if (n_atoms < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (!h->spec) {  // the table-driven backward needs no workspace
    *bytes = 0;
    return ok();
  }
  const size_t esz = h->dtype == SEGPOLY_F32 ? 4 : 8;
  const size_t table = static_cast<size_t>(symcon_bwd_table_bytes(h->num_elements));
  const size_t chunks = static_cast<size_t>(symcon_bwd_max_chunks(n_atoms, h->num_elements));
  *bytes = table + chunks * static_cast<size_t>(h->d.numel) * esz;
  return ok();
}

int symcon_bwd(symcon_handle h, const void* x, const void* species, const void* species_perm, int idx_dtype,
               const void* w, const void* grad_out, int64_t n_atoms, void* grad_x, void* grad_w, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!h) return fail(SEGPOLY_E_INVALID, "null handle");
  if (n_atoms < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (h->spec && !h->spec->launch_bwd)
    return fail(SEGPOLY_E_UNSUPPORTED, "backward needs a specialised kernel for this descriptor");
  const int nseg = static_cast<int>(h->d.couplings.size());
  if (!h->spec && symcon_generic_bwd_lds(h->d.n, h->d.nout, nseg, h->dtype) > kGenericLdsLimit)
    return fail(SEGPOLY_E_UNSUPPORTED, "too many components or couplings per channel for the generic backward");
  if (n_atoms > kMaxGrid) return fail(SEGPOLY_E_UNSUPPORTED, "n_atoms must be below 2^31");
  if (!grad_w) return fail(SEGPOLY_E_INVALID, "null grad_w");
  if (n_atoms > 0 && (!x || !species || !species_perm || !w || !grad_out || !grad_x))
    return fail(SEGPOLY_E_INVALID, "null pointer");
  size_t need = 0;
  symcon_bwd_workspace(h, n_atoms, &need);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SEGPOLY_E_INVALID, "workspace missing or smaller than symcon_bwd_workspace()");
  if (need && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SEGPOLY_E_INVALID, "workspace must be 256-byte aligned");
  if ((h->flags & SEGPOLY_VALIDATE) && n_atoms > 0) {
    int st = idx_dtype == SEGPOLY_I32 ? check_species<int32_t>(species, n_atoms, h->num_elements, stream)
                                      : check_species<int64_t>(species, n_atoms, h->num_elements, stream);
    if (st == SEGPOLY_OK)
      st = idx_dtype == SEGPOLY_I32 ? check_species_perm<int32_t>(species, species_perm, n_atoms, stream)
                                    : check_species_perm<int64_t>(species, species_perm, n_atoms, stream);
    if (st != SEGPOLY_OK) return st;
  }
  SymconBwdArgs a{};
  a.x = x;
  a.species = species;
  a.perm = species_perm;
  a.w = w;
  a.g = grad_out;
  a.dx = grad_x;
  a.dw = grad_w;
  a.workspace = workspace;
  a.n_atoms = n_atoms;
  a.num_elements = h->num_elements;
  a.mul = h->d.mul;
  a.dtype = h->dtype;
  a.idx = idx_dtype;
  a.layout = h->layout;
  a.stream = stream;
  int rc;
  if (h->spec) {
    rc = h->spec->launch_bwd(a);
  } else {
    int st = SEGPOLY_OK;
    void* dp = upload(h->dev, h->mu, h->blob.data(), h->blob.size(), &st);
    if (!dp) return st;
    rc = launch_symcon_generic_bwd(a, generic_symcon_info(h, dp));
  }
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int symcon_destroy(symcon_handle h) {
  if (!h) return ok();
  free_all(h->dev);
  delete h;
  return ok();
}

}  // extern "C"
