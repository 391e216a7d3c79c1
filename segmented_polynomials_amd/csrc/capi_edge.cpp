// C ABI of the edge-embedding assembly of the convolution layer.  Host code.
#include <hip/hip_runtime_api.h>

#include <string>

#include "capi_util.hpp"
#include "edge_scalars.hpp"
#include "segpoly.h"

using namespace segpoly;

namespace {

int common(int dtype, int idx_dtype, int64_t d_emb, int64_t d_src, int64_t d_dst, int64_t n_edges, int64_t n_src,
           int64_t n_dst) {
  if (dtype != SEGPOLY_F32 && dtype != SEGPOLY_F64) return fail(SEGPOLY_E_INVALID, "bad dtype");
  if (idx_dtype != SEGPOLY_I32 && idx_dtype != SEGPOLY_I64) return fail(SEGPOLY_E_INVALID, "bad index dtype");
  if (d_emb < 0 || d_src < 0 || d_dst < 0 || n_edges < 0 || n_src < 0 || n_dst < 0)
    return fail(SEGPOLY_E_INVALID, "negative size");
  if (n_edges > 4 * kMaxGridX || n_src > kMaxGridX || n_dst > kMaxGridX)
    return fail(SEGPOLY_E_UNSUPPORTED, "too many rows for one launch");
  return SEGPOLY_OK;
}

}  // namespace

extern "C" {

int edge_scalars_fwd(int dtype, const void* edge_emb, int64_t d_emb, const void* src_scalars, int64_t d_src,
                     const void* dst_scalars, int64_t d_dst, const void* src, const void* dst, int idx_dtype,
                     int64_t n_edges, int64_t n_src, int64_t n_dst, void* out, void* stream) {
  int rc = common(dtype, idx_dtype, d_emb, d_src, d_dst, n_edges, n_src, n_dst);
  if (rc) return rc;
  if (n_edges == 0 || d_emb + d_src + d_dst == 0) return ok();
  if (!out || (d_emb && !edge_emb) || (d_src && (!src || (n_src && !src_scalars))) ||
      (d_dst && (!dst || (n_dst && !dst_scalars))))
    return fail(SEGPOLY_E_INVALID, "null buffer");
  EdgeScalarArgs a{};
  a.emb = edge_emb, a.ssc = src_scalars, a.dsc = dst_scalars, a.src = src, a.dst = dst, a.out = out;
  a.d_emb = d_emb, a.d_src = d_src, a.d_dst = d_dst, a.n_edges = n_edges, a.n_src = n_src, a.n_dst = n_dst;
  a.dtype = dtype, a.idx = idx_dtype, a.stream = stream;
  rc = launch_edge_scalars(a, false);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("edge scalars launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int edge_scalars_bwd(int dtype, const void* grad_out, int64_t d_emb, int64_t d_src, int64_t d_dst, const void* src,
                     const void* dst, const void* src_perm, int idx_dtype, int64_t n_edges, int64_t n_src,
                     int64_t n_dst, void* grad_emb, void* grad_src, void* grad_dst, void* stream) {
  int rc = common(dtype, idx_dtype, d_emb, d_src, d_dst, n_edges, n_src, n_dst);
  if (rc) return rc;
  if ((d_emb && n_edges && !grad_emb) || (d_src && n_src && !grad_src) || (d_dst && n_dst && !grad_dst))
    return fail(SEGPOLY_E_INVALID, "null gradient buffer");
  if (n_edges && !grad_out && d_emb + d_src + d_dst) return fail(SEGPOLY_E_INVALID, "null grad_out");
  if (d_src && n_src && n_edges && (!src || !src_perm)) return fail(SEGPOLY_E_INVALID, "null src or src_perm");
  if (d_dst && n_dst && n_edges && !dst) return fail(SEGPOLY_E_INVALID, "null dst");
  EdgeScalarArgs a{};
  a.g = grad_out, a.src = src, a.dst = dst, a.perm = src_perm;
  a.gemb = grad_emb, a.gsrc = grad_src, a.gdst = grad_dst;
  a.d_emb = d_emb, a.d_src = d_src, a.d_dst = d_dst, a.n_edges = n_edges, a.n_src = n_src, a.n_dst = n_dst;
  a.dtype = dtype, a.idx = idx_dtype, a.stream = stream;
  rc = launch_edge_scalars(a, true);
  if (rc) return fail(SEGPOLY_E_HIP, std::string("edge scalars launch: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

}  // extern "C"
