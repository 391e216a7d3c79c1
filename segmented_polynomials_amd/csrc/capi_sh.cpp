// C ABI of the spherical harmonics of vectors.  Host code.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <string>

#include "capi_util.hpp"
#include "launch.hpp"
#include "segpoly.h"

using namespace segpoly;

namespace segpoly {

// N_l0 and sqrt2 N_lm, N_lm = sqrt((2l+1) (l-m)! / (l+m)!), in extended
// precision, rounded once.
const ShConsts& sh_consts() {
  static const ShConsts K = [] {
    ShConsts k{};
    for (int l = 0; l <= kShMaxL; ++l)
      for (int m = 0; m <= l; ++m) {
        long double ratio = 1.0L;  // (l-m)! / (l+m)!
        for (int i = l - m + 1; i <= l + m; ++i) ratio /= static_cast<long double>(i);
        long double v = std::sqrt(static_cast<long double>(2 * l + 1) * ratio);
        if (m > 0) v *= std::sqrt(2.0L);
        k.c[l * (l + 1) / 2 + m] = static_cast<double>(v);
      }
    return k;
  }();
  return K;
}

}  // namespace segpoly

namespace {

int sh_common(int lmax, int dtype, int64_t n) {
  if (lmax < 0 || lmax > kShMaxL) return fail(SEGPOLY_E_UNSUPPORTED, "lmax must be in [0, 6]");
  if (dtype != SEGPOLY_F32 && dtype != SEGPOLY_F64) return fail(SEGPOLY_E_INVALID, "bad dtype");
  if (n < 0) return fail(SEGPOLY_E_INVALID, "negative size");
  if (n > static_cast<int64_t>(kMaxGridX) * 128) return fail(SEGPOLY_E_UNSUPPORTED, "too many vectors");
  return SEGPOLY_OK;
}

}  // namespace

extern "C" {

int sh_fwd(int lmax, int normalize, int dtype, const void* vec, int64_t n, void* out, void* stream) {
  int st = sh_common(lmax, dtype, n);
  if (st != SEGPOLY_OK) return st;
  if (n == 0) return ok();
  if (!vec || !out) return fail(SEGPOLY_E_INVALID, "null pointer");
  ShArgs a{vec, nullptr, out, n, lmax, normalize ? 1 : 0, dtype, &sh_consts(), stream};
  const int rc = launch_sh(a);
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

int sh_bwd(int lmax, int normalize, int dtype, const void* vec, const void* grad_sh, int64_t n, void* grad_vec,
           void* stream) {
  int st = sh_common(lmax, dtype, n);
  if (st != SEGPOLY_OK) return st;
  if (n == 0) return ok();
  if (!vec || !grad_sh || !grad_vec) return fail(SEGPOLY_E_INVALID, "null pointer");
  ShArgs a{vec, grad_sh, grad_vec, n, lmax, normalize ? 1 : 0, dtype, &sh_consts(), stream};
  const int rc = launch_sh(a);
  if (rc != 0)
    return fail(SEGPOLY_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(static_cast<hipError_t>(rc)));
  return ok();
}

}  // extern "C"
