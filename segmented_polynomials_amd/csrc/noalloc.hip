// Allocation-free variant of the symmetric-contraction backward.
//
// symcon_bwd takes a caller-supplied workspace (a segment table and the
// per-chunk weight-gradient partials).  Callers that cannot allocate device
// memory on the compute path (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc) use symcon_bwd_noalloc instead: the
// same kernels, with the workspace in a fixed device array of this library.
//
// The array lives in this translation unit's code object, so the runtime
// gives every device the library runs on its own copy, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never a
// device address: the device address of each copy comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept in g_scratch; only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "capi_util.hpp"
#include "segpoly.h"

namespace {

static_assert(SEGPOLY_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

// the workspace of every symcon_bwd_noalloc call on a device
static __device__ __align__(256) unsigned char scratch[SEGPOLY_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (set up on the
// first call on that device); null with the error recorded on failure.
void* scratch_on_current_device(int* status) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = segpoly::fail(SEGPOLY_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = segpoly::fail(SEGPOLY_E_UNSUPPORTED, "device ordinal above the scratch table");
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *status = segpoly::fail(SEGPOLY_E_HIP, std::string("hipGetSymbolAddress (scratch): ") + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

namespace segpoly {
unsigned symcon_handle_flags(symcon_handle h);
}

extern "C" {

int symcon_bwd_noalloc(symcon_handle h, const void* x, const void* species, const void* species_perm, int idx_dtype,
                       const void* w, const void* grad_out, int64_t n_atoms, void* grad_x, void* grad_w,
                       void* stream) {
  if (!h) return segpoly::fail(SEGPOLY_E_INVALID, "null handle");
  if (n_atoms < 0) return segpoly::fail(SEGPOLY_E_INVALID, "negative size");
  if (segpoly::symcon_handle_flags(h) & SEGPOLY_VALIDATE)
    return segpoly::fail(SEGPOLY_E_UNSUPPORTED,
                         "VALIDATE copies the indices into host buffers; the allocation-free backward does not "
                         "validate (create the handle without it)");
  size_t need = 0;
  int st = symcon_bwd_workspace(h, n_atoms, &need);
  if (st != SEGPOLY_OK) return st;
  if (need > SEGPOLY_NOALLOC_SCRATCH_BYTES)
    return segpoly::fail(SEGPOLY_E_UNSUPPORTED,
                         "n_atoms = " + std::to_string(n_atoms) + " needs " + std::to_string(need) +
                             " bytes of workspace, above the fixed scratch of " +
                             std::to_string(static_cast<size_t>(SEGPOLY_NOALLOC_SCRATCH_BYTES)) + " bytes");
  void* ws = scratch_on_current_device(&st);
  if (!ws) return st;
  return symcon_bwd(h, x, species, species_perm, idx_dtype, w, grad_out, n_atoms, grad_x, grad_w, ws,
                    SEGPOLY_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
