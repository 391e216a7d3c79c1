// Status helpers shared by the C ABI translation units (host code).
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "segpoly.h"

namespace segpoly {

// message of the last failure on this thread (segpoly_last_error)
extern thread_local std::string g_last_error;

inline int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

inline int ok() {
  g_last_error.clear();
  return SEGPOLY_OK;
}

// Coefficient tables kept on each device a handle has run on.
struct DeviceBuffer {
  void* ptr = nullptr;
};

// Upload `bytes` of host data once per device; returns the device pointer
// or null (error set) on failure.
inline void* upload(std::map<int, DeviceBuffer>& cache, std::mutex& mu, const void* host, size_t bytes, int* status) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = fail(SEGPOLY_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> g(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second.ptr;
  void* p = nullptr;
  e = hipMalloc(&p, bytes ? bytes : 16);
  if (e != hipSuccess) {
    *status = fail(SEGPOLY_E_OOM, std::string("hipMalloc (coefficient table): ") + hipGetErrorString(e));
    return nullptr;
  }
  if (bytes) {
    e = hipMemcpy(p, host, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(p);
      *status = fail(SEGPOLY_E_HIP, std::string("hipMemcpy (coefficient table): ") + hipGetErrorString(e));
      return nullptr;
    }
  }
  cache[dev].ptr = p;
  return p;
}

inline void free_all(std::map<int, DeviceBuffer>& cache) {
  int cur = 0;
  bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : cache) {
    if (hipSetDevice(kv.first) == hipSuccess) (void)hipFree(kv.second.ptr);
  }
  if (have) (void)hipSetDevice(cur);
  cache.clear();
}

// Host-side index checks of the VALIDATE flag (synchronises the stream).
template <typename Index>
inline int check_indices(const void* dsrc, const void* ddst, int64_t n_edges, int64_t n_src, int64_t n_nodes,
                  void* stream) {
  std::vector<Index> s(n_edges), d(n_edges);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess && n_edges) e = hipMemcpy(s.data(), dsrc, n_edges * sizeof(Index), hipMemcpyDeviceToHost);
  if (e == hipSuccess && n_edges) e = hipMemcpy(d.data(), ddst, n_edges * sizeof(Index), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SEGPOLY_E_HIP, std::string("validate copy: ") + hipGetErrorString(e));
  for (int64_t i = 0; i < n_edges; ++i) {
    if (s[i] < 0 || static_cast<int64_t>(s[i]) >= n_src)
      return fail(SEGPOLY_E_RANGE, "src[" + std::to_string(i) + "] = " + std::to_string(s[i]) + " outside [0, n_src)");
    if (d[i] < 0 || static_cast<int64_t>(d[i]) >= n_nodes)
      return fail(SEGPOLY_E_RANGE, "dst[" + std::to_string(i) + "] = " + std::to_string(d[i]) + " outside [0, n_nodes)");
    if (i && d[i] < d[i - 1])
      return fail(SEGPOLY_E_UNSORTED, "dst is not sorted ascending at edge " + std::to_string(i));
  }
  return ok();
}

// VALIDATE with row pointers instead of dst: sources in range, rp[0] = 0,
// rp non-decreasing, rp[n_nodes] = n_edges.
template <typename Index>
inline int check_rowptr(const void* dsrc, const void* drp, int64_t n_edges, int64_t n_src, int64_t n_nodes,
                        void* stream) {
  std::vector<Index> s(n_edges), r(n_nodes + 1);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess && n_edges) e = hipMemcpy(s.data(), dsrc, n_edges * sizeof(Index), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(r.data(), drp, (n_nodes + 1) * sizeof(Index), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SEGPOLY_E_HIP, std::string("validate copy: ") + hipGetErrorString(e));
  for (int64_t i = 0; i < n_edges; ++i)
    if (s[i] < 0 || static_cast<int64_t>(s[i]) >= n_src)
      return fail(SEGPOLY_E_RANGE, "src[" + std::to_string(i) + "] = " + std::to_string(s[i]) + " outside [0, n_src)");
  if (r[0] != 0 || static_cast<int64_t>(r[n_nodes]) != n_edges)
    return fail(SEGPOLY_E_RANGE, "row_ptr must start at 0 and end at n_edges");
  for (int64_t n = 0; n < n_nodes; ++n)
    if (r[n + 1] < r[n]) return fail(SEGPOLY_E_UNSORTED, "row_ptr decreases at node " + std::to_string(n));
  return ok();
}

// VALIDATE for the backward: perm is a permutation of the edges with
// src[perm[.]] ascending.
template <typename Index>
inline int check_perm(const void* dsrc, const void* dperm, int64_t n_edges, void* stream) {
  std::vector<Index> s(n_edges), p(n_edges);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess && n_edges) e = hipMemcpy(s.data(), dsrc, n_edges * sizeof(Index), hipMemcpyDeviceToHost);
  if (e == hipSuccess && n_edges) e = hipMemcpy(p.data(), dperm, n_edges * sizeof(Index), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SEGPOLY_E_HIP, std::string("validate copy: ") + hipGetErrorString(e));
  std::vector<char> seen(n_edges, 0);
  for (int64_t i = 0; i < n_edges; ++i) {
    const int64_t q = static_cast<int64_t>(p[i]);
    if (q < 0 || q >= n_edges || seen[q])
      return fail(SEGPOLY_E_RANGE, "src_perm is not a permutation of the edges (entry " + std::to_string(i) + ")");
    seen[q] = 1;
    if (i && s[q] < s[p[i - 1]])
      return fail(SEGPOLY_E_UNSORTED, "src[src_perm[.]] is not ascending at entry " + std::to_string(i));
  }
  return ok();
}

// VALIDATE for the backward's row pointers: rp[n] is the first position i
// with key(i) >= n, key(i) = keys[i], or keys[perm[i]] when perm is given
// (dst and src_perm have been checked already).
template <typename Index>
inline int check_rowptr_matches(const void* dkeys, const void* dperm, const void* drp, int64_t n_edges, int64_t n,
                                const char* what, void* stream) {
  std::vector<Index> k(n_edges), p(dperm ? n_edges : 0), r(n + 1);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess && n_edges) e = hipMemcpy(k.data(), dkeys, n_edges * sizeof(Index), hipMemcpyDeviceToHost);
  if (e == hipSuccess && dperm && n_edges)
    e = hipMemcpy(p.data(), dperm, n_edges * sizeof(Index), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(r.data(), drp, (n + 1) * sizeof(Index), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SEGPOLY_E_HIP, std::string("validate copy: ") + hipGetErrorString(e));
  int64_t i = 0;
  for (int64_t v = 0; v <= n; ++v) {
    while (i < n_edges && static_cast<int64_t>(k[dperm ? static_cast<int64_t>(p[i]) : i]) < v) ++i;
    if (static_cast<int64_t>(r[v]) != i)
      return fail(SEGPOLY_E_RANGE, std::string(what) + "[" + std::to_string(v) + "] does not match the indices");
  }
  return ok();
}

constexpr int64_t kMaxGridX = 2147483647;

struct ShConsts;
// normalisation constants of the real harmonics (capi_sh.cpp)
const ShConsts& sh_consts();

}  // namespace segpoly
