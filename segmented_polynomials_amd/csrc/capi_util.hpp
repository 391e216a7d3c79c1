// Status helpers shared by the C ABI translation units (host code).
#pragma once
#include <string>

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

constexpr int64_t kMaxGridX = 2147483647;

struct ShConsts;
// normalisation constants of the real harmonics (capi_sh.cpp)
const ShConsts& sh_consts();

}  // namespace segpoly
