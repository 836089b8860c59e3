// Host-side helpers of the C ABI: the thread-local error text, status
// returns, pointer checks, and the Adam argument validation shared by the
// entry points in api.cpp and stage.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/mtnlg.h"
#include "kernels.hpp"

namespace mtnlg {
namespace abi {

inline thread_local char g_last_error[512] = "";

inline int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
inline int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

inline int hip_fail(hipError_t e, const char* what) {
  return fail(MTNLG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MTNLG_HIP(call, what)                            \
  do {                                                   \
    hipError_t e_ = (call);                              \
    if (e_ != hipSuccess) return hip_fail(e_, what);     \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int check_ptr(const void* p, const char* name) {
  if (!p) return fail(MTNLG_ERR_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(MTNLG_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MTNLG_OK;
}

#define CHECK_PTR(p)                               \
  do {                                             \
    int s_ = check_ptr((p), #p);                   \
    if (s_ != MTNLG_OK) return s_;                 \
  } while (0)

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Validates an Adam step's arguments (cfg ranges, pointers, workspace size for
// n parameters; no workspace check when ws is kNoWorkspace) and fills the
// device scalars; MTNLG_OK or a failure status.
inline const void* const kNoWorkspace = reinterpret_cast<const void*>(~uintptr_t(0));
int adam_args(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v, const float* grad,
              void* w_bf16, float* stats, const void* ws, size_t ws_bytes, AdamScalars* c);

}  // namespace abi
}  // namespace mtnlg
