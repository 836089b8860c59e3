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

// ---- layer halves for the pipeline stage (api.cpp) ----
// Where one half's saved tensors are (ATTN: a = QKV, b = O, c = log-sum-exp;
// MLP: a = U, b = Y, c unused).
struct SavedPtrs {
  void* ln_out;
  float* mean;
  float* rstd;
  void* a;
  void* b;
  float* c;
};
// Outputs of an input-gradient-only backward: dU (MLP) or dQKV (ATTN), and
// the LayerNorm's (dgamma, dbeta) partial rows.
struct DataOnly {
  void* g;
  float* lnp;
};
// Bytes of one micro-batch's copy of each saved field, of g, of the
// LayerNorm partial rows, and of one row of the widest activation.
struct SavedSizes {
  size_t ln_out, stats, a, b, c, g, lnp, widest;
};
int half_saved_sizes(const mtnlg_layer_desc* desc, int half, SavedSizes* out);
// Workspace of half_fwd and half_bwd_data (the layer backward's), and of
// half_weight_grads over mb micro-batches.
size_t half_bwd_ws_bytes(const mtnlg_layer_desc* desc, int half);
size_t half_weight_grads_ws_bytes(const mtnlg_layer_desc* desc, int half, int mb);
// The forward of a half into the saved fields S (mtnlg_layer_fwd's work).
int half_fwd(const mtnlg_layer_desc* desc, int half, const mtnlg_half_params* params, const void* x,
             void* y_partial, const SavedPtrs& S, void* ws, hipStream_t st);
// The backward of a half without its weight products and bias column sums:
// dx_partial, g_out (dU or dQKV) and the LayerNorm partial rows lnp_out.
int half_bwd_data(const mtnlg_layer_desc* desc, int half, const mtnlg_half_params* params, const void* x,
                  const SavedPtrs& S, const void* dy, void* dx_partial, void* g_out, float* lnp_out, void* ws,
                  hipStream_t st);
// The weight, bias and LayerNorm gradients of a half over mb micro-batches
// whose saved fields (S: micro-batch 0's, the rest following each field
// back to back), output gradients dy_all, g_all and partial rows lnp_all lie
// back to back: each weight gradient is one product over mb * T rows.
int half_weight_grads(const mtnlg_layer_desc* desc, int half, int mb, const SavedPtrs& S, const void* dy_all,
                      const void* g_all, const float* lnp_all, const mtnlg_half_grads* grads, void* ws,
                      hipStream_t st);

}  // namespace abi
}  // namespace mtnlg
