// Internal host-side launchers of the gfx950 kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtnlg {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

inline size_t elem_bytes(int dtype) { return dtype == kBF16 ? 2 : 4; }

// Compute units of the current device (queried once per device and kept;
// 256 on MI355X). Used to size the GEMM's rounds of work and its persistent
// grid; 256 when no device can be queried (host-only size queries).
int device_cus();
// The persistent GEMM grid: the CU count rounded down to a multiple of the 8
// XCDs, so that every work item of a workgroup maps to the XCD it runs on.
int persistent_grid();

// ---------------------------------------------------------------- GEMM
enum GemmEpi {
  EPI_STORE = 0,       // C = acc
  EPI_BIAS = 1,        // C = acc + bias[n]
  EPI_BIAS_GELU = 2,   // C = u = acc + bias[n]; C2 = GeLU(u)
  EPI_GELU_GRAD = 3,   // C = acc * GeLU'(aux[m, n])
  EPI_BIAS_F16LO = 4   // C = acc + bias[n]; columns n < f16_cols stored as fp16, the rest as bf16
};

struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  int M, N, K;
  int64_t lda, ldb, ldc;
  const void* bias;
  void* C2;
  const void* aux;
  int epi;
  int tiles_m, tiles_n;
  // Tail split: tiles [0, nfull) (in the XCD/grouped order) are computed whole
  // by the first nfull workgroups; the last tail_tiles tiles are each split
  // tail_split ways along K (k_chunk per piece) into fp32 partials `part`
  // (tile-major, [split][tail tile][BM][BN]) that a reduce kernel sums and
  // passes through the epilogue.
  int nfull, tail_tiles, tail_split, k_chunk;
  float* part;
  int f16_cols;  // EPI_BIAS_F16LO: the leading columns kept in fp16 (a multiple of 8)
};

struct GemmPlan {
  int bm = 256, bn = 256, bk = 32;
  int tiles = 0, tail_tiles = 0, tail_split = 1;
};

GemmPlan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, bool allow_split);
size_t gemm_workspace_bytes(const GemmPlan& pl, int64_t M, int64_t N);
// a_kc: A element (m,k) at A[m*lda+k] (else A[k*lda+m]);
// b_kc: B element (k,n) at B[n*ldb+k] (else B[k*ldb+n]).
hipError_t gemm(int dtype, bool a_kc, bool b_kc, int64_t M, int64_t N, int64_t K, const void* A,
                int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int epi,
                const void* bias, void* C2, const void* aux, const GemmPlan& pl, void* ws,
                hipStream_t st, int f16_cols = 0);

// ---------------------------------------------------------------- LayerNorm
hipError_t layernorm_fwd(int dtype, int64_t rows, int64_t cols, const void* x, const void* gamma,
                         const void* beta, float eps, void* y, float* mean, float* rstd,
                         hipStream_t st);
size_t layernorm_bwd_ws(int64_t rows, int64_t cols);
// gy_dtype: element type of gy (may differ from dtype: fp32 upstream in the bf16 path).
hipError_t layernorm_bwd(int dtype, int gy_dtype, int64_t rows, int64_t cols, const void* gy,
                         const void* x, const float* mean, const float* rstd, const void* gamma,
                         void* dx, void* dgamma, void* dbeta, void* ws, hipStream_t st);
// layernorm_bwd in two steps: dx and the per-workgroup [blocks][2][cols] fp32
// partial sums of (dgamma, dbeta); then their column sums over P partial rows
// (the partials of several calls can be reduced together, rows back to back).
int layernorm_bwd_blocks(int64_t rows);
hipError_t layernorm_bwd_partials(int dtype, int gy_dtype, int64_t rows, int64_t cols, const void* gy,
                                  const void* x, const float* mean, const float* rstd, const void* gamma, void* dx,
                                  float* part, hipStream_t st);
hipError_t layernorm_bwd_reduce(int dtype, int P, int64_t cols, const float* part, void* dgamma, void* dbeta,
                                hipStream_t st);

// ---------------------------------------------------------------- attention
// Dropout on the attention probabilities (bf16 kernels; see attention_bf16.hpp
// for the mask): thr == 0 is no dropout.
struct AttnDropout {
  uint64_t seed, site;
  uint32_t thr;  // drop when the 16-bit draw is below thr
  float scale;   // 65536 / (65536 - thr)
  int head0;     // global index of the launch's head 0
};
hipError_t attention_fwd(int dtype, int batch, int seq, int heads, int head_dim, const void* qkv,
                         void* o, float* lse, const AttnDropout& drop, hipStream_t st);
size_t attention_bwd_ws(int batch, int seq, int heads);
hipError_t attention_fwd_bf16(int batch, int seq, int heads, int head_dim, const void* qkv, void* o, float* lse,
                              const AttnDropout& drop, hipStream_t st);
hipError_t attention_bwd_bf16(int batch, int seq, int heads, int head_dim, const void* qkv, const void* o,
                              const float* lse, const void* dout, void* dqkv, void* ws, const AttnDropout& drop,
                              hipStream_t st);
hipError_t attention_bwd(int dtype, int batch, int seq, int heads, int head_dim, const void* qkv,
                         const void* o, const float* lse, const void* dout, void* dqkv, void* ws,
                         const AttnDropout& drop, hipStream_t st);

// ---------------------------------------------------------------- streaming
constexpr int kMaxPartials = 16;
hipError_t reduce_partials(int dtype, int64_t rows, int64_t cols, const void* const* parts, int n,
                           const void* residual, const void* bias, void* out, hipStream_t st);
// reduce_partials with dropout on (sum + bias) before the residual is added,
// and the matching backward dz = keep * scale * dy. The keep mask comes from
// Philox4x64-10 keyed by (seed, site); thr = drop threshold on 16-bit draws.
hipError_t reduce_partials_dropout(int dtype, int64_t rows, int64_t cols, const void* const* parts, int n,
                                   const void* residual, const void* bias, void* out, uint64_t seed,
                                   uint64_t site, uint32_t thr, hipStream_t st);
hipError_t dropout_bwd(int dtype, int64_t total, const void* dy, void* dz, uint64_t seed, uint64_t site,
                       uint32_t thr, hipStream_t st);
size_t colsum_ws(int64_t rows, int64_t cols);
// out[c] = sum_r x[r, c] (x dtype, out dtype), two-stage deterministic.
hipError_t colsum(int dtype, int64_t rows, int64_t cols, const void* x, void* out, void* ws,
                  hipStream_t st);
hipError_t grad_accumulate(int64_t n, int dtype, const void* grad, float* acc, bool overwrite,
                           hipStream_t st);
size_t adam_ws(int64_t n);
struct AdamScalars {
  float lr, beta1, beta2, eps, weight_decay, max_grad_norm, inv_loss_scale;
  float inv_bc1, inv_bc2;  // 1/(1-beta1^t), 1/(1-beta2^t)
};
hipError_t adam_step(const AdamScalars& c, int64_t n, float* master, float* m, float* v,
                     const float* grad, void* w_bf16, float* stats, void* ws, hipStream_t st);
// adam_step with its norm partials in the library's static per-device scratch
// (adam_static_scratch_bytes() bytes) instead of a caller workspace: nothing is
// allocated; calls that overlap on one device share that scratch.
size_t adam_static_scratch_bytes();
hipError_t adam_step_static(const AdamScalars& c, int64_t n, float* master, float* m, float* v,
                            const float* grad, void* w_bf16, float* stats, hipStream_t st);
// The accumulation that also leaves the norm partials in ws (adam_ws bytes),
// and the Adam step that takes them from there instead of its own norm pass.
hipError_t grad_accumulate_norm(int64_t n, int dtype, const void* grad, float* acc, bool overwrite,
                                float inv_loss_scale, void* ws, hipStream_t st);
// The update's reads and writes with its arithmetic left out (values unchanged).
hipError_t adam_streams(int64_t n, float* master, float* m, float* v, const float* grad, void* w_bf16,
                        hipStream_t st);
hipError_t adam_update(const AdamScalars& c, int64_t n, float* master, float* m, float* v,
                       const float* grad, void* w_bf16, float* stats, const void* ws, hipStream_t st);
// The norm partials of a bf16 gradient read as it is (the launch and summation
// order of grad_accumulate_norm with overwrite, nothing written but the
// partials), and the update that reads that bf16 gradient instead of an fp32
// accumulator: together bit-identical to grad_accumulate_norm(overwrite) +
// adam_update, with 6 bytes per parameter less traffic.
hipError_t grad_norm_bf16(int64_t n, const void* grad, float inv_loss_scale, void* ws, hipStream_t st);
hipError_t adam_update_bf16(const AdamScalars& c, int64_t n, float* master, float* m, float* v, const void* grad,
                            void* w_bf16, float* stats, const void* ws, hipStream_t st);

}  // namespace mtnlg
