// LayerNorm forward / backward over rows, HBM-streaming (gfx950).
//
// Forward: y = gamma * (x - mean) * rstd + beta with mean and biased variance
// over the row, statistics in fp32 (mean, rstd saved for backward). One row
// per workgroup; each thread keeps its 8-element chunks in registers, so x is
// read once and y written once.
//
// Backward on an upstream gradient gy (linear in gy, so a tensor slice may
// apply it to its own partial): with gh = gy * gamma and xhat recomputed from
// x, mean, rstd,
//   dx = rstd * (gh - mean(gh) - xhat * mean(gh * xhat)),
//   dgamma = sum_rows gy * xhat, dbeta = sum_rows gy.
// A workgroup walks a contiguous block of rows; every thread owns the same
// columns in each row, so it accumulates its dgamma/dbeta share in registers
// and writes one fp32 partial row per workgroup; a column reduction in fixed
// order finishes them (deterministic, no atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace mtnlg {

namespace {

template <int NT, typename T, int CPT>
__global__ __launch_bounds__(NT) void ln_fwd_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                                                    const T* __restrict__ beta, float eps, T* __restrict__ y,
                                                    float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                    int cols) {
  __shared__ float red[NT / kWave];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * cols;
  const int nch = cols / 8;
  const int tid = threadIdx.x;
  float v[CPT][8];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
    if (ch < nch) {
      load8(xr + ch * 8, v[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[c][e];
    }
  }
  const float mu = block_sum<NT>(s, red) / (float)cols;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[c][e] - mu;
        q += d * d;
      }
    }
  }
  const float var = block_sum<NT>(q, red) / (float)cols;
  const float rs = 1.0f / sqrtf(var + eps);
  T* yr = y + row * cols;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
    if (ch < nch) {
      float g[8], b[8], o[8];
      load8(gamma + ch * 8, g);
      load8(beta + ch * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = g[e] * ((v[c][e] - mu) * rs) + b[e];
      store8(yr + ch * 8, o);
    }
  }
  if (tid == 0) {
    mean_out[row] = mu;
    rstd_out[row] = rs;
  }
}

template <int NT, typename T, typename G, int CPT>
__global__ __launch_bounds__(NT) void ln_bwd_kernel(const G* __restrict__ gy, const T* __restrict__ x,
                                                    const float* __restrict__ mean, const float* __restrict__ rstd,
                                                    const T* __restrict__ gamma, T* __restrict__ dx,
                                                    float* __restrict__ part, int64_t rows, int cols,
                                                    int rows_per_block) {
  __shared__ float red[NT / kWave];
  const int tid = threadIdx.x;
  const int nch = cols / 8;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  float gam[CPT][8];
  float dg[CPT][8], db[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
#pragma unroll
    for (int e = 0; e < 8; ++e) { dg[c][e] = 0.0f; db[c][e] = 0.0f; gam[c][e] = 0.0f; }
    if (ch < nch) load8(gamma + ch * 8, gam[c]);
  }
  const float inv_cols = 1.0f / (float)cols;
  for (int64_t row = r0; row < r1; ++row) {
    const float mu = mean[row], rs = rstd[row];
    float gv[CPT][8], xh[CPT][8];
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        load8(gy + row * cols + ch * 8, gv[c]);
        load8(x + row * cols + ch * 8, xh[c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[c][e] = (xh[c][e] - mu) * rs;
          const float gh = gv[c][e] * gam[c][e];
          sa += gh;
          sb += gh * xh[c][e];
          dg[c][e] += gv[c][e] * xh[c][e];
          db[c][e] += gv[c][e];
        }
      }
    }
    const float a = block_sum<NT>(sa, red) * inv_cols;
    const float b = block_sum<NT>(sb, red) * inv_cols;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rs * (gv[c][e] * gam[c][e] - a - xh[c][e] * b);
        store8(dx + row * cols + ch * 8, o);
      }
    }
  }
  // partial row of this workgroup: part[blk][0][cols] = dgamma, part[blk][1][cols] = dbeta
  float* pg = part + (int64_t)blockIdx.x * 2 * cols;
  float* pb = pg + cols;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
    if (ch < nch) {
      store8(pg + ch * 8, dg[c]);
      store8(pb + ch * 8, db[c]);
    }
  }
}

// out[j][c] = sum_p part[p][j][c] for j < nout (fixed order over p), rounded to T.
template <typename T>
__global__ __launch_bounds__(256) void col_reduce_kernel(const float* __restrict__ part, int P, int nout,
                                                         int cols, T* __restrict__ out0, T* __restrict__ out1) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int j = blockIdx.y;
  if (c >= cols || j >= nout) return;
  float s = 0.0f;
  for (int p = 0; p < P; ++p) s += part[((int64_t)p * nout + j) * cols + c];
  (j == 0 ? out0 : out1)[c] = Elem<T>::from_f(s);
}

// part[p][c] = sum of x[r][c] over rows r in block p (8 columns per thread).
template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ x, int64_t rows, int cols,
                                                             int rows_per_block, float* __restrict__ part) {
  const int c8 = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c8 >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t r = r0; r < r1; ++r) {
    float v[8];
    load8(x + r * cols + c8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += v[e];
  }
  store8(part + (int64_t)blockIdx.y * cols + c8, s);
}

int ln_cpt(int nch, int nt) { return (nch + nt - 1) / nt; }

template <int NT, typename T>
hipError_t ln_fwd_launch(int64_t rows, int cols, const void* x, const void* g, const void* b, float eps,
                         void* y, float* mean, float* rstd, hipStream_t st) {
  const int cpt = ln_cpt(cols / 8, NT);
#define MTNLG_LNF(C)                                                                                    \
  hipLaunchKernelGGL((ln_fwd_kernel<NT, T, C>), dim3(rows), dim3(NT), 0, st, static_cast<const T*>(x), \
                     static_cast<const T*>(g), static_cast<const T*>(b), eps, static_cast<T*>(y), mean,  \
                     rstd, cols)
  if (cpt <= 1) MTNLG_LNF(1);
  else if (cpt <= 2) MTNLG_LNF(2);
  else if (cpt <= 4) MTNLG_LNF(4);
  else if (cpt <= 6) MTNLG_LNF(6);
  else if (cpt <= 8) MTNLG_LNF(8);
  else if (cpt <= 10) MTNLG_LNF(10);
  else if (cpt <= 16) MTNLG_LNF(16);
  else return hipErrorInvalidValue;
#undef MTNLG_LNF
  return hipGetLastError();
}

constexpr int kLnBwdThreads = 512;

int ln_bwd_blocks(int64_t rows) {
  // about one workgroup per CU; each walks a contiguous range of rows
  const int64_t target = 256;
  const int64_t rpb = (rows + target - 1) / target;
  return (int)((rows + rpb - 1) / rpb);
}

template <typename T, typename G>
hipError_t ln_bwd_launch(int64_t rows, int cols, const void* gy, const void* x, const float* mean,
                         const float* rstd, const void* gamma, void* dx, float* part, int blocks,
                         int rpb, hipStream_t st) {
  constexpr int NT = kLnBwdThreads;
  const int cpt = ln_cpt(cols / 8, NT);
#define MTNLG_LNB(C)                                                                                  \
  hipLaunchKernelGGL((ln_bwd_kernel<NT, T, G, C>), dim3(blocks), dim3(NT), 0, st,                    \
                     static_cast<const G*>(gy), static_cast<const T*>(x), mean, rstd,                \
                     static_cast<const T*>(gamma), static_cast<T*>(dx), part, rows, cols, rpb)
  if (cpt <= 1) MTNLG_LNB(1);
  else if (cpt <= 2) MTNLG_LNB(2);
  else if (cpt <= 3) MTNLG_LNB(3);
  else if (cpt <= 5) MTNLG_LNB(5);
  else if (cpt <= 8) MTNLG_LNB(8);
  else return hipErrorInvalidValue;
#undef MTNLG_LNB
  return hipGetLastError();
}

template <typename T>
hipError_t col_reduce_launch(const float* part, int P, int nout, int cols, void* o0, void* o1, hipStream_t st) {
  dim3 grid((cols + 255) / 256, nout);
  hipLaunchKernelGGL(col_reduce_kernel<T>, grid, dim3(256), 0, st, part, P, nout, cols, static_cast<T*>(o0),
                     static_cast<T*>(o1));
  return hipGetLastError();
}

constexpr int kColsumRows = 64;

}  // namespace

hipError_t layernorm_fwd(int dtype, int64_t rows, int64_t cols, const void* x, const void* gamma,
                         const void* beta, float eps, void* y, float* mean, float* rstd, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int c = (int)cols;
  if (dtype == kBF16) {
    if (c >= 8192) return ln_fwd_launch<256, bf16_t>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
    return ln_fwd_launch<128, bf16_t>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
  }
  if (c >= 8192) return ln_fwd_launch<256, float>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
  return ln_fwd_launch<128, float>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
}

size_t layernorm_bwd_ws(int64_t rows, int64_t cols) {
  return (size_t)ln_bwd_blocks(rows) * 2 * cols * sizeof(float);
}

hipError_t layernorm_bwd(int dtype, int gy_dtype, int64_t rows, int64_t cols, const void* gy, const void* x,
                         const float* mean, const float* rstd, const void* gamma, void* dx, void* dgamma,
                         void* dbeta, void* ws, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int c = (int)cols;
  const int blocks = ln_bwd_blocks(rows);
  const int rpb = (int)((rows + blocks - 1) / blocks);
  float* part = static_cast<float*>(ws);
  hipError_t e;
  if (dtype == kBF16) {
    if (gy_dtype == kBF16)
      e = ln_bwd_launch<bf16_t, bf16_t>(rows, c, gy, x, mean, rstd, gamma, dx, part, blocks, rpb, st);
    else
      e = ln_bwd_launch<bf16_t, float>(rows, c, gy, x, mean, rstd, gamma, dx, part, blocks, rpb, st);
  } else {
    e = ln_bwd_launch<float, float>(rows, c, gy, x, mean, rstd, gamma, dx, part, blocks, rpb, st);
  }
  if (e != hipSuccess) return e;
  if (dtype == kBF16) return col_reduce_launch<bf16_t>(part, blocks, 2, c, dgamma, dbeta, st);
  return col_reduce_launch<float>(part, blocks, 2, c, dgamma, dbeta, st);
}

size_t colsum_ws(int64_t rows, int64_t cols) {
  const int64_t P = (rows + kColsumRows - 1) / kColsumRows;
  return (size_t)P * cols * sizeof(float);
}

hipError_t colsum(int dtype, int64_t rows, int64_t cols, const void* x, void* out, void* ws, hipStream_t st) {
  const int c = (int)cols;
  const int P = (int)((rows + kColsumRows - 1) / kColsumRows);
  float* part = static_cast<float*>(ws);
  dim3 grid((c / 8 + 255) / 256, P);
  if (P == 0) return hipErrorInvalidValue;
  if (dtype == kBF16) {
    hipLaunchKernelGGL(colsum_partial_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(x),
                       rows, c, kColsumRows, part);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    return col_reduce_launch<bf16_t>(part, P, 1, c, out, out, st);
  }
  hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), rows,
                     c, kColsumRows, part);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return col_reduce_launch<float>(part, P, 1, c, out, out, st);
}

}  // namespace mtnlg
