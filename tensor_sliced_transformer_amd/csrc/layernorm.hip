// LayerNorm forward / backward over rows, HBM-streaming (gfx950).
//
// Forward: y = gamma * (x - mean) * rstd + beta with mean and biased variance
// over the row, statistics in fp32 (mean, rstd saved for backward). One row
// at a time per workgroup, the workgroups persistent over the rows; each
// thread keeps its 8-element chunks in registers, so x is read once and y
// written once; the row's mean, then its centred sum of squares, come from
// two workgroup sums (the two-pass form of the definition).
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
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace mtnlg {

namespace {

// Eight consecutive elements kept in their storage type (one 16-byte vector
// of bf16, two of fp32) until they are used, to keep register use low.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float operator[](int e) const {
    const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ float operator[](int e) const {
    const float4& v = e < 4 ? a : b;
    const int k = e & 3;
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
};

// Sum of v over the workgroup (NT threads) through the NT/64 slots of `red`;
// every thread gets the same value (waves added in order).
template <int NT>
__device__ __forceinline__ float block_total(float v, float* red) {
  const float w = wave_sum_dpp(v);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = w;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) t += red[i];
  return t;
}

// Persistent, one workgroup per CU: workgroup b normalises rows b, b + G,
// b + 2G, ... (G workgroups). gamma and beta are loaded once and stay in
// registers; the next row's x is loaded while the current row is reduced.
// Wave sums move through DPP rather than LDS, which made the kernel a quarter
// faster than one row per workgroup with LDS shuffles (the reductions, not
// the memory traffic, bounded it). The reductions of consecutive rows use
// alternating LDS slots: a thread can only overwrite a slot after the
// barriers of the row in between, which every thread reaches only after
// reading that slot.
template <int NT, typename T, int CPT>
__global__ __launch_bounds__(NT) void ln_fwd_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                                                    const T* __restrict__ beta, float eps, T* __restrict__ y,
                                                    float* __restrict__ mean_out, float* __restrict__ rstd_out,
                                                    int64_t rows, int cols) {
  constexpr int NW = NT / kWave;
  __shared__ float red[2][2 * NW];
  const int nch = cols / 8;
  const int tid = threadIdx.x;
  const int64_t step = gridDim.x;
  Raw8<T> gv[CPT], bv[CPT], nx[CPT];
  int64_t row = blockIdx.x;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
    if (ch < nch) {
      nx[c].load(x + row * cols + ch * 8);
      gv[c].load(gamma + ch * 8);
      bv[c].load(beta + ch * 8);
    }
  }
  int parity = 0;
  for (; row < rows; row += step) {
    Raw8<T> xv[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) xv[c] = nx[c];
    if (row + step < rows) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ch = tid + c * NT;
        if (ch < nch) nx[c].load(x + (row + step) * cols + ch * 8);
      }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (tid + c * NT < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s += xv[c][e];
      }
    const float inv_cols = 1.0f / (float)cols;
    const float mu = block_total<NT>(s, red[parity]) * inv_cols;
    float m2 = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (tid + c * NT < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = xv[c][e] - mu;
          m2 += d * d;
        }
      }
    const float rs = 1.0f / sqrtf(block_total<NT>(m2, red[parity] + NW) * inv_cols + eps);
    parity ^= 1;
    T* yr = y + row * cols;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = gv[c][e] * ((xv[c][e] - mu) * rs) + bv[c][e];
        store8(yr + ch * 8, o);
      }
    }
    if (tid == 0) {
      mean_out[row] = mu;
      rstd_out[row] = rs;
    }
  }
}

// One workgroup per block of consecutive rows. gamma sits in LDS (each thread
// reads back only its own chunks), which leaves registers for loading the next
// row's gy and x while the current row is reduced; the two row sums of a row
// share one barrier (the LDS slots alternate between rows, so no second
// barrier is needed before they are reused).
template <int NT, typename T, typename G, int CPT>
__global__ __launch_bounds__(NT) void ln_bwd_kernel(const G* __restrict__ gy, const T* __restrict__ x,
                                                    const float* __restrict__ mean, const float* __restrict__ rstd,
                                                    const T* __restrict__ gamma, T* __restrict__ dx,
                                                    float* __restrict__ part, int64_t rows, int cols,
                                                    int rows_per_block) {
  constexpr int NW = NT / kWave;
  __shared__ float red[2][2 * NW];
  extern __shared__ __align__(16) char gam_lds[];  // cols elements of T
  T* sg = reinterpret_cast<T*>(gam_lds);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int nch = cols / 8;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  float dg[CPT][8], db[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * NT;
#pragma unroll
    for (int e = 0; e < 8; ++e) { dg[c][e] = 0.0f; db[c][e] = 0.0f; }
    if (ch < nch) {
      Raw8<T> g;
      g.load(gamma + ch * 8);
      *reinterpret_cast<Raw8<T>*>(sg + ch * 8) = g;
    }
  }
  const float inv_cols = 1.0f / (float)cols;
  Raw8<G> ng[CPT];
  Raw8<T> nx[CPT];
  auto load_row = [&](int64_t row) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        ng[c].load(gy + row * cols + ch * 8);
        nx[c].load(x + row * cols + ch * 8);
      }
    }
  };
  if (r0 < r1) load_row(r0);
  int parity = 0;
  for (int64_t row = r0; row < r1; ++row) {
    const float mu = mean[row], rs = rstd[row];
    float gv[CPT][8], xh[CPT][8];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gv[c][e] = ng[c][e];
        xh[c][e] = (nx[c][e] - mu) * rs;
      }
    if (row + 1 < r1) load_row(row + 1);
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        const Raw8<T> g = *reinterpret_cast<const Raw8<T>*>(sg + ch * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gh = gv[c][e] * g[e];
          sa += gh;
          sb += gh * xh[c][e];
          dg[c][e] += gv[c][e] * xh[c][e];
          db[c][e] += gv[c][e];
        }
      }
    }
    sa = wave_sum_dpp(sa);
    sb = wave_sum_dpp(sb);
    if (lane == 0) {
      red[parity][w] = sa;
      red[parity][NW + w] = sb;
    }
    __syncthreads();
    float ta = 0.0f, tb = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      ta += red[parity][i];
      tb += red[parity][NW + i];
    }
    parity ^= 1;
    const float a = ta * inv_cols, b = tb * inv_cols;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NT;
      if (ch < nch) {
        const Raw8<T> g = *reinterpret_cast<const Raw8<T>*>(sg + ch * 8);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rs * (gv[c][e] * g[e] - a - xh[c][e] * b);
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

// out[j][c] = sum_p part[p][j][c] for j < nout, rounded to T. A workgroup
// owns 128 columns (32 float4 quads) of one output row j; its 8 thread groups
// take the partials p = g, g+8, g+16, ... with independent loads, and the 8
// group sums are added in fixed order through LDS (deterministic).
constexpr int kCrQuads = 32, kCrGroups = 8;
template <typename T>
__global__ __launch_bounds__(256) void col_reduce_kernel(const float* __restrict__ part, int P, int nout,
                                                         int cols, T* __restrict__ out0, T* __restrict__ out1) {
  __shared__ float4 red[kCrGroups][kCrQuads];
  const int q = threadIdx.x % kCrQuads, g = threadIdx.x / kCrQuads;
  const int j = blockIdx.y;
  const int c4 = (blockIdx.x * kCrQuads + q) * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c4 < cols) {
    const float* base = part + (int64_t)j * cols + c4;
    const int64_t stride = (int64_t)nout * cols;
    int p = g;
    for (; p + 3 * kCrGroups < P; p += 4 * kCrGroups) {  // four loads in flight per thread
      const float4 a = *reinterpret_cast<const float4*>(base + p * stride);
      const float4 b = *reinterpret_cast<const float4*>(base + (p + kCrGroups) * stride);
      const float4 d = *reinterpret_cast<const float4*>(base + (p + 2 * kCrGroups) * stride);
      const float4 e = *reinterpret_cast<const float4*>(base + (p + 3 * kCrGroups) * stride);
      s.x += a.x + b.x + d.x + e.x;
      s.y += a.y + b.y + d.y + e.y;
      s.z += a.z + b.z + d.z + e.z;
      s.w += a.w + b.w + d.w + e.w;
    }
    for (; p < P; p += kCrGroups) {
      const float4 a = *reinterpret_cast<const float4*>(base + p * stride);
      s.x += a.x;
      s.y += a.y;
      s.z += a.z;
      s.w += a.w;
    }
  }
  red[g][q] = s;
  __syncthreads();
  if (g == 0 && c4 < cols) {
#pragma unroll
    for (int h = 1; h < kCrGroups; ++h) {
      const float4 a = red[h][q];
      s.x += a.x;
      s.y += a.y;
      s.z += a.z;
      s.w += a.w;
    }
    T* o = (j == 0 ? out0 : out1) + c4;
    o[0] = Elem<T>::from_f(s.x);
    o[1] = Elem<T>::from_f(s.y);
    o[2] = Elem<T>::from_f(s.z);
    o[3] = Elem<T>::from_f(s.w);
  }
}

// part[p][c] = sum of x[r][c] over rows r in block p (8 columns per thread,
// four independent accumulators so several rows' loads are in flight).
template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ x, int64_t rows, int cols,
                                                             int rows_per_block, float* __restrict__ part) {
  const int c8 = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c8 >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  float s[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[u][e] = 0.0f;
  int64_t r = r0;
  for (; r + 7 < r1; r += 8) {  // eight loads in flight per thread
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8(x + (r + u) * cols + c8, v[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[u & 3][e] += v[u][e];
  }
  for (; r + 3 < r1; r += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8(x + (r + u) * cols + c8, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[u][e] += v[u][e];
  }
  for (; r < r1; ++r) {
    float v[8];
    load8(x + r * cols + c8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[0][e] += v[e];
  }
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (s[0][e] + s[1][e]) + (s[2][e] + s[3][e]);
  store8(part + (int64_t)blockIdx.y * cols + c8, o);
}

int ln_cpt(int nch, int nt) { return (nch + nt - 1) / nt; }

template <int NT, typename T>
hipError_t ln_fwd_launch(int64_t rows, int cols, const void* x, const void* g, const void* b, float eps,
                         void* y, float* mean, float* rstd, hipStream_t st) {
  const int cpt = ln_cpt(cols / 8, NT);
  // one 512-thread workgroup per CU (its registers at the MT-NLG width leave
  // no room for a second)
  const unsigned grid = (unsigned)std::min<int64_t>(rows, (int64_t)device_cus() * std::max(1, 512 / NT));
#define MTNLG_LNF(C)                                                                                    \
  hipLaunchKernelGGL((ln_fwd_kernel<NT, T, C>), dim3(grid), dim3(NT), 0, st, static_cast<const T*>(x), \
                     static_cast<const T*>(g), static_cast<const T*>(b), eps, static_cast<T*>(y), mean,  \
                     rstd, rows, cols)
  if (cpt <= 1) MTNLG_LNF(1);
  else if (cpt <= 2) MTNLG_LNF(2);
  else if (cpt <= 3) MTNLG_LNF(3);
  else if (cpt <= 4) MTNLG_LNF(4);
  else if (cpt <= 5) MTNLG_LNF(5);
  else if (cpt <= 8) MTNLG_LNF(8);
  else return hipErrorInvalidValue;
#undef MTNLG_LNF
  return hipGetLastError();
}

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
  constexpr int NT = 512;
  const int cpt = ln_cpt(cols / 8, NT);
#define MTNLG_LNB(C)                                                                                  \
  hipLaunchKernelGGL((ln_bwd_kernel<NT, T, G, C>), dim3(blocks), dim3(NT), (size_t)cols * sizeof(T), st, \
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
  dim3 grid((cols + 4 * kCrQuads - 1) / (4 * kCrQuads), nout);
  hipLaunchKernelGGL(col_reduce_kernel<T>, grid, dim3(256), 0, st, part, P, nout, cols, static_cast<T*>(o0),
                     static_cast<T*>(o1));
  return hipGetLastError();
}

// 32 rows per workgroup: at 2048 rows and 10240-20480 columns that is 320-640
// workgroups, enough loads in flight to stream at close to the copy rate.
constexpr int kColsumRows = 32;

}  // namespace

hipError_t layernorm_fwd(int dtype, int64_t rows, int64_t cols, const void* x, const void* gamma,
                         const void* beta, float eps, void* y, float* mean, float* rstd, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int c = (int)cols;
  if (dtype == kBF16) {
    if (c > 8192) return ln_fwd_launch<512, bf16_t>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
    if (c > 2048) return ln_fwd_launch<256, bf16_t>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
    return ln_fwd_launch<128, bf16_t>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
  }
  if (c > 8192) return ln_fwd_launch<512, float>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
  if (c > 2048) return ln_fwd_launch<256, float>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
  return ln_fwd_launch<128, float>(rows, c, x, gamma, beta, eps, y, mean, rstd, st);
}

size_t layernorm_bwd_ws(int64_t rows, int64_t cols) {
  return (size_t)ln_bwd_blocks(rows) * 2 * cols * sizeof(float);
}

int layernorm_bwd_blocks(int64_t rows) { return rows > 0 ? ln_bwd_blocks(rows) : 0; }

hipError_t layernorm_bwd_partials(int dtype, int gy_dtype, int64_t rows, int64_t cols, const void* gy,
                                  const void* x, const float* mean, const float* rstd, const void* gamma, void* dx,
                                  float* part, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int c = (int)cols;
  const int blocks = ln_bwd_blocks(rows);
  const int rpb = (int)((rows + blocks - 1) / blocks);
  if (dtype == kBF16) {
    if (gy_dtype == kBF16)
      return ln_bwd_launch<bf16_t, bf16_t>(rows, c, gy, x, mean, rstd, gamma, dx, part, blocks, rpb, st);
    return ln_bwd_launch<bf16_t, float>(rows, c, gy, x, mean, rstd, gamma, dx, part, blocks, rpb, st);
  }
  return ln_bwd_launch<float, float>(rows, c, gy, x, mean, rstd, gamma, dx, part, blocks, rpb, st);
}

hipError_t layernorm_bwd_reduce(int dtype, int P, int64_t cols, const float* part, void* dgamma, void* dbeta,
                                hipStream_t st) {
  if (P == 0) return hipSuccess;
  if (dtype == kBF16) return col_reduce_launch<bf16_t>(part, P, 2, (int)cols, dgamma, dbeta, st);
  return col_reduce_launch<float>(part, P, 2, (int)cols, dgamma, dbeta, st);
}

hipError_t layernorm_bwd(int dtype, int gy_dtype, int64_t rows, int64_t cols, const void* gy, const void* x,
                         const float* mean, const float* rstd, const void* gamma, void* dx, void* dgamma,
                         void* dbeta, void* ws, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  float* part = static_cast<float*>(ws);
  const hipError_t e = layernorm_bwd_partials(dtype, gy_dtype, rows, cols, gy, x, mean, rstd, gamma, dx, part, st);
  if (e != hipSuccess) return e;
  return layernorm_bwd_reduce(dtype, ln_bwd_blocks(rows), cols, part, dgamma, dbeta, st);
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
