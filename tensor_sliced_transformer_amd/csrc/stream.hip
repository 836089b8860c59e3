// HBM-streaming kernels (gfx950): the local sum of slice partials (with an
// optional dropout), fp32 gradient accumulation, and the fused mixed-precision
// Adam step.
//
// * Partial sum (operator g's forward / f's backward of the tensor-slicing
//   example in the STRONGHOLD slides, done on one device):
//   out = residual + bias + sum of partials, fp32 sum, one rounding.
// * Gradient accumulation over micro-batches (Elamur summary of the MT-NLG
//   paper, Key points): acc = (overwrite ? 0 : acc) + grad.
// * Adam over the flat share (same page: about 20 bytes per parameter with
//   mixed precision): (1) per-workgroup partial sums of the squared unscaled
//   gradient in fp64 plus a non-finite flag, (2) a one-workgroup finish in
//   fixed order that writes {norm, clip coef, found_inf} to device memory,
//   (3) the update, which reads those scalars itself and leaves every buffer
//   untouched when found_inf is set -- the host never waits. Step (1) can
//   instead ride along the last micro-batch's accumulation (grad_accumulate_norm,
//   then adam_update runs (2) and (3)).
// Grid-stride loops over 16-byte vectors; all pointers are 16-byte aligned
// (checked on the host) and the ragged tail is done per element.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace mtnlg {

namespace {

constexpr int kStreamThreads = 256;

int stream_grid(int64_t units, int64_t max_blocks = 256 * 8) {
  int64_t b = (units + kStreamThreads - 1) / kStreamThreads;
  return (int)(b < 1 ? 1 : (b > max_blocks ? max_blocks : b));
}

// The optimizer streams (accumulation, norm, update) touch every byte once.
// The passes that leave one fp64 partial per workgroup (the norm, the
// accumulation that also forms it) are capped at kOptBlocks workgroups, the
// size of the partials in the optimizer workspace; the norm and update passes
// use non-temporal accesses (measured faster there, slower for the
// accumulation).
constexpr int64_t kOptBlocks = 256 * 128;
// Streams that write no per-workgroup partials launch one thread per vector
// group (each thread's loop runs once): on MI355X that streams 10-25% faster
// than a grid-stride loop over a few thousand workgroups (measured: copy
// 6.5 vs 5.1 TB/s, the update's 4-read/4-write mix 5.6 vs 5.0 TB/s).
constexpr int64_t kOneShotBlocks = int64_t(1) << 30;
typedef float nf4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt(const float4* p) {
  const nf4_t v = __builtin_nontemporal_load(reinterpret_cast<const nf4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
// four gradient values from a 16-byte (fp32) or 8-byte (bf16) group
__device__ __forceinline__ float4 ld4_nt(const float* g, int64_t u) {
  return ld_nt(reinterpret_cast<const float4*>(g) + u);
}
__device__ __forceinline__ float4 ld4_nt(const bf16_t* g, int64_t u) {
  typedef unsigned int nu2_t __attribute__((ext_vector_type(2)));
  const nu2_t w = __builtin_nontemporal_load(reinterpret_cast<const nu2_t*>(g) + u);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xffff0000u));
}
__device__ __forceinline__ void st_nt(float4* p, const float4& v) {
  const nf4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nf4_t*>(p));
}
__device__ __forceinline__ void st_nt(uint2* p, const uint2& v) {
  typedef unsigned int nu2_t __attribute__((ext_vector_type(2)));
  const nu2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<nu2_t*>(p));
}

struct PartialPtrs {
  const void* p[kMaxPartials];
};

template <typename T>
__global__ __launch_bounds__(kStreamThreads) void reduce_partials_kernel(PartialPtrs parts, int n, int64_t total,
                                                                         int64_t cols, const T* __restrict__ residual,
                                                                         const T* __restrict__ bias,
                                                                         T* __restrict__ out) {
  const int64_t units = total / 8;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = u * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (residual) load8(residual + i, acc);
    for (int j = 0; j < n; ++j) {
      float v[8];
      load8(static_cast<const T*>(parts.p[j]) + i, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
    if (bias) {
      float b[8];
      load8(bias + (i % cols), b);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += b[e];
    }
    store8(out + i, acc);
  }
}

// ---- dropout on the sum of the partials (counter-based mask) ----
//
// One Philox4x64-10 block (philox4x64 in common.hpp) yields 256 bits, sixteen
// 16-bit draws: element e of a row-major tensor uses block e / 16 (counter (e/16, 0, 0, 0),
// key (seed, site)) and the draw at bits 16 * (e % 4) of word (e % 16) / 4.
// It is kept when draw >= thr; kept values are multiplied by scale.
__device__ __forceinline__ void philox_block(uint64_t c0, uint64_t k0, uint64_t k1, uint64_t w[4]) {
  philox4x64(c0, 0, 0, 0, k0, k1, w);
}

struct DropoutArgs {
  uint64_t seed, site;
  uint32_t thr;  // drop when the 16-bit draw is below thr
  float scale;   // 65536 / (65536 - thr)
};

// keep bit j (0..15) of a 16-element group as a 16-bit mask
__device__ __forceinline__ uint32_t keep_bits(uint64_t group, const DropoutArgs& d) {
  uint64_t w[4];
  philox_block(group, d.seed, d.site, w);
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) bits |= (uint32_t)(((w[j >> 2] >> (16 * (j & 3))) & 0xFFFFu) >= d.thr) << j;
  return bits;
}

// out = residual + keep * scale * (sum of partials + bias), 16 elements (one
// generator block) per thread and iteration; total is a multiple of 8.
template <typename T>
__global__ __launch_bounds__(kStreamThreads) void reduce_dropout_kernel(PartialPtrs parts, int n, int64_t total,
                                                                        int64_t cols, const T* __restrict__ residual,
                                                                        const T* __restrict__ bias,
                                                                        T* __restrict__ out, DropoutArgs d) {
  const int64_t groups = (total + 15) / 16;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t keep = keep_bits((uint64_t)g, d);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int64_t i = g * 16 + hf * 8;
      if (i >= total) break;
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int j = 0; j < n; ++j) {
        float v[8];
        load8(static_cast<const T*>(parts.p[j]) + i, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] += v[e];
      }
      if (bias) {
        float b[8];
        load8(bias + (i % cols), b);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] += b[e];
      }
      float r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (residual) load8(residual + i, r);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] += ((keep >> (hf * 8 + e)) & 1u) ? z[e] * d.scale : 0.0f;
      store8(out + i, r);
    }
  }
}

// dz = keep * scale * dy (the same mask, regenerated)
template <typename T>
__global__ __launch_bounds__(kStreamThreads) void dropout_bwd_kernel(int64_t total, const T* __restrict__ dy,
                                                                     T* __restrict__ dz, DropoutArgs d) {
  const int64_t groups = (total + 15) / 16;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t keep = keep_bits((uint64_t)g, d);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int64_t i = g * 16 + hf * 8;
      if (i >= total) break;
      float v[8];
      load8(dy + i, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = ((keep >> (hf * 8 + e)) & 1u) ? v[e] * d.scale : 0.0f;
      store8(dz + i, v);
    }
  }
}

// acc = (overwrite ? 0 : acc) + grad. With NORM the same pass also leaves, per
// workgroup, the fp64 sum of (acc * s)^2 over the elements it wrote and a
// non-finite flag: the norm pass of the optimizer folded into the last
// micro-batch's accumulation, one fewer read of the accumulator. Without
// STORE (overwrite only) nothing is written but those partials: the norm pass
// over a gradient that the update then reads as it is.
template <typename T, bool NORM, bool STORE = true>
__global__ __launch_bounds__(kStreamThreads) void grad_acc_kernel(int64_t n, const T* __restrict__ g,
                                                                  float* __restrict__ acc, int overwrite, float s,
                                                                  double* __restrict__ part,
                                                                  int* __restrict__ flag) {
  const int64_t units = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 2;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x * 2 + threadIdx.x;
  double sq2[2] = {0.0, 0.0};  // one fp64 sum per unit slot: shorter dependency chains
  int bad = 0;
  for (int64_t u0 = t0; u0 < units; u0 += stride) {
    float v[2][8], a[2][8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t u = u0 + (int64_t)k * blockDim.x;
      if (u < units) {
        load8(g + u * 8, v[k]);  // plain loads: non-temporal ones measured slower here
        if (!overwrite) load8(acc + u * 8, a[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t u = u0 + (int64_t)k * blockDim.x;
      if (u < units) {
        if (!overwrite) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[k][e] += a[k][e];
        }
        if (STORE) store8(acc + u * 8, v[k]);
        if (NORM) {
          double q[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float t = v[k][e] * s;
            bad |= !isfinite(t);
            q[e] = (double)t * t;
          }
          sq2[k] += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
        }
      }
    }
  }
  double sq = sq2[0] + sq2[1];
  const int64_t s1 = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = units * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += s1) {
    const float v = Elem<T>::to_f(g[i]);
    const float r = overwrite ? v : acc[i] + v;
    if (STORE) acc[i] = r;
    if (NORM) {
      const float t = r * s;
      bad |= !isfinite(t);
      sq += (double)t * t;
    }
  }
  if (NORM) {
    __shared__ double red[kStreamThreads / kWave];
    const double tot = block_sum<kStreamThreads>(sq, red);
    const double nbad = block_sum<kStreamThreads>((double)bad, red);
    if (threadIdx.x == 0) {
      part[blockIdx.x] = tot;
      flag[blockIdx.x] = nbad > 0.0;
    }
  }
}

// (1) partial sums of (grad * s)^2 in fp64 and a non-finite flag per workgroup
__global__ __launch_bounds__(kStreamThreads) void adam_norm_kernel(int64_t n, const float* __restrict__ grad,
                                                                   float s, double* __restrict__ part,
                                                                   int* __restrict__ flag) {
  __shared__ double red[kStreamThreads / kWave];
  __shared__ int bad_any;
  if (threadIdx.x == 0) bad_any = 0;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = n / 4;
  // four 16-byte loads in flight per thread and two independent fp64 sums
  // (a fixed order, so the result is deterministic)
  constexpr int U = 4;
  double acc2[2] = {0.0, 0.0};
  int bad = 0;
  for (int64_t u0 = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; u0 < n4; u0 += U * stride) {
    float4 g[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t u = u0 + (int64_t)k * blockDim.x;
      g[k] = u < n4 ? ld_nt(reinterpret_cast<const float4*>(grad) + u) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float a = g[k].x * s, b = g[k].y * s, c = g[k].z * s, d = g[k].w * s;
      bad |= !isfinite(a) | !isfinite(b) | !isfinite(c) | !isfinite(d);
      acc2[k & 1] += ((double)a * a + (double)b * b) + ((double)c * c + (double)d * d);
    }
  }
  double acc = acc2[0] + acc2[1];
  for (int64_t i = n4 * 4 + t0; i < n; i += stride) {
    const float a = grad[i] * s;
    bad |= !isfinite(a);
    acc += (double)a * a;
  }
  if (bad) bad_any = 1;  // benign race: every writer stores 1
  const double tot = block_sum<kStreamThreads>(acc, red);
  if (threadIdx.x == 0) {
    part[blockIdx.x] = tot;
    flag[blockIdx.x] = bad_any;
  }
}

// (2) one workgroup: fixed-order sum of the partials -> stats {norm, coef, found_inf}
__global__ __launch_bounds__(kStreamThreads) void adam_finish_kernel(const double* __restrict__ part,
                                                                     const int* __restrict__ flag, int nparts,
                                                                     float max_norm, float* __restrict__ stats) {
  __shared__ double red[kStreamThreads / kWave];
  __shared__ int bad_any;
  if (threadIdx.x == 0) bad_any = 0;
  __syncthreads();
  double acc = 0.0;
  int bad = 0;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) {
    acc += part[i];
    bad |= flag[i];
  }
  if (bad) bad_any = 1;
  const double tot = block_sum<kStreamThreads>(acc, red);
  if (threadIdx.x == 0) {
    const int found_inf = bad_any || !isfinite(tot);
    const double norm = sqrt(tot);
    double coef = 1.0;
    if (max_norm > 0.0f) {
      const double c = (double)max_norm / (norm + 1e-6);
      if (c < 1.0) coef = c;
    }
    stats[0] = found_inf ? __builtin_nanf("") : (float)norm;
    stats[1] = found_inf ? 1.0f : (float)coef;
    stats[2] = found_inf ? 1.0f : 0.0f;
  }
}

__device__ __forceinline__ void adam_one(float& p, float& m, float& v, float g, const AdamScalars& c) {
  if (c.weight_decay > 0.0f) p *= 1.0f - c.lr * c.weight_decay;
  m = c.beta1 * m + (1.0f - c.beta1) * g;
  v = c.beta2 * v + (1.0f - c.beta2) * g * g;
  const float mhat = m * c.inv_bc1;
  const float vhat = v * c.inv_bc2;
  p -= c.lr * mhat / (sqrtf(vhat) + c.eps);
}

// (3) the update; reads found_inf and coef written by (2) on the same stream.
// G: the gradient's type (fp32 accumulator, or a bf16 gradient read as it is)
template <typename G>
__global__ __launch_bounds__(kStreamThreads) void adam_update_kernel(AdamScalars c, int64_t n,
                                                                     float* __restrict__ master, float* __restrict__ m,
                                                                     float* __restrict__ v,
                                                                     const G* __restrict__ grad,
                                                                     bf16_t* __restrict__ w,
                                                                     const float* __restrict__ stats) {
  if (stats[2] != 0.0f) return;
  const float gs = c.inv_loss_scale * stats[1];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = n / 4;
  // one 16-byte group of each stream per thread (the launch covers n/4 threads):
  // measured faster than two groups per thread (5.8 vs 5.4 TB/s at 1.9e9)
  for (int64_t u = t0; u < n4; u += stride) {
    float4 p = ld_nt(reinterpret_cast<const float4*>(master) + u);
    float4 mm = ld_nt(reinterpret_cast<const float4*>(m) + u);
    float4 vv = ld_nt(reinterpret_cast<const float4*>(v) + u);
    const float4 g = ld4_nt(grad, u);
    adam_one(p.x, mm.x, vv.x, g.x * gs, c);
    adam_one(p.y, mm.y, vv.y, g.y * gs, c);
    adam_one(p.z, mm.z, vv.z, g.z * gs, c);
    adam_one(p.w, mm.w, vv.w, g.w * gs, c);
    st_nt(reinterpret_cast<float4*>(master) + u, p);
    st_nt(reinterpret_cast<float4*>(m) + u, mm);
    st_nt(reinterpret_cast<float4*>(v) + u, vv);
    if (w) st_nt(reinterpret_cast<uint2*>(w) + u, make_uint2(pack_bf16x2(p.x, p.y), pack_bf16x2(p.z, p.w)));
  }
  for (int64_t i = n4 * 4 + t0; i < n; i += stride) {
    float p = master[i], mm = m[i], vv = v[i];
    adam_one(p, mm, vv, Elem<G>::to_f(grad[i]) * gs, c);
    master[i] = p;
    m[i] = mm;
    v[i] = vv;
    if (w) w[i] = f2bf(p);
  }
}

// The Adam update's memory traffic without its arithmetic: the same launch,
// the same streams in the same order (master, m, v and the gradient read; master,
// m, v and the bf16 copy written, with the same cache hints), each value written
// back unchanged (the gradient is only waited for). Its rate is what the memory
// system gives this access mix, the ceiling against which the update is judged.
__global__ __launch_bounds__(kStreamThreads) void adam_streams_kernel(int64_t n, float* __restrict__ master,
                                                                      float* __restrict__ m,
                                                                      float* __restrict__ v,
                                                                      const float* __restrict__ grad,
                                                                      bf16_t* __restrict__ w) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = n / 4;
  for (int64_t u = t0; u < n4; u += stride) {
    const float4 p = ld_nt(reinterpret_cast<const float4*>(master) + u);
    const float4 mm = ld_nt(reinterpret_cast<const float4*>(m) + u);
    const float4 vv = ld_nt(reinterpret_cast<const float4*>(v) + u);
    const float4 g = ld_nt(reinterpret_cast<const float4*>(grad) + u);
    asm volatile("" : : "v"(g.x), "v"(g.y), "v"(g.z), "v"(g.w));
    st_nt(reinterpret_cast<float4*>(master) + u, p);
    st_nt(reinterpret_cast<float4*>(m) + u, mm);
    st_nt(reinterpret_cast<float4*>(v) + u, vv);
    if (w) st_nt(reinterpret_cast<uint2*>(w) + u, make_uint2(pack_bf16x2(p.x, p.y), pack_bf16x2(p.z, p.w)));
  }
  for (int64_t i = n4 * 4 + t0; i < n; i += stride) {
    const float g = grad[i];
    asm volatile("" : : "v"(g));
    const float p = master[i];
    master[i] = p;
    m[i] = m[i];
    v[i] = v[i];
    if (w) w[i] = f2bf(p);
  }
}

constexpr int kNormBlocks = 8192;

}  // namespace

hipError_t reduce_partials(int dtype, int64_t rows, int64_t cols, const void* const* parts, int n,
                           const void* residual, const void* bias, void* out, hipStream_t st) {
  const int64_t total = rows * cols;
  if (total == 0) return hipSuccess;
  PartialPtrs pp{};
  for (int j = 0; j < n; ++j) pp.p[j] = parts[j];
  const int grid = stream_grid(total / 8, kOneShotBlocks);
  if (dtype == kBF16)
    hipLaunchKernelGGL(reduce_partials_kernel<bf16_t>, dim3(grid), dim3(kStreamThreads), 0, st, pp, n, total, cols,
                       static_cast<const bf16_t*>(residual), static_cast<const bf16_t*>(bias),
                       static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(grid), dim3(kStreamThreads), 0, st, pp, n, total, cols,
                       static_cast<const float*>(residual), static_cast<const float*>(bias),
                       static_cast<float*>(out));
  return hipGetLastError();
}

namespace {
DropoutArgs dropout_args(uint64_t seed, uint64_t site, uint32_t thr) {
  DropoutArgs d;
  d.seed = seed;
  d.site = site;
  d.thr = thr;
  d.scale = (float)(65536.0 / (65536.0 - (double)thr));
  return d;
}
}  // namespace

hipError_t reduce_partials_dropout(int dtype, int64_t rows, int64_t cols, const void* const* parts, int n,
                                   const void* residual, const void* bias, void* out, uint64_t seed,
                                   uint64_t site, uint32_t thr, hipStream_t st) {
  const int64_t total = rows * cols;
  if (total == 0) return hipSuccess;
  PartialPtrs pp{};
  for (int j = 0; j < n; ++j) pp.p[j] = parts[j];
  const DropoutArgs d = dropout_args(seed, site, thr);
  const int grid = stream_grid((total + 15) / 16, kOneShotBlocks);
  if (dtype == kBF16)
    hipLaunchKernelGGL(reduce_dropout_kernel<bf16_t>, dim3(grid), dim3(kStreamThreads), 0, st, pp, n, total, cols,
                       static_cast<const bf16_t*>(residual), static_cast<const bf16_t*>(bias),
                       static_cast<bf16_t*>(out), d);
  else
    hipLaunchKernelGGL(reduce_dropout_kernel<float>, dim3(grid), dim3(kStreamThreads), 0, st, pp, n, total, cols,
                       static_cast<const float*>(residual), static_cast<const float*>(bias),
                       static_cast<float*>(out), d);
  return hipGetLastError();
}

hipError_t dropout_bwd(int dtype, int64_t total, const void* dy, void* dz, uint64_t seed, uint64_t site,
                       uint32_t thr, hipStream_t st) {
  if (total == 0) return hipSuccess;
  const DropoutArgs d = dropout_args(seed, site, thr);
  const int grid = stream_grid((total + 15) / 16, kOneShotBlocks);
  if (dtype == kBF16)
    hipLaunchKernelGGL(dropout_bwd_kernel<bf16_t>, dim3(grid), dim3(kStreamThreads), 0, st, total,
                       static_cast<const bf16_t*>(dy), static_cast<bf16_t*>(dz), d);
  else
    hipLaunchKernelGGL(dropout_bwd_kernel<float>, dim3(grid), dim3(kStreamThreads), 0, st, total,
                       static_cast<const float*>(dy), static_cast<float*>(dz), d);
  return hipGetLastError();
}

int acc_grid(int64_t n) { return stream_grid(n / 16 + 1, kOptBlocks); }

hipError_t grad_accumulate(int64_t n, int dtype, const void* grad, float* acc, bool overwrite, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int grid = stream_grid(n / 16 + 1, kOneShotBlocks);
  if (dtype == kBF16)
    hipLaunchKernelGGL((grad_acc_kernel<bf16_t, false>), dim3(grid), dim3(kStreamThreads), 0, st, n,
                       static_cast<const bf16_t*>(grad), acc, (int)overwrite, 1.0f, nullptr, nullptr);
  else
    hipLaunchKernelGGL((grad_acc_kernel<float, false>), dim3(grid), dim3(kStreamThreads), 0, st, n,
                       static_cast<const float*>(grad), acc, (int)overwrite, 1.0f, nullptr, nullptr);
  return hipGetLastError();
}

// Workspace: per-workgroup fp64 partial sums and int flags, sized for the
// larger of the two grids that fill it (the norm pass, the accumulation).
size_t adam_ws(int64_t) { return (size_t)kOptBlocks * (sizeof(double) + sizeof(int)); }

hipError_t grad_accumulate_norm(int64_t n, int dtype, const void* grad, float* acc, bool overwrite,
                                float inv_loss_scale, void* ws, hipStream_t st) {
  double* part = static_cast<double*>(ws);
  int* flag = reinterpret_cast<int*>(part + kOptBlocks);
  const int grid = acc_grid(n);  // n == 0 still writes the one (zero) partial
  if (dtype == kBF16)
    hipLaunchKernelGGL((grad_acc_kernel<bf16_t, true>), dim3(grid), dim3(kStreamThreads), 0, st, n,
                       static_cast<const bf16_t*>(grad), acc, (int)overwrite, inv_loss_scale, part, flag);
  else
    hipLaunchKernelGGL((grad_acc_kernel<float, true>), dim3(grid), dim3(kStreamThreads), 0, st, n,
                       static_cast<const float*>(grad), acc, (int)overwrite, inv_loss_scale, part, flag);
  return hipGetLastError();
}

namespace {
// (2) + (3): the finish over nparts partials, then the update
template <typename G>
hipError_t finish_and_update(const AdamScalars& c, int64_t n, float* master, float* m, float* v, const G* grad,
                             void* w_bf16, float* stats, const double* part, const int* flag, int nparts,
                             hipStream_t st) {
  hipLaunchKernelGGL(adam_finish_kernel, dim3(1), dim3(kStreamThreads), 0, st, part, flag, nparts,
                     c.max_grad_norm, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  const int grid = stream_grid(n / 4 + 1, kOneShotBlocks);
  hipLaunchKernelGGL(adam_update_kernel<G>, dim3(grid), dim3(kStreamThreads), 0, st, c, n, master, m, v, grad,
                     static_cast<bf16_t*>(w_bf16), stats);
  return hipGetLastError();
}
}  // namespace

namespace {
// (1) + (2) + (3) with the norm partials in `part` and `flag` (at least
// kNormBlocks entries each)
hipError_t adam_step_parts(const AdamScalars& c, int64_t n, float* master, float* m, float* v, const float* grad,
                           void* w_bf16, float* stats, double* part, int* flag, hipStream_t st) {
  const int nb = n == 0 ? 1 : std::min<int>(kNormBlocks, stream_grid(n / 8 + 1, kNormBlocks));
  hipLaunchKernelGGL(adam_norm_kernel, dim3(nb), dim3(kStreamThreads), 0, st, n, grad, c.inv_loss_scale, part,
                     flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish_and_update(c, n, master, m, v, grad, w_bf16, stats, part, flag, nb, st);
}

// The optimizer scratch of adam_step_static: one fp64 partial and one flag
// per norm workgroup (96 KiB), in the library's own device memory, one copy
// per GPU, held until the process ends. Host code must not use this name as
// an address (it is a host-side stand-in): kernels get the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNormBlocks * (sizeof(double) + sizeof(int))];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, looked up on first use.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

size_t adam_static_scratch_bytes() { return sizeof(scratch); }

hipError_t adam_step(const AdamScalars& c, int64_t n, float* master, float* m, float* v, const float* grad,
                     void* w_bf16, float* stats, void* ws, hipStream_t st) {
  double* part = static_cast<double*>(ws);
  return adam_step_parts(c, n, master, m, v, grad, w_bf16, stats, part, reinterpret_cast<int*>(part + kOptBlocks),
                         st);
}

hipError_t adam_step_static(const AdamScalars& c, int64_t n, float* master, float* m, float* v, const float* grad,
                            void* w_bf16, float* stats, hipStream_t st) {
  void* p = nullptr;
  const hipError_t e = scratch_ptr(&p);
  if (e != hipSuccess) return e;
  double* part = static_cast<double*>(p);
  return adam_step_parts(c, n, master, m, v, grad, w_bf16, stats, part, reinterpret_cast<int*>(part + kNormBlocks),
                         st);
}

hipError_t adam_streams(int64_t n, float* master, float* m, float* v, const float* grad, void* w_bf16,
                        hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int grid = stream_grid(n / 4 + 1, kOneShotBlocks);
  hipLaunchKernelGGL(adam_streams_kernel, dim3(grid), dim3(kStreamThreads), 0, st, n, master, m, v, grad,
                     static_cast<bf16_t*>(w_bf16));
  return hipGetLastError();
}

hipError_t adam_update(const AdamScalars& c, int64_t n, float* master, float* m, float* v, const float* grad,
                       void* w_bf16, float* stats, const void* ws, hipStream_t st) {
  const double* part = static_cast<const double*>(ws);
  const int* flag = reinterpret_cast<const int*>(part + kOptBlocks);
  return finish_and_update(c, n, master, m, v, grad, w_bf16, stats, part, flag, acc_grid(n), st);
}

hipError_t grad_norm_bf16(int64_t n, const void* grad, float inv_loss_scale, void* ws, hipStream_t st) {
  double* part = static_cast<double*>(ws);
  int* flag = reinterpret_cast<int*>(part + kOptBlocks);
  // the launch and per-thread order of grad_accumulate_norm: the same partials
  hipLaunchKernelGGL((grad_acc_kernel<bf16_t, true, false>), dim3(acc_grid(n)), dim3(kStreamThreads), 0, st, n,
                     static_cast<const bf16_t*>(grad), nullptr, 1, inv_loss_scale, part, flag);
  return hipGetLastError();
}

hipError_t adam_update_bf16(const AdamScalars& c, int64_t n, float* master, float* m, float* v, const void* grad,
                            void* w_bf16, float* stats, const void* ws, hipStream_t st) {
  const double* part = static_cast<const double*>(ws);
  const int* flag = reinterpret_cast<const int*>(part + kOptBlocks);
  return finish_and_update(c, n, master, m, v, static_cast<const bf16_t*>(grad), w_bf16, stats, part, flag,
                           acc_grid(n), st);
}

}  // namespace mtnlg
