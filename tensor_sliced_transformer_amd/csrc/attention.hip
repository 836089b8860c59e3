// Causal multi-head attention, forward and backward, on MFMA (gfx950): the
// fp32 kernels, and the dispatch of both dtypes (bf16 runs the kernels of
// attention_bf16.hip).
//
// Per sequence and head: S = Q K^T / sqrt(d), keys after the query masked,
// P = softmax(S) row-wise, O = P V (the left-to-right decoder of the MT-NLG
// pages; the scale is the usual 1/sqrt(head_dim)). The forward keeps a
// running max and sum per query (online softmax) so S is never written to
// memory, and saves lse = log of each row's normaliser for the backward.
//
// Wavefront layout (32x32 MFMA blocks, wave64):
//   * Forward: a workgroup of 4 waves owns 128 queries (32 per wave) and
//     walks 64-key blocks up to the diagonal. Each wave computes
//     S^T = K Q^T, so in the MFMA output a lane owns ONE query (its column)
//     and 32 of the 64 keys; the row max / sum need one cross-lane step
//     (lane ^ 32). Then O^T += V^T P^T reuses the P values straight from the
//     accumulator registers as the B operand: the k-slots of an MFMA may be
//     any permutation as long as A and B agree, so V^T is read from LDS in the
//     matching (permuted) key order. The running rescale of O^T is per lane.
//   * Backward, dK/dV: a workgroup owns 128 keys (K, V rows kept in
//     registers), walks 64-query blocks from the diagonal on: S = Q K^T,
//     dP = dO V^T, P from lse, dS = P (dP - D) with D = rowsum(dO * O); then
//     dV^T += dO^T P and dK^T += Q^T dS with the same permuted-k trick.
//   * Backward, dQ: a workgroup owns 128 queries (Q, dO in registers), walks
//     key blocks up to the diagonal: dQ^T += K^T dS^T.
//   Two kernels instead of atomics keep the result deterministic.
//   * Key tiles live in LDS as rows of head_dim with one 16-byte pad chunk
//     per row; transposed tiles (V^T, Q^T, dO^T, K^T) are produced by
//     loading VECxVEC micro-blocks and transposing them in registers.
//   * Workgroups are launched heaviest first (causal work grows with the
//     query index for the forward and dQ, shrinks for dK/dV).
#include "common.hpp"
#include "kernels.hpp"

namespace mtnlg {

namespace {

constexpr int kBQ = 128;   // queries (or keys) per workgroup
constexpr int kBKV = 64;   // keys (or queries) per inner block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void transpose_vec(const uint4* in, uint4* out, bf16_t) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = i >> 1;
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[i * 4 + q] = __builtin_amdgcn_perm(w[(2 * q + 1) * 4 + d], w[(2 * q) * 4 + d], sel);
  }
}
__device__ __forceinline__ void transpose_vec(const uint4* in, uint4* out, float) {
  const float* f = reinterpret_cast<const float*>(in);
  float* o = reinterpret_cast<float*>(out);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[i * 4 + j] = f[j * 4 + i];
}

// One 16-byte chunk per lane of A and B (see the GEMM): 32x32 MFMA(s).
__device__ __forceinline__ void mma_chunk(const uint4& a, const uint4& b, f32x16_t& c, bf16_t) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                              0, 0, 0);
}
__device__ __forceinline__ void mma_chunk(const uint4& a, const uint4& b, f32x16_t& c, float) {
  const float* fa = reinterpret_cast<const float*>(&a);
  const float* fb = reinterpret_cast<const float*>(&b);
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[j], fb[j], c, 0, 0, 0);
}

// acc += X^T-tile * P where P is a 32x32 block held in MFMA output layout
// (lane: column lane%32, rows 8*blk + 4*g + r at index 4*blk + r) and is
// used as the B operand without moving it; `row` points at the LDS row (the
// output row of this lane) of a tile stored contiguous along the reduction
// index, already offset to the 32-wide block being reduced.
__device__ __forceinline__ void mma_perm(const char* row, const f32x16_t& p, f32x16_t& acc, int g, bf16_t) {
  const bf16_t* r = reinterpret_cast<const bf16_t*>(row);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint2 lo = *reinterpret_cast<const uint2*>(r + 16 * t + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(r + 16 * t + 8 + 4 * g);
    uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
    uint4 b;
    b.x = pack_bf16x2(p[8 * t + 0], p[8 * t + 1]);
    b.y = pack_bf16x2(p[8 * t + 2], p[8 * t + 3]);
    b.z = pack_bf16x2(p[8 * t + 4], p[8 * t + 5]);
    b.w = pack_bf16x2(p[8 * t + 6], p[8 * t + 7]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
  }
}
__device__ __forceinline__ void mma_perm(const char* row, const f32x16_t& p, f32x16_t& acc, int g, float) {
  const float* r = reinterpret_cast<const float*>(row);
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const float4 a = *reinterpret_cast<const float4*>(r + 8 * blk + 4 * g);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, p[4 * blk + 0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, p[4 * blk + 1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, p[4 * blk + 2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, p[4 * blk + 3], acc, 0, 0, 0);
  }
}

template <typename T, int D>
struct Geo {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int CPR = D / VEC;           // 16-byte chunks per row of head_dim
  static constexpr int KS = CPR + 1;            // padded LDS row stride (chunks)
  static constexpr int EB = D / 32;             // 32-wide blocks of head_dim
  static constexpr int TS = kBKV * (int)sizeof(T) + 16;   // bytes per row of a transposed tile
};

// rows [r0, r0+64) of a head's D columns (row stride ld) -> LDS, natural layout
template <typename T, int D>
__device__ __forceinline__ void load_rows(const T* __restrict__ src, int64_t ld, uint4* dst, int tid) {
  using G = Geo<T, D>;
  for (int id = tid; id < kBKV * G::CPR; id += 256) {
    const int r = id / G::CPR, c = id % G::CPR;
    dst[r * G::KS + c] = *reinterpret_cast<const uint4*>(src + (int64_t)r * ld + c * G::VEC);
  }
}

// rows [r0, r0+64) -> LDS transposed: dst row e (of D) holds the 64 rows' values
template <typename T, int D>
__device__ __forceinline__ void load_rows_t(const T* __restrict__ src, int64_t ld, char* dst, int tid) {
  using G = Geo<T, D>;
  constexpr int VEC = G::VEC;
  for (int id = tid; id < (kBKV / VEC) * G::CPR; id += 256) {
    const int rb = id / G::CPR, eb = id % G::CPR;
    uint4 in[VEC], out[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) in[j] = *reinterpret_cast<const uint4*>(src + (int64_t)(rb * VEC + j) * ld + eb * VEC);
    transpose_vec(in, out, T());
#pragma unroll
    for (int i = 0; i < VEC; ++i) *reinterpret_cast<uint4*>(dst + (eb * VEC + i) * G::TS + rb * 16) = out[i];
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// ------------------------------------------------------------------ forward
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ o,
                                                       float* __restrict__ lse, int seq, int nh, int64_t tokens,
                                                       float scale_log2) {
  using G = Geo<T, D>;
  __shared__ uint4 sK[kBKV * G::KS];
  __shared__ __align__(16) char sVt[D * G::TS];

  const int nqb = seq / kBQ;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int n = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.z * seq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, g = lane >> 5;
  const int64_t ld = 3LL * nh * D;
  const T* Qp = qkv + (int64_t)n * D;
  const T* Kp = qkv + (int64_t)(nh + n) * D;
  const T* Vp = qkv + (int64_t)(2 * nh + n) * D;

  const int q = qb * kBQ + wave * 32 + lq;
  uint4 qr[G::CPR / 2];
#pragma unroll
  for (int s = 0; s < G::CPR / 2; ++s)
    qr[s] = *reinterpret_cast<const uint4*>(Qp + (row0 + q) * ld + (2 * s + g) * G::VEC);

  f32x16_t oacc[G::EB];
#pragma unroll
  for (int e = 0; e < G::EB; ++e)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[e][i] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const int wave_qmax = qb * kBQ + wave * 32 + 31;
  const int nkv = (qb * kBQ + kBQ - 1) / kBKV + 1;

  for (int kb = 0; kb < nkv; ++kb) {
    const int kv0 = kb * kBKV;
    __syncthreads();
    load_rows<T, D>(Kp + (row0 + kv0) * ld, ld, sK, tid);
    load_rows_t<T, D>(Vp + (row0 + kv0) * ld, ld, sVt, tid);
    __syncthreads();
    if (kv0 > wave_qmax) continue;

    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[sub][i] = 0.0f;
#pragma unroll
      for (int st = 0; st < G::CPR / 2; ++st)
        mma_chunk(sK[(sub * 32 + lq) * G::KS + 2 * st + g], qr[st], s[sub], T());
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kv = kv0 + sub * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        float v = s[sub][i] * scale_log2;
        if (kv > q) v = -INFINITY;
        s[sub][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m, mx);
    const float corr = exp2f(m - m_new);
    l *= corr;
#pragma unroll
    for (int e = 0; e < G::EB; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[e][i] *= corr;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(s[sub][i] - m_new);
        l += p;
        s[sub][i] = p;
      }
    m = m_new;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int e = 0; e < G::EB; ++e)
        mma_perm(sVt + (e * 32 + lq) * G::TS + sub * 32 * (int)sizeof(T), s[sub], oacc[e], g, T());
  }
  l += __shfl_xor(l, 32, kWave);
  const float inv = 1.0f / l;
  T* orow = o + (row0 + q) * (int64_t)(nh * D) + (int64_t)n * D;
#pragma unroll
  for (int e = 0; e < G::EB; ++e)
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
      store4<T>(orow + e * 32 + 8 * blk + 4 * g, oacc[e][4 * blk] * inv, oacc[e][4 * blk + 1] * inv,
                oacc[e][4 * blk + 2] * inv, oacc[e][4 * blk + 3] * inv);
  if (g == 0) lse[(int64_t)n * tokens + row0 + q] = (m + log2f(l)) * kLn2;
}

// ---------------------------------------------------- backward: D = rowsum(dO * O)
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                           float* __restrict__ dd, int nh, int64_t tokens) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (token, head)
  if (id >= tokens * nh) return;
  const int64_t t = id / nh;
  const int n = (int)(id % nh);
  const T* a = o + t * (int64_t)(nh * D) + (int64_t)n * D;
  const T* b = dout + t * (int64_t)(nh * D) + (int64_t)n * D;
  float s = 0.0f;
#pragma unroll 4
  for (int c = 0; c < D; c += 8) {
    float x[8], y[8];
    load8(a + c, x);
    load8(b + c, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[e] * y[e];
  }
  dd[(int64_t)n * tokens + t] = s;
}

// ---------------------------------------------------------- backward: dK, dV
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ dd, T* __restrict__ dqkv,
                                                            int seq, int nh, int64_t tokens, float scale,
                                                            float scale_log2) {
  using G = Geo<T, D>;
  __shared__ uint4 sQ[kBKV * G::KS];
  __shared__ uint4 sdO[kBKV * G::KS];
  __shared__ __align__(16) char sQt[D * G::TS];
  __shared__ __align__(16) char sdOt[D * G::TS];
  __shared__ float sL[kBKV], sD[kBKV];

  const int kb = blockIdx.x;               // key block of 128: low blocks see the most queries
  const int n = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.z * seq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, g = lane >> 5;
  const int64_t ld = 3LL * nh * D;
  const int64_t ldo = (int64_t)nh * D;
  const T* Qp = qkv + (int64_t)n * D;
  const T* Kp = qkv + (int64_t)(nh + n) * D;
  const T* Vp = qkv + (int64_t)(2 * nh + n) * D;
  const T* dOp = dout + (int64_t)n * D;

  const int kv = kb * kBQ + wave * 32 + lq;
  uint4 kr[G::CPR / 2], vr[G::CPR / 2];
#pragma unroll
  for (int s = 0; s < G::CPR / 2; ++s) {
    kr[s] = *reinterpret_cast<const uint4*>(Kp + (row0 + kv) * ld + (2 * s + g) * G::VEC);
    vr[s] = *reinterpret_cast<const uint4*>(Vp + (row0 + kv) * ld + (2 * s + g) * G::VEC);
  }
  f32x16_t dv[G::EB], dk[G::EB];
#pragma unroll
  for (int e = 0; e < G::EB; ++e)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dv[e][i] = 0.0f; dk[e][i] = 0.0f; }

  const int wave_kvmin = kb * kBQ + wave * 32;
  const int nqblk = seq / kBKV;
  for (int qb = (kb * kBQ) / kBKV; qb < nqblk; ++qb) {
    const int q0 = qb * kBKV;
    __syncthreads();
    load_rows<T, D>(Qp + (row0 + q0) * ld, ld, sQ, tid);
    load_rows<T, D>(dOp + (row0 + q0) * ldo, ldo, sdO, tid);
    load_rows_t<T, D>(Qp + (row0 + q0) * ld, ld, sQt, tid);
    load_rows_t<T, D>(dOp + (row0 + q0) * ldo, ldo, sdOt, tid);
    if (tid < kBKV) {
      sL[tid] = lse[(int64_t)n * tokens + row0 + q0 + tid] * kLog2e;
      sD[tid] = dd[(int64_t)n * tokens + row0 + q0 + tid];
    }
    __syncthreads();
    if (q0 + kBKV - 1 < wave_kvmin) continue;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16_t s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[i] = 0.0f; dp[i] = 0.0f; }
#pragma unroll
      for (int st = 0; st < G::CPR / 2; ++st) {
        mma_chunk(sQ[(sub * 32 + lq) * G::KS + 2 * st + g], kr[st], s, T());
        mma_chunk(sdO[(sub * 32 + lq) * G::KS + 2 * st + g], vr[st], dp, T());
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = sub * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        const float p = (kv > q0 + qi) ? 0.0f : exp2f(s[i] * scale_log2 - sL[qi]);
        s[i] = p;
        dp[i] = p * (dp[i] - sD[qi]);
      }
#pragma unroll
      for (int e = 0; e < G::EB; ++e) {
        mma_perm(sdOt + (e * 32 + lq) * G::TS + sub * 32 * (int)sizeof(T), s, dv[e], g, T());
        mma_perm(sQt + (e * 32 + lq) * G::TS + sub * 32 * (int)sizeof(T), dp, dk[e], g, T());
      }
    }
  }
  // lane holds key `kv` (its column) and head_dim rows e*32 + 8*blk + 4*g + r
  T* dkrow = dqkv + (row0 + kv) * ld + (int64_t)(nh + n) * D;
  T* dvrow = dqkv + (row0 + kv) * ld + (int64_t)(2 * nh + n) * D;
#pragma unroll
  for (int e = 0; e < G::EB; ++e)
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int c = e * 32 + 8 * blk + 4 * g;
      store4<T>(dkrow + c, dk[e][4 * blk] * scale, dk[e][4 * blk + 1] * scale, dk[e][4 * blk + 2] * scale,
                dk[e][4 * blk + 3] * scale);
      store4<T>(dvrow + c, dv[e][4 * blk], dv[e][4 * blk + 1], dv[e][4 * blk + 2], dv[e][4 * blk + 3]);
    }
}

// --------------------------------------------------------------- backward: dQ
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                          const float* __restrict__ lse, const float* __restrict__ dd,
                                                          T* __restrict__ dqkv, int seq, int nh, int64_t tokens,
                                                          float scale, float scale_log2) {
  using G = Geo<T, D>;
  __shared__ uint4 sK[kBKV * G::KS];
  __shared__ uint4 sV[kBKV * G::KS];
  __shared__ __align__(16) char sKt[D * G::TS];

  const int nqb = seq / kBQ;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int n = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.z * seq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, g = lane >> 5;
  const int64_t ld = 3LL * nh * D;
  const int64_t ldo = (int64_t)nh * D;
  const T* Qp = qkv + (int64_t)n * D;
  const T* Kp = qkv + (int64_t)(nh + n) * D;
  const T* Vp = qkv + (int64_t)(2 * nh + n) * D;
  const T* dOp = dout + (int64_t)n * D;

  const int q = qb * kBQ + wave * 32 + lq;
  uint4 qr[G::CPR / 2], dor[G::CPR / 2];
#pragma unroll
  for (int s = 0; s < G::CPR / 2; ++s) {
    qr[s] = *reinterpret_cast<const uint4*>(Qp + (row0 + q) * ld + (2 * s + g) * G::VEC);
    dor[s] = *reinterpret_cast<const uint4*>(dOp + (row0 + q) * ldo + (2 * s + g) * G::VEC);
  }
  const float lq2 = lse[(int64_t)n * tokens + row0 + q] * kLog2e;
  const float dq_d = dd[(int64_t)n * tokens + row0 + q];
  f32x16_t dq[G::EB];
#pragma unroll
  for (int e = 0; e < G::EB; ++e)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[e][i] = 0.0f;

  const int wave_qmax = qb * kBQ + wave * 32 + 31;
  const int nkv = (qb * kBQ + kBQ - 1) / kBKV + 1;
  for (int kb = 0; kb < nkv; ++kb) {
    const int kv0 = kb * kBKV;
    __syncthreads();
    load_rows<T, D>(Kp + (row0 + kv0) * ld, ld, sK, tid);
    load_rows<T, D>(Vp + (row0 + kv0) * ld, ld, sV, tid);
    load_rows_t<T, D>(Kp + (row0 + kv0) * ld, ld, sKt, tid);
    __syncthreads();
    if (kv0 > wave_qmax) continue;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16_t s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[i] = 0.0f; dp[i] = 0.0f; }
#pragma unroll
      for (int st = 0; st < G::CPR / 2; ++st) {
        mma_chunk(sK[(sub * 32 + lq) * G::KS + 2 * st + g], qr[st], s, T());
        mma_chunk(sV[(sub * 32 + lq) * G::KS + 2 * st + g], dor[st], dp, T());
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kvi = kv0 + sub * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        const float p = (kvi > q) ? 0.0f : exp2f(s[i] * scale_log2 - lq2);
        dp[i] = p * (dp[i] - dq_d);
      }
#pragma unroll
      for (int e = 0; e < G::EB; ++e)
        mma_perm(sKt + (e * 32 + lq) * G::TS + sub * 32 * (int)sizeof(T), dp, dq[e], g, T());
    }
  }
  T* dqrow = dqkv + (row0 + q) * ld + (int64_t)n * D;
#pragma unroll
  for (int e = 0; e < G::EB; ++e)
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
      store4<T>(dqrow + e * 32 + 8 * blk + 4 * g, dq[e][4 * blk] * scale, dq[e][4 * blk + 1] * scale,
                dq[e][4 * blk + 2] * scale, dq[e][4 * blk + 3] * scale);
}

template <typename T, int D>
hipError_t fwd_launch(int batch, int seq, int heads, const void* qkv, void* o, float* lse, hipStream_t st) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  dim3 grid(seq / kBQ, heads, batch);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(qkv),
                     static_cast<T*>(o), lse, seq, heads, (int64_t)batch * seq, scale_log2);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_launch(int batch, int seq, int heads, const void* qkv, const void* o, const float* lse,
                      const void* dout, void* dqkv, float* dd, hipStream_t st) {
  const int64_t tokens = (int64_t)batch * seq;
  const float scale = 1.0f / sqrtf((float)D);
  const float scale_log2 = kLog2e * scale;
  const int64_t pairs = tokens * heads;
  hipLaunchKernelGGL((attn_bwd_pre_kernel<T, D>), dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, st,
                     static_cast<const T*>(o), static_cast<const T*>(dout), dd, heads, tokens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(seq / kBQ, heads, batch);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(qkv),
                     static_cast<const T*>(dout), lse, dd, static_cast<T*>(dqkv), seq, heads, tokens, scale,
                     scale_log2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T*>(qkv),
                     static_cast<const T*>(dout), lse, dd, static_cast<T*>(dqkv), seq, heads, tokens, scale,
                     scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t attention_fwd(int dtype, int batch, int seq, int heads, int head_dim, const void* qkv, void* o,
                         float* lse, const AttnDropout& drop, hipStream_t st) {
  if (batch == 0) return hipSuccess;
#define MTNLG_AF(T, D) \
  if (head_dim == D) return fwd_launch<T, D>(batch, seq, heads, qkv, o, lse, st);
  if (dtype == kBF16) return attention_fwd_bf16(batch, seq, heads, head_dim, qkv, o, lse, drop, st);
  if (drop.thr) return hipErrorInvalidValue;  // dropout on the probabilities: bf16 kernels only
  MTNLG_AF(float, 64) MTNLG_AF(float, 128)
#undef MTNLG_AF
  return hipErrorInvalidValue;
}

// bf16: one (lse * log2 e, rowsum(dO * O)) float pair per (token, head); fp32: the rowsum only.
size_t attention_bwd_ws(int batch, int seq, int heads) { return (size_t)batch * seq * heads * 2 * sizeof(float); }

hipError_t attention_bwd(int dtype, int batch, int seq, int heads, int head_dim, const void* qkv, const void* o,
                         const float* lse, const void* dout, void* dqkv, void* ws, const AttnDropout& drop,
                         hipStream_t st) {
  if (batch == 0) return hipSuccess;
  float* dd = static_cast<float*>(ws);
#define MTNLG_AB(T, D) \
  if (head_dim == D) return bwd_launch<T, D>(batch, seq, heads, qkv, o, lse, dout, dqkv, dd, st);
  if (dtype == kBF16) return attention_bwd_bf16(batch, seq, heads, head_dim, qkv, o, lse, dout, dqkv, ws, drop, st);
  if (drop.thr) return hipErrorInvalidValue;
  MTNLG_AB(float, 64) MTNLG_AB(float, 128)
#undef MTNLG_AB
  return hipErrorInvalidValue;
}

}  // namespace mtnlg
