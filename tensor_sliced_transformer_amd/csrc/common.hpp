// Device-side helpers shared by the gfx950 kernels: element types, bf16
// conversion, 16-byte vector access and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtnlg {

typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

// Two floats -> packed bf16x2 in one dword (lo in bits 0-15), round to
// nearest even: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Element traits: VEC = elements per 16-byte vector.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int VEC = 8;
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  static __device__ __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};

// Load 8 consecutive elements as floats from a 16B-aligned (bf16) or two
// 16B-aligned (f32) vectors.
__device__ __forceinline__ void load8(const bf16_t* p, float* out) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const float* v) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
// 8 floats -> 8 IEEE binary16 values, round to nearest even.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}
__device__ __forceinline__ void store8_f16(uint16_t* p, const float* v) {
  uint4 u;
  u.x = pack_f16x2(v[0], v[1]);
  u.y = pack_f16x2(v[2], v[3]);
  u.z = pack_f16x2(v[4], v[5]);
  u.w = pack_f16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Sum over the 64 lanes of a wavefront; every lane gets the result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Block-wide sum for blockDim.x = NT threads (NT a multiple of 64); `red`
// is LDS scratch of at least NT/64 entries. All threads get the result.
template <int NT, typename F>
__device__ __forceinline__ F block_sum(F v, F* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  F s = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC 2011) of the counter (c0, c1, c2, c3) under the key
// (k0, k1): ten rounds, each multiplying two of the four 64-bit words by a
// round constant into 128-bit products and mixing the halves with the other
// words and the key; the key advances by two Weyl increments between rounds.
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64(uint64_t x0, uint64_t x1, uint64_t x2, uint64_t x3, uint64_t k0,
                                           uint64_t k1, uint64_t w[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kPhiloxM0, x0), lo0 = kPhiloxM0 * x0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, x2), lo1 = kPhiloxM1 * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  w[0] = x0;
  w[1] = x1;
  w[2] = x2;
  w[3] = x3;
}

// ---- direct-to-LDS loads and transposing LDS reads (gfx950) ----

typedef short s16x4_t __attribute__((ext_vector_type(4)));
#define MTNLG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// A buffer-load offset past any num_records used here: the load returns zeros.
constexpr uint32_t kOobOffset = 0x80000000u;

// 128-bit buffer resource over `bytes` bytes from p (raw, stride 0): a load at
// an offset past num_records returns zeros and a store there is dropped, so
// ragged edges need no branch around the memory instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                         off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, off, 0, 0);
}

// DPP lane permutation of a float (every source lane valid for the patterns used).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over the 64 lanes of a wavefront without LDS traffic: butterflies over
// pairs and quads (quad_perm), then 8 and 16 lanes (row_half_mirror,
// row_mirror; each pair of partners adds the same two values, so every lane
// of a 16-lane row holds the same sum), then the four row sums in order.
// The result is uniform across the wavefront.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// Buffer resource as four words: 48-bit base, stride 0, num_records bytes,
// and the raw-buffer format word.
__device__ __forceinline__ i32x4_t rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  i32x4_t r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)((a >> 32) & 0xffffu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from a buffer into LDS at m0 + 16*lane. Written as inline
// asm on purpose: the compiler cannot tell which LDS bytes such a load writes
// and would otherwise wait for ALL outstanding loads before every LDS read,
// defeating a prefetch ring; callers wait on vmcnt themselves before the
// barrier that publishes what was loaded.
__device__ __forceinline__ void dtl16(i32x4_t rsrc, const void* lds_base, uint32_t off) {
  // the stage base is the same for every lane; make that explicit for the SGPR operand
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)MTNLG_LDS(lds_base));
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// As dtl16, with the destination given as a 32-bit LDS byte address (no
// generic-to-LDS pointer conversion on the issue path).
__device__ __forceinline__ void dtl16_at(i32x4_t rsrc, uint32_t lds_addr, uint32_t off) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// As dtl16_at, with a wave-uniform byte offset `soff` added to every lane's `off`.
__device__ __forceinline__ void dtl16_at_so(i32x4_t rsrc, uint32_t lds_addr, uint32_t off, uint32_t soff) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds), "s"(so)
               : "memory", "m0");
}

// As dtl16, with a wave-uniform byte offset `soff` added to every lane's `off`.
__device__ __forceinline__ void dtl16_so(i32x4_t rsrc, const void* lds_base, uint32_t off, uint32_t soff) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)MTNLG_LDS(lds_base));
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds), "s"(so)
               : "memory", "m0");
}

__device__ __forceinline__ uint2 ds_read_tr(const char* p) {
  s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, t);
}

// s_waitcnt for at most n outstanding vector-memory loads (vmcnt: bits [3:0] and [15:14]).
#define MTNLG_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

}  // namespace mtnlg
