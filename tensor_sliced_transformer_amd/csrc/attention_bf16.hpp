// Shared pieces of the bf16 attention kernels (gfx950): tile layout in LDS,
// direct-to-LDS tile loads, MFMA fragment reads and the LDS ring walk.
// The kernels themselves and what they compute are described in
// attention_bf16.hip.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace mtnlg {
namespace attn {

constexpr int kRows = 64;      // rows per workgroup block and per streamed tile
constexpr int kRing = 3;       // LDS ring depth (tiles in flight)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Tile {
  static constexpr int EB = D / 32;               // 32-column blocks of head_dim
  static constexpr int SUB = D / 16;              // 16-wide reduction steps over head_dim
  static constexpr int BYTES = kRows * D * 2;     // one 64-row tile
  static constexpr int IPW = BYTES / 1024 / 4;    // 1 KiB loads per wave per tile (= EB)
};

__device__ __forceinline__ int chunk_off(int e, int r, int c) {
  return e * 4096 + r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}

// Per-lane byte offset, relative to the tile's first row and head column, of
// this wave's u-th 1 KiB load: load q = wave*IPW + u covers 32-column block
// q/4 and rows 16*(q%4) .. +15; lane l fills row 16*(q%4) + l/4, LDS slot l%4.
template <int D>
__device__ __forceinline__ uint32_t tile_voff(int wave, int u, int lane, int64_t ld) {
  const int q = wave * Tile<D>::IPW + u;
  const int r = 16 * (q & 3) + (lane >> 2);
  const int c = (lane & 3) ^ ((r >> 2) & 3);
  return (uint32_t)(((int64_t)r * ld + (q >> 2) * 32 + c * 8) * 2);
}

template <int D>
__device__ __forceinline__ void issue_tile(i32x4_t rs, const uint32_t* voff, uint32_t soff, char* dst, int wave) {
#pragma unroll
  for (int u = 0; u < Tile<D>::IPW; ++u) dtl16_so(rs, dst + (wave * Tile<D>::IPW + u) * 1024, voff[u], soff);
}

// 16-byte row fragment: row r, head_dim columns 16*s + 8*g .. +7.
__device__ __forceinline__ bf16x8_t frag_row(const char* tile, int r, int s, int g) {
  const int ch = 2 * s + g;
  return *reinterpret_cast<const bf16x8_t*>(tile + chunk_off(ch >> 2, r, ch & 3));
}

// Transposed fragment of a tile X for the MFMA A operand of X^T Y: lane l
// holds column 32*e + l%32 and, in its 8 reduction slots, rows
// rb + 16*t + 4*g + {0..3} then rb + 16*t + 8 + 4*g + {0..3} (g = l/32): the
// order in which a 32x32 MFMA accumulator holds its rows.
__device__ __forceinline__ bf16x8_t frag_tr(const char* tile, int e, int rb, int t, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int r = rb + 16 * t + 4 * (G >> 1) + (i >> 2);
  const int c = 2 * (G & 1) + ((i & 3) >> 1);
  const uint2 lo = ds_read_tr(tile + chunk_off(e, r, c) + 8 * (i & 1));
  const uint2 hi = ds_read_tr(tile + chunk_off(e, r + 8, c) + 8 * (i & 1));
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Accumulator entries 8t .. 8t+7 as the bf16 B operand matching frag_tr(.., t, ..).
__device__ __forceinline__ bf16x8_t pack_slots(const f32x16_t& a, int t) {
  uint4 u;
  u.x = pack_bf16x2(a[8 * t + 0], a[8 * t + 1]);
  u.y = pack_bf16x2(a[8 * t + 2], a[8 * t + 3]);
  u.z = pack_bf16x2(a[8 * t + 4], a[8 * t + 5]);
  u.w = pack_bf16x2(a[8 * t + 6], a[8 * t + 7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ f32x16_t mma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Q and K are kept in IEEE binary16 (the QKV product writes them so): the
// scores' softmax magnifies their rounding (at the MT-NLG slice the scores
// have a standard deviation near 8), and fp16 carries three more fraction
// bits than bf16. S = Q K^T runs on the fp16 MFMA; a fragment holds the 16-bit
// patterns either way.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16_t mma_f16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}
// dQ = dS K and dK = dS^T Q pair dS with the fp16 Q and K fragments on the
// fp16 MFMA, dS packed as fp16 (pack_slots_f16). The backward kernels compute
// P, and so dS, scaled by 2^-kDsShift (the shift is folded into the
// exponent's offset): fp16 then holds |dS| up to 65504 * 2^kDsShift, and the
// accumulated dQ, dK and dV are multiplied by 2^kDsShift at the end (exact).
constexpr float kDsShift = 8.0f;
constexpr float kDsUp = 256.0f;
__device__ __forceinline__ bf16x8_t pack_slots_f16(const f32x16_t& a, int t) {
  uint4 u;
  u.x = pack_f16x2(a[8 * t + 0], a[8 * t + 1]);
  u.y = pack_f16x2(a[8 * t + 2], a[8 * t + 3]);
  u.z = pack_f16x2(a[8 * t + 4], a[8 * t + 5]);
  u.w = pack_f16x2(a[8 * t + 6], a[8 * t + 7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ void zero(f32x16_t& a) {
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = 0.0f;
}

// Wait until at most k tiles' worth (n loads each) of this wave's loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_tiles(int k) {
  static_assert(2 * N < 64, "vmcnt is 6 bits");
  if (k >= 2) {
    MTNLG_VMCNT(2 * N);
  } else if (k == 1) {
    MTNLG_VMCNT(N);
  } else {
    MTNLG_VMCNT(0);
  }
}

// An empty asm that reads x: the compiler must complete the load of x before
// it. Used on the register-resident operands before the tile loop, so that
// none of their loads is still pending (from the compiler's view) inside the
// loop, where waiting for it would also wait for every prefetch.
__device__ __forceinline__ void settle(const bf16x8_t& x) { asm volatile("" : : "v"(x)); }

// 2^x by the hardware instruction (results below 2^-126 flush to zero, which
// is immaterial next to the softmax row sum of at least 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max and sum of x over lanes l and l ^ 32 (the two halves of a 32x32
// accumulator column), with v_permlane32_swap: the swap puts the other half's
// values beside this half's, in registers (no LDS round trip).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The walk over `count` streamed tiles through the LDS ring. issue(t, stage)
// starts the loads of tile t into a ring stage; body(it, stage) computes on
// tile it. The loop is unrolled by the ring depth so that each stage index,
// and with it every LDS address of the body, is a compile-time offset.
// RING is the number of ring stages (kRing unless a kernel trades depth for a
// second resident workgroup). The caller may have issued tiles 0 .. PRE-1
// itself (ahead of its own register loads, so that both latencies overlap).
template <int NLD, int RING = kRing, int PRE = 0, typename Issue, typename Body>
__device__ __forceinline__ void ring_walk(int count, Issue&& issue, Body&& body) {
  static_assert(PRE <= RING - 1, "at most RING - 1 tiles ahead");
#pragma unroll
  for (int t = PRE; t < RING - 1; ++t)
    if (t < count) issue(t, t);
  for (int it0 = 0; it0 < count; it0 += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      const int it = it0 + j;
      if (it < count) {
        wait_tiles<NLD>(min(RING - 2, count - 1 - it));
        __syncthreads();
        if (it + RING - 1 < count) issue(it + RING - 1, (j + RING - 1) % RING);
        body(it, j);
      }
    }
  }
}

__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// ---- dropout on the attention probabilities ----
//
// Element (b, head, q, k) is kept when the 16-bit draw at bits 16 * (k % 4)
// of word q % 4 of Philox4x64-10 at counter (q / 4, k / 4, head, b), key
// (seed, site), is >= thr (head: the global head index). One generator call
// thus serves a 4 x 4 block of (query, key) pairs, and the four lanes of a
// quad (lanes 4a .. 4a+3) hold, in either accumulator layout, the 16
// elements of four such blocks between them: each lane makes one call and a
// transpose of 4-bit rows across the quad (two DPP exchanges) hands every
// lane its own 16 keep bits.
//   forward / dQ layout (query per lane column): lane 4a+t of a wave whose
//     queries start at qw0 and keys at kw0 draws block
//     (qw0/4 + a, kw0/4 + 2t + g);
//   dK/dV layout (key per lane column): block (qw0/4 + 2t + g, kw0/4 + a),
//     its bits transposed within the 4 x 4 block first.
// Bit i of the result is the keep bit of accumulator slot i.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <bool KEY_LANES>
__device__ __forceinline__ uint32_t attn_keep_bits(const AttnDropout& d, uint64_t c0, uint64_t c1, int head, int b,
                                                   int lane) {
  uint64_t w[4];
  philox4x64(c0, c1, (uint64_t)head, (uint64_t)b, d.seed, d.site, w);
  uint32_t m = 0;  // bit 4r + c: draw c of word r (row r = q % 4, column c = k % 4)
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) m |= (uint32_t)(((w[r] >> (16 * c)) & 0xFFFFu) >= d.thr) << (4 * r + c);
  if (KEY_LANES) {  // bit 4r + c -> bit 4c + r
    uint32_t t = (m ^ (m >> 3)) & 0x0A0Au;
    m ^= t ^ (t << 3);
    t = (m ^ (m >> 6)) & 0x00CCu;
    m ^= t ^ (t << 6);
  }
  // nibble j of lane t' <- nibble t' of lane j (within the quad)
  const int t = lane & 3;
  uint32_t p = dpp_u<0xB1>(m);  // lane t ^ 1
  m = (t & 1) ? ((m & 0xF0F0u) | ((p & 0xF0F0u) >> 4)) : ((m & 0x0F0Fu) | ((p & 0x0F0Fu) << 4));
  p = dpp_u<0x4E>(m);  // lane t ^ 2
  m = (t & 2) ? ((m & 0xFF00u) | ((p & 0xFF00u) >> 8)) : ((m & 0x00FFu) | ((p & 0x00FFu) << 8));
  return m;
}

// dK and dV given the (L, D) pairs the dQ kernel stores (attention_bf16_dkdv.hip).
hipError_t dkdv_bf16(int batch, int seq, int heads, int head_dim, const void* qkv, const void* dout,
                     const float2* ldw, void* dqkv, const AttnDropout& drop, hipStream_t st);

}  // namespace attn
}  // namespace mtnlg
