// Tiled MFMA GEMM for gfx950: C[M,N] = op(A)[M,K] * op(B)[K,N] with an
// epilogue, fp32 accumulation.
//
// Every linear of the sliced layer maps onto this one kernel: the forward
// projections (X W: A K-contiguous, B N-contiguous), the input-gradient
// products (dY W^T: both K-contiguous) and the weight-gradient products
// (X^T dY: both M/N-contiguous), see the layer driver.
//
// Design (CDNA4, wave64). Two code paths share the tile scheduling and the
// epilogue:
//   * bf16 (the layer's path): operand tiles move from memory straight into
//     LDS with buffer_load_dwordx4 ... lds; M/N-contiguous operands stay in
//     their natural layout and MFMA fragments are read with the transposing
//     ds_read_b64_tr_b16, so all four layouts share one MFMA loop.
//       - 256x256 tiles: K tiles 64 deep (a k-contiguous operand row is one
//         128-byte line per tile), a 2-stage LDS ring, 8 waves in a 2x4 grid
//         (128x64 each, two waves per SIMD so one wave's MFMAs cover the
//         other's LDS reads and barrier waits).
//       - 128x128 tiles (small problems): K tiles 32 deep, a 4-stage ring,
//         4 waves in a 2x2 grid.
//   * fp32 (the small checked configuration): register-staged copies into
//     LDS rows of 32 k, M/N-contiguous operands transposed in registers as
//     4x4 micro-blocks; two stages, prefetch distance 2; 4 waves in a 2x2 grid
//     on v_mfma_f32_32x32x2f32.
//   * MFMA blocks are 32x32 (v_mfma_f32_32x32x16_bf16); fragments are
//     double-buffered across 16-deep k-substeps. Out-of-range elements come
//     from buffer loads past num_records (zeros), not from branches.
//   * Work ids are remapped so that each XCD (ids round-robin over 8 XCDs)
//     gets a contiguous range of tiles, walked in groups of 8 tile rows so
//     that concurrently running tiles share operand panels in that XCD's L2.
//   * Wave quantisation: when the last round of tiles would leave at least
//     half the CUs idle, only those leftover tiles are split along K into
//     fp32 partials that a second kernel sums before the epilogue; the pieces
//     are ordered split-major before being handed out per XCD.
//   * The 256x256 kernels are persistent (one workgroup per CU looping over
//     work items): the first K tiles of the next item are loaded while the
//     current item's epilogue runs from a private 16-row LDS slab per wave.
//   * Two 256x256 kernels share that design: when an operand is K-contiguous
//     the tiles go through registers and are written to LDS spread over each K
//     tile (gemm_bf16_rs_kernel); the weight-gradient products (both operands
//     M/N-contiguous) load straight into LDS (gemm_bf16_dtl64_kernel).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mtnlg {

namespace {

constexpr int kCH = 8;        // 16-byte chunks per LDS row
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;  // MI355X: work-group ids go round-robin over 8 XCDs

__device__ __forceinline__ float gelu_f(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_grad_f(float u) {
  const float cdf = 0.5f * (1.0f + erff(u * 0.70710678118654752f));
  const float pdf = 0.39894228040143268f * __expf(-0.5f * u * u);
  return cdf + u * pdf;
}

// Transpose a VECxVEC block held as VEC 16-byte rows: out[i] element j = in[j] element i.
__device__ __forceinline__ void transpose_block(const uint4* in, uint4* out, bf16_t) {
  // in[j] holds 8 bf16 of row j (k = j), dwords hold element pairs (2q, 2q+1).
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[j*4 + d]
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = i >> 1;
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // low half <- element i of row 2q, high half <- element i of row 2q+1
      o[i * 4 + q] = __builtin_amdgcn_perm(w[(2 * q + 1) * 4 + d], w[(2 * q) * 4 + d], sel);
    }
  }
}
__device__ __forceinline__ void transpose_block(const uint4* in, uint4* out, float) {
  const float* f = reinterpret_cast<const float*>(in);
  float* o = reinterpret_cast<float*>(out);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[i * 4 + j] = f[j * 4 + i];
}

// LDS chunk swizzle: 16-byte chunk c of LDS row `row` lives at slot
// c ^ ((row >> 1) & 7). With 128-byte rows, 16 consecutive rows reading the
// same logical chunk then touch 16 distinct 16-byte bank groups (row parity
// picks the half of a 256-byte bank period, the XOR picks the slot in it).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Operands are read through buffer resources (make_rsrc) over the whole
// operand; loads at offsets beyond num_records return zero, which is how
// ragged tiles are handled without branches (an out-of-range element gets the
// offset kOob).
constexpr uint32_t kOob = kOobOffset;

// Loader of one operand tile (R rows of the M or N dimension, BK of K) into
// LDS rows of K. KC: source is K-contiguous (elem(r,k) = p[r*ld + k]),
// otherwise R-contiguous (elem(r,k) = p[k*ld + r]).
template <typename T, int R, bool KC>
struct TileLoader {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BK = kCH * VEC;
  // K-contiguous: R*kCH chunks; R-contiguous: kCH*(R/VEC) micro-blocks of VEC chunks.
  static constexpr int UNITS = KC ? R * kCH : kCH * (R / VEC);
  static constexpr int PER_T = (UNITS + kThreads - 1) / kThreads;
  static constexpr int REGS = KC ? PER_T : PER_T * VEC;
  uint4 st[REGS];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t ld, int r0, int rmax, int k0, int kend,
                                       int tid) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int id = tid + u * kThreads;
      if (KC) {
        const int row = id / kCH, ch = id % kCH;
        const int r = r0 + row, k = k0 + ch * VEC;
        const bool ok = id < UNITS && r < rmax && k < kend;
        const uint32_t off = ok ? (uint32_t)(((int64_t)r * ld + k) * (int64_t)sizeof(T)) : kOob;
        st[u] = buf_load16(rs, off);
      } else {
        // chunk index fastest across lanes: a store instruction then covers every
        // chunk slot of its rows (see store) and a load instruction reads
        // 8 rows x 8 consecutive 16-byte segments
        const int kb = id % kCH, rb = id / kCH;
        const int r = r0 + rb * VEC;
        const bool rok = id < UNITS && r < rmax;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int k = k0 + kb * VEC + j;
          const uint32_t off =
              (rok && k < kend) ? (uint32_t)(((int64_t)k * ld + r) * (int64_t)sizeof(T)) : kOob;
          st[u * VEC + j] = buf_load16(rs, off);
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint4* s, int tid) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int id = tid + u * kThreads;
      if (id >= UNITS) continue;
      if (KC) {
        const int row = id / kCH, ch = id % kCH;
        s[row * kCH + (ch ^ swz(row))] = st[u];
      } else {
        const int kb = id % kCH, rb = id / kCH;
        uint4 t[VEC];
        transpose_block(&st[u * VEC], t, T());
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const int row = rb * VEC + i;
          s[row * kCH + (kb ^ swz(row))] = t[i];
        }
      }
    }
  }
};

// Applies the epilogue to the 8 consecutive fp32 values v of row `row`,
// columns col..col+7 (in range), and stores them.
template <typename T>
__device__ __forceinline__ void apply_epi_store(const GemmArgs& p, int row, int col, float* v) {
  const int64_t off = (int64_t)row * p.ldc + col;
  switch (p.epi) {
    case EPI_GELU_GRAD: {
      float u8[8];
      load8(static_cast<const T*>(p.aux) + off, u8);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= gelu_grad_f(u8[e]);
      store8(static_cast<T*>(p.C) + off, v);
      break;
    }
    case EPI_BIAS_GELU: {
      float b8[8], y8[8];
      load8(static_cast<const T*>(p.bias) + col, b8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] += b8[e];
        y8[e] = gelu_f(v[e]);
      }
      store8(static_cast<T*>(p.C) + off, v);
      store8(static_cast<T*>(p.C2) + off, y8);
      break;
    }
    case EPI_BIAS: {
      float b8[8];
      load8(static_cast<const T*>(p.bias) + col, b8);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += b8[e];
      store8(static_cast<T*>(p.C) + off, v);
      break;
    }
    case EPI_BIAS_F16LO: {
      float b8[8];
      load8(static_cast<const T*>(p.bias) + col, b8);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += b8[e];
      if (col < p.f16_cols) store8_f16(reinterpret_cast<uint16_t*>(static_cast<T*>(p.C) + off), v);
      else store8(static_cast<T*>(p.C) + off, v);
      break;
    }
    default:
      store8(static_cast<T*>(p.C) + off, v);
  }
}

// Epilogue over a staged 32 x WN fp32 slab (row stride SROW floats) whose
// first element is tile-local (rl0, cl0) of the tile at (m0, n0): each lane
// takes 8-wide row vectors and either applies the epilogue (whole tile) or
// stores the raw fp32 values into the tile-major partial `pt` (BN wide) of a
// tail piece. Not unrolled: it touches no register arrays.
template <typename T, int WN, int SROW, int BN>
__device__ __forceinline__ void epilogue_slab(const GemmArgs& p, const float* stage, int m0, int n0, int rl0,
                                              int cl0, int lane, float* pt) {
  constexpr int VPR = WN / 8;  // vectors per slab row
#pragma unroll 1
  for (int u = lane; u < 32 * VPR; u += kWave) {
    const int rr = u / VPR, cc = (u % VPR) * 8;
    float v[8];
    const float4 a = *reinterpret_cast<const float4*>(stage + rr * SROW + cc);
    const float4 b = *reinterpret_cast<const float4*>(stage + rr * SROW + cc + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    if (pt) {
      store8(pt + (int64_t)(rl0 + rr) * BN + cl0 + cc, v);
      continue;
    }
    const int row = m0 + rl0 + rr, col = n0 + cl0 + cc;
    if (row >= p.M || col >= p.N) continue;
    apply_epi_store<T>(p, row, col, v);
  }
}

// ---- epilogue of a 256 x 256 work item (register-staged and direct-to-LDS
// kernels): kind = the launch's GemmArgs::epi for a whole tile, kEpiPart for
// a tail piece (its raw fp32 sums into the piece's slot).
//
// A wave's 128 x 64 block leaves its accumulators in 8 passes of 16 rows
// through the wave's private slab (row r's column c at c ^ (32 * ((r >> 2) &
// 1)), so the two row groups of an accumulator write disjoint banks); lane l
// then takes rows l/8 and l/8 + 8 of the pass, columns 8*(l%8) .. +7, which
// stay the lane's columns for the whole tile. Every global access goes
// through a buffer resource whose range ends at the last row (an offset past
// the last column is moved out of range), so no branch surrounds a memory
// instruction: the pass loop is straight-line, the bias is loaded once per
// tile, the GeLU' input of the next pass is loaded before this pass's
// stores, and no pass waits for the stores of the one before.
constexpr int kEpiPart = 100;

// vector-memory instructions one lane issues in the epilogue of a tile
template <int KIND>
constexpr int epi_vm_ops() {
  return (KIND == EPI_BIAS_GELU || KIND == EPI_GELU_GRAD || KIND == kEpiPart) ? 32 : 16;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack_bf16x8(const float* v) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ uint4 pack_f16x8(const float* v) {
  return make_uint4(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]),
                    pack_f16x2(v[6], v[7]));
}

// The lane's 8 bias values of a tile (loaded before the K loop; zeros past N).
__device__ __forceinline__ uint4 epi_bias_load(const GemmArgs& p, int n0, int wn, int lane) {
  const int col = n0 + wn * 64 + (lane & 7) * 8;
  return buf_load16(make_rsrc(p.bias, (uint32_t)p.N * 2u), col < p.N ? (uint32_t)col * 2u : kOob);
}

// A buffer resource over a bf16 M x ldc matrix from row r0 on (none past M).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, const GemmArgs& p, int r0) {
  const bf16_t* b = static_cast<const bf16_t*>(base) + (int64_t)r0 * p.ldc;
  return make_rsrc(b, r0 < p.M ? (uint32_t)((int64_t)(p.M - r0) * p.ldc * 2) : 0u);
}

// mid() runs before pass FM (halfway): the register-staged kernel writes the
// next item's first K tile to LDS there.
template <int KIND, int FM, int FN, int TN, int BN, typename Mid>
__device__ __forceinline__ void epilogue256(const GemmArgs& p, f32x16_t (&acc)[FM][FN], float* slab, int m0,
                                           int n0, int wm, int wn, int lane, float* pt, uint4 bias_raw,
                                           Mid&& mid) {
  static_assert(TN == 64, "lane columns assume 64-column wave blocks");
  constexpr int TM = FM * 32;
  // Opaque lane id: the slab and store offsets below depend only on the lane
  // and wave, and without this the compiler computes them once per kernel and
  // keeps them live across every item's K loop (up to 14 of them spilled, and
  // each reload waited for all stores in flight).
  asm volatile("" : "+v"(lane));
  const int lrow = lane & 31, lg = lane >> 5;
  const int rr = lane >> 3, cc = (lane & 7) * 8;
  const int col = n0 + wn * TN + cc;
  const int row_w = m0 + wm * TM;
  uint32_t vo[2];  // bytes from a pass's first row, rows rr and rr + 8 (bf16 outputs and aux)
#pragma unroll
  for (int q = 0; q < 2; ++q)
    vo[q] = col < p.N ? (uint32_t)(((int64_t)(rr + 8 * q) * p.ldc + col) * 2) : kOob;
  float bias[8];
  unpack_bf16x8(bias_raw, bias);
  const bool f16 = col < p.f16_cols;
  uint4 ax[2][2];  // GeLU' inputs of a pass, double-buffered by pass parity
  auto aux_load = [&](int pass, uint4* dst) {
    const __amdgpu_buffer_rsrc_t r = rows_rsrc(p.aux, p, row_w + 16 * pass);
#pragma unroll
    for (int q = 0; q < 2; ++q) dst[q] = buf_load16(r, vo[q]);
  };
  if constexpr (KIND == EPI_GELU_GRAD) aux_load(0, ax[0]);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (i == FM / 2) mid();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int pass = 2 * i + hh;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 8 * b + 4 * lg + r;
            slab[row * TN + ((j * 32 + lrow) ^ (32 * ((row >> 2) & 1)))] = acc[i][j][(2 * hh + b) * 4 + r];
          }
      if constexpr (KIND == EPI_GELU_GRAD)
        if (pass + 1 < 2 * FM) aux_load(pass + 1, ax[(pass + 1) & 1]);
      const int prow = row_w + 16 * pass;
      __amdgpu_buffer_rsrc_t rc;
      if constexpr (KIND == kEpiPart)
        rc = make_rsrc(pt, 256u * BN * 4u);
      else
        rc = rows_rsrc(p.C, p, prow);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int sr = rr + 8 * q;
        const float* sp = slab + sr * TN + (cc ^ (32 * ((sr >> 2) & 1)));
        const float4 a = *reinterpret_cast<const float4*>(sp);
        const float4 c = *reinterpret_cast<const float4*>(sp + 4);
        float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        if constexpr (KIND == kEpiPart) {
          const uint32_t po = (uint32_t)(((wm * TM + 16 * pass + sr) * BN + wn * TN + cc) * 4);
          buf_store16(rc, po, __builtin_bit_cast(uint4, a));
          buf_store16(rc, po + 16, __builtin_bit_cast(uint4, c));
        } else if constexpr (KIND == EPI_GELU_GRAD) {
          float u[8];
          unpack_bf16x8(ax[pass & 1][q], u);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= gelu_grad_f(u[e]);
          buf_store16(rc, vo[q], pack_bf16x8(v));
        } else if constexpr (KIND == EPI_BIAS_GELU) {
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] += bias[e];
            y[e] = gelu_f(v[e]);
          }
          buf_store16(rc, vo[q], pack_bf16x8(v));
          buf_store16(rows_rsrc(p.C2, p, prow), vo[q], pack_bf16x8(y));
        } else if constexpr (KIND == EPI_BIAS || KIND == EPI_BIAS_F16LO) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += bias[e];
          if constexpr (KIND == EPI_BIAS_F16LO)
            buf_store16(rc, vo[q], f16 ? pack_f16x8(v) : pack_bf16x8(v));
          else
            buf_store16(rc, vo[q], pack_bf16x8(v));
        } else {
          buf_store16(rc, vo[q], pack_bf16x8(v));
        }
      }
    }
  }
}

// Runs body(integral_constant<kind>) for a work item of a kernel built for
// epilogue EPI: EPI itself for a whole tile, kEpiPart for a tail piece. (The
// kind is a kernel template parameter: one kernel holding every kind's code
// spilled registers around the epilogue, and a spill reload waits for every
// store in flight.)
template <int EPI, typename Body>
__device__ __forceinline__ void epi_dispatch(bool piece, Body&& body) {
  if (piece)
    body(std::integral_constant<int, kEpiPart>{});
  else
    body(std::integral_constant<int, EPI>{});
}

// Tile position of tile index L: groups of kGroupM tile rows, walked column by column.
__device__ __forceinline__ void tile_pos(const GemmArgs& p, int L, int& tm, int& tn) {
  const int group = kGroupM * p.tiles_n;
  const int gq = L / group;
  const int first_m = gq * kGroupM;
  const int gm = min(p.tiles_m - first_m, kGroupM);
  tm = first_m + (L % group) % gm;
  tn = (L % group) / gm;
}

// Tile index L, K range and tail piece (split < 0: whole tile) of work item w.
// Consecutive ids go round-robin over the 8 XCDs (XCD w & 7), so each XCD is
// given a contiguous range of whole tiles, and of tail pieces ordered
// split-major: the pieces sharing an XCD's L2 then cover one K range of
// neighbouring tiles rather than every K range of one tile row.
struct TileWork {
  int tm, tn, split, tl, kbeg, kend;
};
__device__ __forceinline__ TileWork tile_work(const GemmArgs& p, int w) {
  TileWork t;
  int L;
  const int xcd = w & 7;
  if (w < p.nfull) {
    const int idx = w >> 3;
    const int base = p.nfull >> 3, rem = p.nfull & 7;
    L = xcd * base + min(xcd, rem) + idx;
    t.split = -1;
    t.tl = 0;
    t.kbeg = 0;
    t.kend = p.K;
  } else {
    const int np = p.tail_tiles * p.tail_split;
    const int u = w - p.nfull;
    // pieces u on this XCD are u0, u0 + 8, ...; XCDs before it own the first pieces in split-major order
    const int u0 = (xcd - p.nfull) & 7;
    int first = 0;
    for (int y = 0; y < xcd; ++y) {
      const int uy = (y - p.nfull) & 7;
      first += uy < np ? (np - uy + 7) >> 3 : 0;
    }
    const int v = first + ((u - u0) >> 3);
    t.tl = v % p.tail_tiles;
    t.split = v / p.tail_tiles;
    L = p.nfull + t.tl;
    t.kbeg = t.split * p.k_chunk;
    t.kend = min(p.K, t.kbeg + p.k_chunk);
  }
  tile_pos(p, L, t.tm, t.tn);
  return t;
}

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  // One 16-byte chunk per lane = 8 consecutive k for one row: one 32x32x16 MFMA.
  static __device__ __forceinline__ void run(const uint4& a, const uint4& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // One chunk = 4 consecutive k; the lane group (lane/32) picks the k slot of
  // 32x32x2, element j the MFMA: A and B use the same mapping, so the sum is exact.
  static __device__ __forceinline__ void run(const uint4& a, const uint4& b, f32x16_t& c) {
    const float* fa = reinterpret_cast<const float*>(&a);
    const float* fb = reinterpret_cast<const float*>(&b);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[j], fb[j], c, 0, 0, 0);
  }
};

template <typename T, int BM, int BN, int WM, int WN, bool A_KC, bool B_KC>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
  static_assert(WM * WN == kThreads / kWave, "4 waves");
  using E = Elem<T>;
  constexpr int VEC = E::VEC;
  constexpr int BK = kCH * VEC;
  constexpr int TM = BM / WM, TN = BN / WN;      // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;      // 32x32 MFMA blocks per wave
  static_assert(FM * 32 == TM && FN * 32 == TN, "wave tile must be a multiple of 32");
  constexpr int SUB = kCH / 2;                   // MFMA k-substeps per K tile
  __shared__ uint4 smem[2 * (BM + BN) * kCH];
  uint4* const sA0 = smem;                        // two A stages, then two B stages
  uint4* const sB0 = smem + 2 * BM * kCH;

  const TileWork tw = tile_work(p, blockIdx.x);
  const int m0 = tw.tm * BM, n0 = tw.tn * BN;
  const int kbeg = tw.kbeg, kend = tw.kend;
  const int nk = (kend - kbeg + BK - 1) / BK;
  float* const pt = tw.split >= 0 ? p.part + ((int64_t)tw.split * p.tail_tiles + tw.tl) * BM * BN : nullptr;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane & 31, lg = lane >> 5;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.M * p.K * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, (uint32_t)((int64_t)p.K * p.N * sizeof(T)));

  TileLoader<T, BM, A_KC> la;
  TileLoader<T, BN, B_KC> lb;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // per-lane LDS row offsets (in chunks) of this wave's fragments
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = (wm * TM + i * 32 + lrow) * kCH;
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = (wn * TN + j * 32 + lrow) * kCH;
  const int sw = swz(lrow);  // the same for every fragment row of this lane (rows start at multiples of 32)

  uint4 af[2][FM], bfr[2][FN];
  auto load_frags = [&](const uint4* a_s, const uint4* b_s, int s, int buf) {
    const int ch = (2 * s + lg) ^ sw;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[buf][i] = a_s[arow[i] + ch];
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[buf][j] = b_s[brow[j] + ch];
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) Mfma<T>::run(af[buf][i], bfr[buf][j], acc[i][j]);
  };

  if (nk > 0) {
    la.load(ra, p.lda, m0, p.M, kbeg, kend, tid);
    lb.load(rb, p.ldb, n0, p.N, kbeg, kend, tid);
    la.store(sA0, tid);
    lb.store(sB0, tid);
    if (nk > 1) {
      la.load(ra, p.lda, m0, p.M, kbeg + BK, kend, tid);
      lb.load(rb, p.ldb, n0, p.N, kbeg + BK, kend, tid);
    }
    __syncthreads();
    load_frags(sA0, sB0, 0, 0);
  }

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    const uint4* a_s = sA0 + cur * BM * kCH;
    const uint4* b_s = sB0 + cur * BN * kCH;
    uint4* a_n = sA0 + nxt * BM * kCH;
    uint4* b_n = sB0 + nxt * BN * kCH;
    // tile kt+1 (loaded during tile kt-1) goes to the other stage; then start tile kt+2
    if (kt + 1 < nk) {
      la.store(a_n, tid);
      lb.store(b_n, tid);
    }
    if (kt + 2 < nk) {
      const int k0 = kbeg + (kt + 2) * BK;
      la.load(ra, p.lda, m0, p.M, k0, kend, tid);
      lb.load(rb, p.ldb, n0, p.N, k0, kend, tid);
    }
#pragma unroll
    for (int s = 0; s < SUB - 1; ++s) {
      load_frags(a_s, b_s, s + 1, (s + 1) & 1);
      mfmas(s & 1);
    }
    // one barrier per K tile: every wave has finished writing stage `nxt` and
    // reading stage `cur` (its last fragments are in registers)
    __syncthreads();
    if (kt + 1 < nk) load_frags(a_n, b_n, 0, SUB & 1);
    mfmas((SUB - 1) & 1);
  }

  // ---- epilogue: stage one 32-row slab of each wave's sub-tile in LDS (now
  // free), then write 8-wide row vectors; the MFMA output layout (lane: column
  // lrow, rows 8*blk + 4*lg + r) is turned into row-contiguous stores here.
  __syncthreads();
  constexpr int SROW = TN + 4;  // padded so the two lane groups' rows hit different banks
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * SROW;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) stage[(8 * blk + 4 * lg + r) * SROW + j * 32 + lrow] = acc[i][j][blk * 4 + r];
    __syncthreads();
    epilogue_slab<T, TN, SROW, BN>(p, stage, m0, n0, wm * TM + i * 32, wn * TN, lane, pt);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 GEMM with direct-to-LDS loads, 32-deep K tiles (128x128 tiles)
//
// * Operand tiles move from HBM/L2 to LDS with buffer_load_dwordx4 ... lds:
//   no staging registers and no ds_write; lane l of a wave instruction lands
//   at base + 16*l, so the swizzle is applied to the GLOBAL address each lane
//   fetches. A ring of kStages K-tiles of 32 (bf16) lets the loads of tile
//   t+kStages-1 start while tile t is multiplied (three tiles of slack).
// * K-contiguous operands: LDS rows of 32 k (64 B = 4 chunks); chunk c of
//   row r sits at slot c ^ ((r >> 2) & 3), so 16 rows read by one MFMA
//   operand fetch (ds_read_b128) hit 16 distinct 16-byte bank groups.
// * M/N-contiguous operands stay in their natural layout in LDS (rows of k,
//   R elements each, chunk c of row k at slot c ^ (4 * (k & 3))) and MFMA
//   fragments are read with ds_read_b64_tr_b16: within 16 lanes, lane i
//   supplies the 8 bytes at (row k0 + i/4, elements 4*(i%4)..+3) and lane j
//   receives element j%4.. i.e. 4 consecutive k of element j -- exactly half
//   of a 32x32x16 operand fragment; two reads make the 8 k of a lane.
// * One barrier per K-tile, between its two k-substeps: it publishes tile
//   t+1 (loads waited with vmcnt) and frees the stage of tile t-1 for the next
//   prefetch, while the fragments of the next substep are read ahead.
// ---------------------------------------------------------------------------
#ifndef MTNLG_GEMM_STAGES
#define MTNLG_GEMM_STAGES 4
#endif
constexpr int kStages = MTNLG_GEMM_STAGES;  // K-tiles in the LDS ring
constexpr int kBKd = 32;                    // bf16 K per stage

// One operand of the direct-to-LDS GEMM: R rows of M (or N) per tile.
template <int R, bool KC, int NW>
struct DtlOperand {
  static constexpr int STAGE_BYTES = R * kBKd * 2;
  static constexpr int INSTR = STAGE_BYTES / 1024;     // 1 KiB per wave-wide load
  static constexpr int PER_WAVE = INSTR / NW;
  static constexpr int RB = R * 2;                     // bytes per LDS row (MN layout)
  static_assert(PER_WAVE >= 1 && INSTR % NW == 0, "tile too small");
  // per-lane, per-instruction (row/col) of the element this lane fetches
  int r_[PER_WAVE];      // M/N index within the tile (KC) or k within the tile (MN)
  int c_[PER_WAVE];      // k within the tile (KC) or M/N index within the tile (MN)

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int q = wave * PER_WAVE + u;
      if (KC) {
        const int r = q * 16 + lane / 4;                 // 16 rows of 64 B per KiB
        const int slot = lane & 3;
        r_[u] = r;
        c_[u] = 8 * (slot ^ ((r >> 2) & 3));
      } else {
        const int rows_per = 1024 / RB;                  // 2 (R=256) or 4 (R=128)
        const int k = q * rows_per + (16 * lane) / RB;
        const int slot = ((16 * lane) % RB) / 16;
        r_[u] = k;
        c_[u] = 8 * (slot ^ (4 * (k & 3)));
      }
    }
  }

  // issue this wave's u-th load of the K-tile starting at k0 into stage `dst`
  __device__ __forceinline__ void load_one(int u, i32x4_t rs, int64_t ld, int r0, int rmax, int k0, int kend,
                                           char* dst, int wave) const {
    const int q = wave * PER_WAVE + u;
    uint32_t off;
    if (KC) {
      const int m = r0 + r_[u], k = k0 + c_[u];
      off = (m < rmax && k < kend) ? (uint32_t)(((int64_t)m * ld + k) * 2) : kOob;
    } else {
      const int k = k0 + r_[u], m = r0 + c_[u];
      off = (m < rmax && k < kend) ? (uint32_t)(((int64_t)k * ld + m) * 2) : kOob;
    }
    dtl16(rs, dst + q * 1024, off);
  }
};

// Byte offset (within a stage) of this lane's fragment of the 32-row block
// starting at tile row `rb32*32`, k-substep s (16 k): KC operand via b128.
__device__ __forceinline__ int kc_frag_off(int rb32, int s, int lane) {
  const int fr = lane & 31, g = lane >> 5;
  const int r = rb32 * 32 + fr;
  return r * 64 + (((2 * s + g) ^ ((fr >> 2) & 3)) * 16);
}
// MN operand via two transposing reads; returns the offset of read h = 0 (h = 1 adds 4 rows).
template <int RB>
__device__ __forceinline__ int mn_frag_off(int rb32, int s, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int k = s * 16 + 8 * (G >> 1) + (i >> 2);
  const int c = 4 * (rb32 ^ (i >> 2)) + 2 * (G & 1) + ((i >> 1) & 1);
  return k * RB + c * 16 + 8 * (i & 1);
}

template <int BM, int BN, bool A_KC, bool B_KC, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_dtl_kernel(GemmArgs p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  using OA = DtlOperand<BM, A_KC, NW>;
  using OB = DtlOperand<BN, B_KC, NW>;
  constexpr int SA = OA::STAGE_BYTES, SB = OB::STAGE_BYTES, SS = SA + SB;
  __shared__ __align__(1024) char smem[kStages * SS];

  const TileWork tw = tile_work(p, blockIdx.x);
  const int m0 = tw.tm * BM, n0 = tw.tn * BN;
  const int kbeg = tw.kbeg, kend = tw.kend;
  const int nk = (kend - kbeg + kBKd - 1) / kBKd;
  float* const pt = tw.split >= 0 ? p.part + ((int64_t)tw.split * p.tail_tiles + tw.tl) * BM * BN : nullptr;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const i32x4_t ra = rsrc_words(p.A, (uint32_t)((int64_t)p.M * p.K * 2));
  const i32x4_t rb = rsrc_words(p.B, (uint32_t)((int64_t)p.K * p.N * 2));
  OA oa;
  OB ob;
  oa.init(wave, lane);
  ob.init(wave, lane);

  // fragment offsets within a stage (substep 0; substep 1 adds a constant)
  int aoff[FM], boff[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
    aoff[i] = A_KC ? kc_frag_off(wm * FM + i, 0, lane) : mn_frag_off<OA::RB>(wm * FM + i, 0, lane);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    boff[j] = SA + (B_KC ? kc_frag_off(wn * FN + j, 0, lane) : mn_frag_off<OB::RB>(wn * FN + j, 0, lane));
  // substep 1 offset: KC: chunk 2s+g -> the XOR with a lane constant of (2 + ...) ; handled by recomputing
  int aoff1[FM], boff1[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
    aoff1[i] = A_KC ? kc_frag_off(wm * FM + i, 1, lane) : mn_frag_off<OA::RB>(wm * FM + i, 1, lane);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    boff1[j] = SA + (B_KC ? kc_frag_off(wn * FN + j, 1, lane) : mn_frag_off<OB::RB>(wn * FN + j, 1, lane));

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint4 af[2][FM], bfr[2][FN];
  auto read_frags = [&](const char* st, int s, int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const char* q = st + (s ? aoff1[i] : aoff[i]);
      if (A_KC) {
        af[buf][i] = *reinterpret_cast<const uint4*>(q);
      } else {
        const uint2 lo = ds_read_tr(q), hi = ds_read_tr(q + 4 * OA::RB);
        af[buf][i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const char* q = st + (s ? boff1[j] : boff[j]);
      if (B_KC) {
        bfr[buf][j] = *reinterpret_cast<const uint4*>(q);
      } else {
        const uint2 lo = ds_read_tr(q), hi = ds_read_tr(q + 4 * OB::RB);
        bfr[buf][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  };
  // Loads of K-tile t: its A half is issued during substep 1 of tile t-(S-1),
  // its B half during substep 0 of tile t-(S-2), one load after every few
  // MFMAs so the issue cost hides under the matrix core. Stage t % S is free
  // once every wave has passed the barrier of tile t-(S-1) (they have all
  // finished tile t-S by then).
  constexpr int S = kStages;
  static_assert(OA::PER_WAVE == OB::PER_WAVE, "square tiles");
  constexpr int ND = OA::PER_WAVE;          // loads per half tile per lane
  constexpr int NM = FM * FN;               // MFMAs per substep
  static_assert(NM % ND == 0, "interleave");
  auto load_a = [&](int t, int u) {
    char* st = smem + (t % S) * SS;
    oa.load_one(u, ra, p.lda, m0, p.M, kbeg + t * kBKd, kend, st, wave);
  };
  auto load_b = [&](int t, int u) {
    char* st = smem + (t % S) * SS;
    ob.load_one(u, rb, p.ldb, n0, p.N, kbeg + t * kBKd, kend, st + SA, wave);
  };
  // the MFMAs of one substep with the loads of one half tile (t < 0: none) woven in
  auto mfmas_with = [&](int buf, int t, bool half_a) {
#pragma unroll
    for (int idx = 0; idx < NM; ++idx) {
      Mfma<bf16_t>::run(af[buf][idx / FN], bfr[buf][idx % FN], acc[idx / FN][idx % FN]);
      if ((idx + 1) % (NM / ND) == 0 && t >= 0) {
        __builtin_amdgcn_sched_barrier(0);
        if (half_a) load_a(t, (idx + 1) / (NM / ND) - 1);
        else load_b(t, (idx + 1) / (NM / ND) - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // s_waitcnt immediate for vmcnt(n) alone (expcnt and lgkmcnt at their maxima);
  // vmcnt is 6 bits, low 4 in [3:0], high 2 in [15:14]
  constexpr int W0 = 0x0F70;
  static_assert((2 * (S - 3) + 1) * ND < 64, "vmcnt is 6 bits");
  // wait until at most h half-tiles of this lane's loads are outstanding
  auto wait_halves = [&](int h) {
#define MTNLG_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
    switch (h) {
      case 0: MTNLG_VM(0); break;
      case 1: MTNLG_VM(ND); break;
      case 2: MTNLG_VM(2 * ND); break;
      case 3: MTNLG_VM(3 * ND); break;
      case 4: MTNLG_VM(4 * ND); break;
      default: MTNLG_VM(5 * ND); break;
    }
#undef MTNLG_VM
  };
  static_assert(2 * (S - 3) + 1 <= 5, "extend wait_halves");

  // prologue: tiles 0 .. S-3 whole and the A half of tile S-2; then tile 0 must be complete
  for (int t = 0; t < S - 2 && t < nk; ++t)
    for (int u = 0; u < ND; ++u) { load_a(t, u); load_b(t, u); }
  if (S - 2 < nk)
    for (int u = 0; u < ND; ++u) load_a(S - 2, u);
  if (nk > 0) {
    const int whole = min(nk - 1, S - 3);                 // tiles 1 .. S-3 that exist
    wait_halves(2 * whole + (S - 2 < nk ? 1 : 0));
    __syncthreads();
    read_frags(smem, 0, 0);
  }

  for (int kt = 0; kt < nk; ++kt) {
    const char* st = smem + (kt % S) * SS;
    read_frags(st, 1, 1);
    mfmas_with(0, kt + S - 2 < nk ? kt + S - 2 : -1, false);   // B half of tile kt+S-2
    // publish tile kt+1: tiles kt+2 .. kt+S-2 may still be in flight
    if (kt + 1 < nk) wait_halves(2 * min(nk - 2 - kt, S - 3));
    __syncthreads();
    if (kt + 1 < nk) read_frags(smem + ((kt + 1) % S) * SS, 0, 0);
    mfmas_with(1, kt + S - 1 < nk ? kt + S - 1 : -1, true);    // A half of tile kt+S-1
  }

  // ---- epilogue: through LDS, one 32-row slab of the wave's sub-tile at a time ----
  __builtin_amdgcn_s_waitcnt(W0);  // no load may still be writing LDS (all waited above)
  __syncthreads();
  constexpr int SROW = TN + 4;
  static_assert(NW * 32 * SROW * 4 <= kStages * SS, "epilogue staging exceeds the ring");
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * SROW;
  const int lrow = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) stage[(8 * blk + 4 * lg + r) * SROW + j * 32 + lrow] = acc[i][j][blk * 4 + r];
    __syncthreads();
    epilogue_slab<bf16_t, TN, SROW, BN>(p, stage, m0, n0, wm * TM + i * 32, wn * TN, lane, pt);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 GEMM with direct-to-LDS loads, 64-deep K tiles (256x256 tiles)
//
// * k-contiguous operands: LDS rows of 64 k (128 B = 8 chunks), chunk c of
//   row r at slot c ^ ((r >> 1) & 7): the 8 rows that one 16-byte operand
//   read serves at a time land in 8 distinct bank groups, and each row of a
//   tile is one whole 128-byte line in memory.
// * M/N-contiguous operands: as in the 32-deep kernel, 64 rows of k.
// * A 2-stage ring (2 x 64 KiB) and one barrier per K tile, placed before
//   the tile's last k-substep: by then every fragment of the tile is in
//   registers, so the barrier both publishes tile t+1 and frees the stage of
//   tile t. The last substep's MFMAs then cover the first fragment reads of
//   tile t+1 and the loads of tile t+2 into the freed stage, which have a
//   whole tile to land before the next barrier waits for them (vmcnt). Those
//   loads come from one wave per SIMD only.
// * Each substep issues all reads of the next substep's fragments right
//   after its first MFMA, in the order the next substep consumes them, so
//   they have the rest of the substep to arrive.
// * The direct-to-LDS destination (m0) is computed as a 32-bit LDS address
//   from the array base, not from a generic pointer.
// * Persistent: one workgroup per CU (the ring fills LDS anyway) takes work
//   items b, b + 256, ... Once an item's last fragments are read, the first
//   two K tiles of the next item are issued into the ring and the epilogue
//   runs from a private 16 x 64 fp32 slab per wave (the 32 KiB left beside
//   the ring, so no workgroup barrier), hiding the next item's load latency
//   behind the epilogue (+1 to 2.5% on the K = 2048 weight-gradient shapes).
// * Per-lane load and fragment offsets are affine in the load index and the
//   k-substep, so only their bases are kept, and they are recomputed per work
//   item so that they are not live across the epilogue (no VGPR spills at the
//   256-register budget of two waves per SIMD).
// ---------------------------------------------------------------------------
constexpr int kBK64 = 64;

template <int R, bool KC, int NW>
struct Dtl64 {
  static constexpr int STAGE_BYTES = R * kBK64 * 2;
  static constexpr int INSTR = STAGE_BYTES / 1024;
  static constexpr int PER_WAVE = INSTR / NW;
  static constexpr int RB = R * 2;  // MN layout: bytes per k row
  // rows (KC: of M/N, MN: of k) that one wave-wide KiB load covers
  static constexpr int STEP = KC ? 8 : 1024 / RB;
  static_assert(PER_WAVE >= 1 && INSTR % NW == 0, "tile too small");
  static_assert(PER_WAVE % 2 == 0 && (KC || RB == 512), "slot pattern assumes even loads per wave, 256-wide MN rows");
  // Load q = wave * PER_WAVE + u covers row r0 + (q - wave * PER_WAVE) * STEP;
  // its column within the row depends only on q's parity (cpar[q & 1]).
  int r0, cpar[2];
  __device__ __forceinline__ void init(int wave, int lane) {
    const int q = wave * PER_WAVE;  // even
    if (KC) {
      r0 = q * 8 + lane / 8;        // 8 rows of 128 B per KiB
      const int slot = lane & 7;    // chunk slot ^ ((r >> 1) & 7), (r >> 1) & 7 = 4 (q & 1) + lane / 16
#pragma unroll
      for (int e = 0; e < 2; ++e) cpar[e] = 8 * (slot ^ (4 * e + lane / 16));
    } else {
      r0 = q * 2 + lane / 32;       // 2 k rows of 512 B per KiB
      const int slot = lane & 31;   // chunk slot ^ 4 (k & 3), k & 3 = 2 (q & 1) + lane / 32
#pragma unroll
      for (int e = 0; e < 2; ++e) cpar[e] = 8 * (slot ^ (4 * (2 * e + lane / 32)));
    }
  }
  // byte offset in the operand of load u (+ QOFF) of the K-tile at k0 (kOob outside it)
  template <int QOFF = 0>
  __device__ __forceinline__ uint32_t goff(int u, int64_t ld, int rb0, int rmax, int k0, int kend) const {
    const int r = r0 + (u + QOFF) * STEP, c = cpar[u & 1];
    if (KC) {
      const int m = rb0 + r, k = k0 + c;
      return (m < rmax && k < kend) ? (uint32_t)(((int64_t)m * ld + k) * 2) : kOob;
    }
    const int k = k0 + r, m = rb0 + c;
    return (m < rmax && k < kend) ? (uint32_t)(((int64_t)k * ld + m) * 2) : kOob;
  }
  // issue load u (+ QOFF, an even count of loads of other waves) of the K-tile at k0 into the stage at dst
  template <int QOFF = 0>
  __device__ __forceinline__ void load_one(int u, i32x4_t rs, int64_t ld, int rb0, int rmax, int k0, int kend,
                                           uint32_t dst, int wave) const {
    dtl16_at(rs, dst + (uint32_t)(wave * PER_WAVE + u + QOFF) * 1024u, goff<QOFF>(u, ld, rb0, rmax, k0, kend));
  }
  // Whole K tiles (every K tile of every item in range; M/N-contiguous
  // layout): the lane's byte offset of its first k row at the item's first k,
  // per column parity (kOob past rmax); load u (+ QOFF) of K tile t adds the
  // wave-uniform rest, (64 t + (u + QOFF) STEP) rows, as the instruction's
  // scalar offset, so a load costs no vector arithmetic.
  uint32_t vbase[2];
  __device__ __forceinline__ void item_base(int64_t ld, int rb0, int rmax, int kbeg) {
    static_assert(!KC, "scalar-offset loads are for the M/N-contiguous layout");
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int m = rb0 + cpar[e];
      vbase[e] = m < rmax ? (uint32_t)(((int64_t)(kbeg + r0) * ld + m) * 2) : kOob;
    }
  }
  template <int QOFF = 0>
  __device__ __forceinline__ void load_fullk(int u, i32x4_t rs, int64_t ld, int t, uint32_t dst, int wave) const {
    const uint32_t so = (uint32_t)(((int64_t)t * kBK64 + (u + QOFF) * STEP) * ld * 2);
    dtl16_at_so(rs, dst + (uint32_t)(wave * PER_WAVE + u + QOFF) * 1024u, vbase[u & 1], so);
  }
};

__device__ __forceinline__ int kc64_frag_off(int rb32, int s, int lane) {
  const int r = rb32 * 32 + (lane & 31);
  const int c = 2 * s + (lane >> 5);
  return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

template <int BM, int BN, bool A_KC, bool B_KC, int WM, int WN, int EPI, bool FULLK>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_dtl64_kernel(GemmArgs p) {
  static_assert(!FULLK || (!A_KC && !B_KC), "scalar-offset loads only for M/N-contiguous operands");
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  using OA = Dtl64<BM, A_KC, NW>;
  using OB = Dtl64<BN, B_KC, NW>;
  constexpr int SA = OA::STAGE_BYTES, SB = OB::STAGE_BYTES, SS = SA + SB;
  // the ring, then one private 16-row epilogue slab per wave
  constexpr int ESLAB = 16 * TN;  // floats
  __shared__ __align__(1024) char smem[2 * SS + NW * ESLAB * 4];

  // Persistent: workgroup b takes work items b, b + gridDim.x, ... (gridDim.x a
  // multiple of 8, so every item of a workgroup maps to the XCD it runs on).
  const int total = p.nfull + p.tail_tiles * p.tail_split;
  int w = blockIdx.x;
  if (w >= total) return;
  TileWork tw = tile_work(p, w);
  int m0 = tw.tm * BM, n0 = tw.tn * BN;
  int kbeg = tw.kbeg, kend = tw.kend;
  int nk = (kend - kbeg + kBK64 - 1) / kBK64;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t lds0 = (uint32_t)(uintptr_t)MTNLG_LDS(smem);
  const i32x4_t ra = rsrc_words(p.A, (uint32_t)((int64_t)p.M * p.K * 2));
  const i32x4_t rb = rsrc_words(p.B, (uint32_t)((int64_t)p.K * p.N * 2));
  OA oa;
  OB ob;
  constexpr int AN = A_KC ? 4 : FM, BN_ = B_KC ? 4 : FN;
  int abase[AN], bbase[BN_];
  // Per-lane offsets, (re)computed for every work item from an opaque copy of
  // the lane id so that they are not kept live across the epilogue.
  auto lane_setup = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    oa.init(wave, ln);
    ob.init(wave, ln);
#pragma unroll
    for (int e = 0; e < AN; ++e)
      abase[e] = A_KC ? kc64_frag_off(wm * FM, e, ln) : mn_frag_off<OA::RB>(wm * FM + e, 0, ln);
#pragma unroll
    for (int e = 0; e < BN_; ++e)
      bbase[e] = SA + (B_KC ? kc64_frag_off(wn * FN, e, ln) : mn_frag_off<OB::RB>(wn * FN + e, 0, ln));
  };
  auto aoff = [&](int s, int i) { return A_KC ? abase[s] + i * 4096 : abase[i] + s * 16 * OA::RB; };
  auto boff = [&](int s, int j) { return B_KC ? bbase[s] + j * 4096 : bbase[j] + s * 16 * OB::RB; };

  f32x16_t acc[FM][FN];
  uint4 af[2][FM], bfr[2][FN];
  // fragments are read in the order the MFMAs consume them: a0, b0 .. b(FN-1), a1 .. a(FM-1)
  auto read_a = [&](const char* st, int s, int buf, int i) {
    const char* q = st + aoff(s, i);
    if (A_KC) {
      af[buf][i] = *reinterpret_cast<const uint4*>(q);
    } else {
      const uint2 lo = ds_read_tr(q), hi = ds_read_tr(q + 4 * OA::RB);
      af[buf][i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  auto read_b = [&](const char* st, int s, int buf, int j) {
    const char* q = st + boff(s, j);
    if (B_KC) {
      bfr[buf][j] = *reinterpret_cast<const uint4*>(q);
    } else {
      const uint2 lo = ds_read_tr(q), hi = ds_read_tr(q + 4 * OB::RB);
      bfr[buf][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  auto read_frags = [&](const char* st, int s, int buf) {
    read_a(st, s, buf, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) read_b(st, s, buf, j);
#pragma unroll
    for (int i = 1; i < FM; ++i) read_a(st, s, buf, i);
  };
  // every wave's share of K-tile t of the tile at (tm0, tn0) from k offset kb
  // (FULLK: of the item whose bases item_base set)
  auto issue = [&](int t, int tm0, int tn0, int kb, int ke) {
    const uint32_t st = lds0 + (uint32_t)((t & 1) * SS);
#pragma unroll
    for (int u = 0; u < OA::PER_WAVE; ++u) {
      if constexpr (FULLK) oa.load_fullk(u, ra, p.lda, t, st, wave);
      else oa.load_one(u, ra, p.lda, tm0, p.M, kb + t * kBK64, ke, st, wave);
    }
#pragma unroll
    for (int u = 0; u < OB::PER_WAVE; ++u) {
      if constexpr (FULLK) ob.load_fullk(u, rb, p.ldb, t, st + SA, wave);
      else ob.load_one(u, rb, p.ldb, tn0, p.N, kb + t * kBK64, ke, st + SA, wave);
    }
  };
  auto item_bases = [&]() {
    if constexpr (FULLK) {
      oa.item_base(p.lda, m0, p.M, kbeg);
      ob.item_base(p.ldb, n0, p.N, kbeg);
    }
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        Mfma<bf16_t>::run(af[buf][i], bfr[buf][j], acc[i][j]);
      }
  };

  // Schedule of one substep: its first MFMA, then every read of the next
  // substep's fragments, then the remaining MFMAs, so the reads have almost
  // the whole substep to arrive.
  constexpr int NM = FM * FN;
  constexpr int NR = (A_KC ? FM : 2 * FM) + (B_KC ? FN : 2 * FN);
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, NM - 1, 0);
  };

  // In the loop, tiles are loaded by the first NW/2 waves only (one per SIMD:
  // waves go round-robin over the 4 SIMDs), each issuing its own share and
  // that of wave + NW/2, so a wave stalled on a full address queue leaves the
  // other wave of its SIMD free to issue MFMAs (+1% on the layer's shapes).
  auto load_u = [&](int t, int u) {  // the u-th load of tile t: own A, own B, partner A, partner B
    const uint32_t st = lds0 + (uint32_t)((t & 1) * SS);
    const int k0 = kbeg + t * kBK64;
    constexpr int PA = OA::PER_WAVE, PB = OB::PER_WAVE;
    constexpr int QA = NW / 2 * PA, QB = NW / 2 * PB;  // the partner's loads, as offsets of this wave's
    if constexpr (FULLK) {
      if (u < PA) oa.load_fullk(u, ra, p.lda, t, st, wave);
      else if (u < PA + PB) ob.load_fullk(u - PA, rb, p.ldb, t, st + SA, wave);
      else if (u < 2 * PA + PB) oa.template load_fullk<QA>(u - PA - PB, ra, p.lda, t, st, wave);
      else ob.template load_fullk<QB>(u - 2 * PA - PB, rb, p.ldb, t, st + SA, wave);
    } else {
      if (u < PA) oa.load_one(u, ra, p.lda, m0, p.M, k0, kend, st, wave);
      else if (u < PA + PB) ob.load_one(u - PA, rb, p.ldb, n0, p.N, k0, kend, st + SA, wave);
      else if (u < 2 * PA + PB) oa.template load_one<QA>(u - PA - PB, ra, p.lda, m0, p.M, k0, kend, st, wave);
      else ob.template load_one<QB>(u - 2 * PA - PB, rb, p.ldb, n0, p.N, k0, kend, st + SA, wave);
    }
  };
  constexpr int NL = OA::PER_WAVE + OB::PER_WAVE;  // loads per tile per wave when every wave loads
  constexpr int NL2 = 2 * NL;                      // per loading wave in the loop
  const bool loader = wave < NW / 2;

  // K-tiles 0 and 1 of the first work item; later items have theirs issued
  // before the previous item's epilogue.
  lane_setup();
  item_bases();
  if (nk > 0) issue(0, m0, n0, kbeg, kend);
  if (nk > 1) issue(1, m0, n0, kbeg, kend);
  bool first = true;
  float* const slab = reinterpret_cast<float*>(smem + 2 * SS) + wave * ESLAB;

  for (;;) {
    if (!first) lane_setup();
    float* const pt = tw.split >= 0 ? p.part + ((int64_t)tw.split * p.tail_tiles + tw.tl) * BM * BN : nullptr;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
      // tile 0 landed (for later items the previous epilogue waited for it)
      if (first) {
        if (nk > 1) MTNLG_VMCNT(NL);
        else __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      }
      __syncthreads();
      read_frags(smem, 0, 0);
    }
    first = false;
    for (int kt = 0; kt < nk; ++kt) {
      const char* st = smem + (kt & 1) * SS;
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        read_frags(st, s + 1, (s + 1) & 1);
        mfmas(s & 1);
        interleave();
      }
      // Substep 3: its fragments are in registers. Publish tile kt+1 (loaded
      // since substep 3 of the previous tile) and free this stage; then the
      // first reads of tile kt+1 and the loads of tile kt+2 into this stage are
      // woven into the last MFMAs of tile kt.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      Mfma<bf16_t>::run(af[1][0], bfr[1][0], acc[0][0]);
      __builtin_amdgcn_sched_barrier(0);
      // (after the last tile this reads a stale stage; the values are unused)
      read_frags(smem + ((kt + 1) & 1) * SS, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      const bool more = kt + 2 < nk;
#pragma unroll
      for (int idx = 1; idx < NM; ++idx) {
        Mfma<bf16_t>::run(af[1][idx / FN], bfr[1][idx % FN], acc[idx / FN][idx % FN]);
        __builtin_amdgcn_sched_barrier(0);
        if (more && loader) {
          // NL2 loads over MFMAs 1 .. NM-1
          const int lo = (idx - 1) * NL2 / (NM - 1), hi = idx * NL2 / (NM - 1);
#pragma unroll
          for (int u = lo; u < hi; ++u) load_u(kt + 2, u);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // Every wave is done with the ring (its last reads waited, then a
    // barrier): K-tiles 0 and 1 of the next work item go in flight now and
    // land while this item's epilogue runs from the per-wave slabs. (The bias
    // of bias kinds is waited for first: the loads below are invisible to the
    // compiler's count, which would otherwise wait for them too.)
    const int wnext = w + (int)gridDim.x;
    const bool has_next = wnext < total;
    const int m0c = m0, n0c = n0;
    constexpr bool kBias = EPI == EPI_BIAS || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_F16LO;
    const bool has_bias = kBias && pt == nullptr;
    uint4 bias_raw = make_uint4(0u, 0u, 0u, 0u);
    if (has_bias) {
      bias_raw = epi_bias_load(p, n0c, wn, lane);
      asm volatile("" : : "v"(bias_raw.x), "v"(bias_raw.y), "v"(bias_raw.z), "v"(bias_raw.w));
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __syncthreads();
    if (has_next) {
      lane_setup();
      tw = tile_work(p, wnext);
      m0 = tw.tm * BM;
      n0 = tw.tn * BN;
      kbeg = tw.kbeg;
      kend = tw.kend;
      nk = (kend - kbeg + kBK64 - 1) / kBK64;
      item_bases();
      if (nk > 0) issue(0, m0, n0, kbeg, kend);
      if (nk > 1) issue(1, m0, n0, kbeg, kend);
    }

    // Then tile 0 of the next item: the wait counts this epilogue's stores and
    // the next item's tile 1 (issued after tile 0), so it does not wait for
    // the stores to drain.
    epi_dispatch<EPI>(pt != nullptr, [&](auto kind) {
      constexpr int KIND = decltype(kind)::value;
      epilogue256<KIND, FM, FN, TN, BN>(p, acc, slab, m0c, n0c, wm, wn, lane, pt, bias_raw, [] {});
      constexpr int E = epi_vm_ops<KIND>();
      static_assert(NL + E <= 63, "vmcnt is 6 bits");
      if (has_next) {
        if (nk > 1) MTNLG_VMCNT(NL + E);
        else MTNLG_VMCNT(E);
      }
    });
    if (!has_next) break;
    w = wnext;
  }
}

// ---------------------------------------------------------------------------
// bf16 GEMM, 256x256 tiles, WM x WN waves, operand tiles staged through
// registers (instantiated as 2 x 4 waves of 128x64, two per SIMD)
//
// * Operand tiles are 64 deep with the LDS layouts and swizzles of the
//   direct-to-LDS kernel, but move through registers: during K tile t each
//   wave writes its share of tile t+1 (loaded during tile t-1) into the free
//   LDS stage and issues the global loads of tile t+2 into the registers it
//   just wrote out, a write and a load between every few MFMAs of the first
//   three k-substeps. No burst of loads stalls the MFMA issue (the
//   direct-to-LDS kernel can only refill a stage in a tile's last substep),
//   and each load has a whole K tile to land.
// * A 2 x 2 instance (one wave of 128x128 per SIMD, accumulators in AGPRs)
//   reads a third less LDS per MFMA but measured 3% slower over the layer's
//   products: one wave cannot hide its own LDS and barrier waits.
// * One barrier per K tile, before its last k-substep: every wave has then
//   written its share of tile t+1 and holds the last fragments of tile t, so
//   the barrier both publishes tile t+1 and frees tile t's stage; the last
//   substep's MFMAs cover the first fragment reads of tile t+1.
// * Persistent, with the XCD-aware walk and the tail split of the other
//   kernels. The next work item's first K tile is loaded and written to LDS
//   while the current item's epilogue runs from per-wave slabs beside the
//   ring.
// ---------------------------------------------------------------------------
template <int WM, int WN, bool A_KC, bool B_KC, bool FULLK, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_rs_kernel(GemmArgs p) {
  constexpr int BM = 256, BN = 256, NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  using OA = Dtl64<BM, A_KC, NW>;
  using OB = Dtl64<BN, B_KC, NW>;
  constexpr int SA = OA::STAGE_BYTES, SB = OB::STAGE_BYTES, SS = SA + SB;
  constexpr int PA = OA::PER_WAVE, PB = OB::PER_WAVE, NL = PA + PB;  // loads per wave per K tile
  constexpr int ESLAB = 16 * TN;                                    // floats of one wave's epilogue slab
  __shared__ __align__(1024) char smem[2 * SS + NW * ESLAB * 4];

  const int total = p.nfull + p.tail_tiles * p.tail_split;
  int w = blockIdx.x;
  if (w >= total) return;
  TileWork tw = tile_work(p, w);
  int m0 = tw.tm * BM, n0 = tw.tn * BN;
  int kbeg = tw.kbeg, kend = tw.kend;
  int nk = (kend - kbeg + kBK64 - 1) / kBK64;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.M * p.K * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, (uint32_t)((int64_t)p.K * p.N * 2));
  OA oa;
  OB ob;
  constexpr int AN = A_KC ? 4 : FM, BN_ = B_KC ? 4 : FN;
  int abase[AN], bbase[BN_];
  auto lane_setup = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    oa.init(wave, ln);
    ob.init(wave, ln);
#pragma unroll
    for (int e = 0; e < AN; ++e)
      abase[e] = A_KC ? kc64_frag_off(wm * FM, e, ln) : mn_frag_off<OA::RB>(wm * FM + e, 0, ln);
#pragma unroll
    for (int e = 0; e < BN_; ++e)
      bbase[e] = SA + (B_KC ? kc64_frag_off(wn * FN, e, ln) : mn_frag_off<OB::RB>(wn * FN + e, 0, ln));
  };
  auto aoff = [&](int s, int i) { return A_KC ? abase[s] + i * 4096 : abase[i] + s * 16 * OA::RB; };
  auto boff = [&](int s, int j) { return B_KC ? bbase[s] + j * 4096 : bbase[j] + s * 16 * OB::RB; };

  f32x16_t acc[FM][FN];
  uint4 af[2][FM], bfr[2][FN];
  uint4 stg[NL];
  auto read_a = [&](const char* st, int s, int buf, int i) {
    const char* q = st + aoff(s, i);
    if (A_KC) {
      af[buf][i] = *reinterpret_cast<const uint4*>(q);
    } else {
      const uint2 lo = ds_read_tr(q), hi = ds_read_tr(q + 4 * OA::RB);
      af[buf][i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  auto read_b = [&](const char* st, int s, int buf, int j) {
    const char* q = st + boff(s, j);
    if (B_KC) {
      bfr[buf][j] = *reinterpret_cast<const uint4*>(q);
    } else {
      const uint2 lo = ds_read_tr(q), hi = ds_read_tr(q + 4 * OB::RB);
      bfr[buf][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  // in the order the MFMAs consume them: a0, b0 .. b3, a1 .. a3
  auto read_frags = [&](const char* st, int s, int buf) {
    read_a(st, s, buf, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) read_b(st, s, buf, j);
#pragma unroll
    for (int i = 1; i < FM; ++i) read_a(st, s, buf, i);
  };
  // global load u of K tile t of the current work item into staging register u.
  // FULLK (every K tile of every item is whole, K % 64 == 0): the lane's offset
  // of tile 0 is kept per item and tile t adds t times the tile's byte step as
  // the instruction's scalar offset, so a load costs no vector arithmetic; past
  // the item's last tile a resource of zero bytes makes every load return zero.
  // Otherwise every load computes its offset with the K bound (kOob past it).
  uint32_t voff[FULLK ? NL : 1];
  const uint32_t kstep_a = A_KC ? 2u * kBK64 : (uint32_t)(2 * kBK64 * p.lda);
  const uint32_t kstep_b = B_KC ? 2u * kBK64 : (uint32_t)(2 * kBK64 * p.ldb);
  const __amdgpu_buffer_rsrc_t ra0 = make_rsrc(p.A, 0u), rb0 = make_rsrc(p.B, 0u);
  auto item_offsets = [&]() {
    if constexpr (FULLK) {
#pragma unroll
      for (int u = 0; u < NL; ++u)
        voff[u] = u < PA ? oa.goff(u, p.lda, m0, p.M, kbeg, kend) : ob.goff(u - PA, p.ldb, n0, p.N, kbeg, kend);
    }
  };
  auto gload = [&](int u, int t) {
    if constexpr (FULLK) {
      const bool in = t < nk;
      if (u < PA)
        stg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(in ? ra : ra0, voff[u],
                                                                                 (uint32_t)t * kstep_a, 0));
      else
        stg[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(in ? rb : rb0, voff[u],
                                                                                 (uint32_t)t * kstep_b, 0));
    } else {
      const int k0 = kbeg + t * kBK64;
      if (u < PA) stg[u] = buf_load16(ra, oa.goff(u, p.lda, m0, p.M, k0, kend));
      else stg[u] = buf_load16(rb, ob.goff(u - PA, p.ldb, n0, p.N, k0, kend));
    }
  };
  // staging register u into LDS stage `stage`, where the direct-to-LDS kernel's
  // load u of this wave would have put it
  auto swrite = [&](int u, int stage) {
    char* dst = smem + stage * SS + (u < PA ? (wave * PA + u) * 1024 : SA + (wave * PB + u - PA) * 1024) + lane * 16;
    *reinterpret_cast<uint4*>(dst) = stg[u];
  };
  constexpr int NR = (A_KC ? FM : 2 * FM) + (B_KC ? FN : 2 * FN);  // DS read instructions per substep
  constexpr int NM = FM * FN;
  // units (a staging write and the load that refills it) in substeps 0, 1, 2
  constexpr int U0 = (NL + 2) / 3, U1 = (NL + 1) / 3;
  static_assert(U0 + U1 + NL / 3 == NL && 2 * U0 + 1 <= NM, "interleave");

  float* const slab = reinterpret_cast<float*>(smem + 2 * SS) + wave * ESLAB;

  // first work item: tile 0 into stage 0, tile 1 into the staging registers
  lane_setup();
  item_offsets();
#pragma unroll
  for (int u = 0; u < NL; ++u) gload(u, 0);
#pragma unroll
  for (int u = 0; u < NL; ++u) swrite(u, 0);
#pragma unroll
  for (int u = 0; u < NL; ++u) gload(u, 1);

  for (;;) {
    float* const pt = tw.split >= 0 ? p.part + ((int64_t)tw.split * p.tail_tiles + tw.tl) * BM * BN : nullptr;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's writes of tile 0 are done
    __syncthreads();
    read_frags(smem, 0, 0);

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const char* st = smem + cur * SS;
      auto substep = [&](auto S_) {
        constexpr int s = decltype(S_)::value;
        read_frags(st, s + 1, (s + 1) & 1);
        constexpr int ub = s == 0 ? 0 : (s == 1 ? U0 : U0 + U1);
        constexpr int un = s == 0 ? U0 : (s == 1 ? U1 : NL / 3);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) Mfma<bf16_t>::run(af[s & 1][i], bfr[s & 1][j], acc[i][j]);
#pragma unroll
        for (int u = ub; u < ub + un; ++u) {
          swrite(u, cur ^ 1);  // tile kt+1 (stage cur^1 was freed by the last barrier)
          gload(u, kt + 2);    // past the item's last tile these are zero-filled, no memory is read
        }
        // the MFMA first, then every read of the next substep's fragments, then
        // the staging writes and loads between the remaining MFMAs
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
        for (int u = 0; u < un; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM - 1 - 2 * un, 0);
      };
      substep(std::integral_constant<int, 0>{});
      substep(std::integral_constant<int, 1>{});
      substep(std::integral_constant<int, 2>{});
      // substep 3: publish tile kt+1, free this stage; the first fragment reads
      // of tile kt+1 go under this substep's MFMAs
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      read_frags(smem + (cur ^ 1) * SS, 0, 0);  // (after the last tile: unused)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<bf16_t>::run(af[1][i], bfr[1][j], acc[i][j]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NM - 1, 0);
    }

    // every wave is done with the ring: load the bias of this tile's columns
    // (bias kinds), then the next item's K tile 0, which is written to stage 0
    // halfway through the epilogue, when its tile 1 is loaded
    const int wnext = w + (int)gridDim.x;
    const bool has_next = wnext < total;
    const int m0c = m0, n0c = n0;
    constexpr bool kBias = EPI == EPI_BIAS || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_F16LO;
    const bool has_bias = kBias && pt == nullptr;
    const uint4 bias_raw = has_bias ? epi_bias_load(p, n0c, wn, lane) : make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __syncthreads();
    if (!has_next) {
      epi_dispatch<EPI>(pt != nullptr, [&](auto kind) {
        epilogue256<decltype(kind)::value, FM, FN, TN, BN>(p, acc, slab, m0c, n0c, wm, wn, lane, pt, bias_raw,
                                                           [] {});
      });
      break;
    }
    // The next item's loads and the LDS writes that consume them share one
    // branch, so that no path leaves those loads pending into the K loop
    // (where the compiler would then wait for them at every iteration).
    lane_setup();
    tw = tile_work(p, wnext);
    m0 = tw.tm * BM;
    n0 = tw.tn * BN;
    kbeg = tw.kbeg;
    kend = tw.kend;
    nk = (kend - kbeg + kBK64 - 1) / kBK64;
    item_offsets();
#pragma unroll
    for (int u = 0; u < NL; ++u) gload(u, 0);
    epi_dispatch<EPI>(pt != nullptr, [&](auto kind) {
      epilogue256<decltype(kind)::value, FM, FN, TN, BN>(p, acc, slab, m0c, n0c, wm, wn, lane, pt, bias_raw, [&]() {
#pragma unroll
        for (int u = 0; u < NL; ++u) swrite(u, 0);
#pragma unroll
        for (int u = 0; u < NL; ++u) gload(u, 1);
      });
    });
    w = wnext;
  }
}

// Sums the tail pieces of each tail tile (fixed order over the splits) and
// applies the epilogue: one thread per 8-wide row vector of a tail tile.
template <typename T, int BM, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(GemmArgs p) {
  constexpr int VPT = BM * BN / 8;  // vectors per tile
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)p.tail_tiles * VPT) return;
  const int tl = (int)(gid / VPT), v = (int)(gid % VPT);
  const int rl = v / (BN / 8), cl = (v % (BN / 8)) * 8;
  int tm, tn;
  tile_pos(p, p.nfull + tl, tm, tn);
  const int row = tm * BM + rl, col = tn * BN + cl;
  if (row >= p.M || col >= p.N) return;
  float s[8];
  const float* base = p.part + (int64_t)tl * BM * BN + (int64_t)rl * BN + cl;
  load8(base, s);
  for (int z = 1; z < p.tail_split; ++z) {
    float t[8];
    load8(base + (int64_t)z * p.tail_tiles * BM * BN, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += t[e];
  }
  apply_epi_store<T>(p, row, col, s);
}

template <typename T, int BM, int BN, int WM, int WN, bool AK, bool BKc>
hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
  dim3 grid(a.nfull + a.tail_tiles * a.tail_split);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, AK, BKc>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <bool AK, bool BKc, int EPI>
void launch_256(const GemmArgs& a, dim3 grid, bool fullk, hipStream_t st) {
  if constexpr (AK || BKc) {
    if (fullk)
      hipLaunchKernelGGL((gemm_bf16_rs_kernel<2, 4, AK, BKc, true, EPI>), grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((gemm_bf16_rs_kernel<2, 4, AK, BKc, false, EPI>), grid, dim3(512), 0, st, a);
  } else if (fullk) {
    hipLaunchKernelGGL((gemm_bf16_dtl64_kernel<256, 256, AK, BKc, 2, 4, EPI, true>), grid, dim3(512), 0, st, a);
  } else {
    hipLaunchKernelGGL((gemm_bf16_dtl64_kernel<256, 256, AK, BKc, 2, 4, EPI, false>), grid, dim3(512), 0, st, a);
  }
}

template <int BM, int BN, bool AK, bool BKc>
hipError_t launch_dtl(const GemmArgs& a, hipStream_t st) {
  const int total = a.nfull + a.tail_tiles * a.tail_split;
  dim3 grid(total);
  if constexpr (BM >= 256) {  // 64-deep K tiles; persistent, one workgroup per CU
    grid.x = std::min(total, persistent_grid());
    // 8 waves (2 x 4, 128 x 64 each). Register-staged loads when at least one
    // operand is K-contiguous (measured 2-9% faster there); direct-to-LDS loads
    // when both are M/N-contiguous (the weight-gradient products, where the
    // staging writes share the LDS with twice as many transposing reads and
    // measured 2-4.5% slower).
    // Whole K tiles everywhere (K and the pieces' K range multiples of 64) let
    // the loads use scalar offsets (+1-4% measured).
    const bool fullk = a.K % kBK64 == 0 && a.k_chunk % kBK64 == 0;
    switch (a.epi) {
      case EPI_BIAS: launch_256<AK, BKc, EPI_BIAS>(a, grid, fullk, st); break;
      case EPI_BIAS_GELU: launch_256<AK, BKc, EPI_BIAS_GELU>(a, grid, fullk, st); break;
      case EPI_GELU_GRAD: launch_256<AK, BKc, EPI_GELU_GRAD>(a, grid, fullk, st); break;
      case EPI_BIAS_F16LO: launch_256<AK, BKc, EPI_BIAS_F16LO>(a, grid, fullk, st); break;
      default: launch_256<AK, BKc, EPI_STORE>(a, grid, fullk, st); break;
    }
  } else {           // 32-deep K tiles, 4 waves (2 x 2)
    hipLaunchKernelGGL((gemm_bf16_dtl_kernel<BM, BN, AK, BKc, 2, 2>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_dtl_layout(const GemmArgs& a, bool a_kc, bool b_kc, hipStream_t st) {
  if (a_kc && !b_kc) return launch_dtl<BM, BN, true, false>(a, st);
  if (a_kc && b_kc) return launch_dtl<BM, BN, true, true>(a, st);
  if (!a_kc && !b_kc) return launch_dtl<BM, BN, false, false>(a, st);
  return launch_dtl<BM, BN, false, true>(a, st);
}

template <typename T, int BM, int BN, int WM, int WN>
hipError_t launch_layout(const GemmArgs& a, bool a_kc, bool b_kc, hipStream_t st) {
  if (a_kc && !b_kc) return launch_tile<T, BM, BN, WM, WN, true, false>(a, st);
  if (a_kc && b_kc) return launch_tile<T, BM, BN, WM, WN, true, true>(a, st);
  if (!a_kc && !b_kc) return launch_tile<T, BM, BN, WM, WN, false, false>(a, st);
  return launch_tile<T, BM, BN, WM, WN, false, true>(a, st);
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int persistent_grid() { return std::max(kXcds, device_cus() / kXcds * kXcds); }

GemmPlan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, bool allow_split) {
  GemmPlan pl;
  const int num_cu = persistent_grid();
  if (dtype == kBF16) {
    const int64_t big = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    const int kt_big = ceil_div(K, kBK64);
    // 256x256 tiles whenever they fill the chip, or can be made to by
    // splitting every tile along K (at least 8 K-tiles per piece); 128x128
    // tiles only for problems too small for either.
    const bool split_fill = allow_split && big * 2 <= num_cu && kt_big / 2 >= 8;
    if (M >= 256 && N >= 256 && (big >= num_cu || big * 4 >= 3 * num_cu || split_fill)) {
      pl.bm = pl.bn = 256;
      pl.bk = kBK64;
    } else {
      pl.bm = pl.bn = 128;
      pl.bk = kBKd;
    }
  } else {
    pl.bm = pl.bn = (M >= 1024 && N >= 1024) ? 128 : 64;
    pl.bk = 32;
  }
  pl.tiles = ceil_div(M, pl.bm) * ceil_div(N, pl.bn);
  // Wave quantisation: one workgroup per CU (the LDS ring fills a CU), so the
  // last round of tiles may leave most CUs idle. When at most half a round is
  // left over, those tiles are split along K across the idle CUs; a problem
  // of at most half a round is split whole.
  const int tail = pl.tiles % num_cu;
  if (allow_split && dtype == kBF16 && tail > 0 && tail <= num_cu / 2) {
    const int ktiles = ceil_div(K, pl.bk);
    int s = num_cu / tail;
    while (s > 1 && ktiles / s < 8) --s;  // keep >= 8 K-tiles per piece
    if (s > 1) {
      pl.tail_tiles = tail;
      pl.tail_split = s;
    }
  }
  return pl;
}

size_t gemm_workspace_bytes(const GemmPlan& pl, int64_t, int64_t) {
  return pl.tail_split > 1 ? (size_t)pl.tail_tiles * pl.tail_split * pl.bm * pl.bn * sizeof(float) : 0;
}

hipError_t gemm(int dtype, bool a_kc, bool b_kc, int64_t M, int64_t N, int64_t K, const void* A,
                int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int epi,
                const void* bias, void* C2, const void* aux, const GemmPlan& pl, void* ws,
                hipStream_t st, int f16_cols) {
  GemmArgs a{};
  a.f16_cols = f16_cols;
  a.A = A; a.B = B; a.C = C;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc;
  a.bias = bias; a.C2 = C2; a.aux = aux;
  a.epi = epi;
  a.tiles_m = ceil_div(M, pl.bm);
  a.tiles_n = ceil_div(N, pl.bn);
  const bool tail = pl.tail_split > 1 && ws != nullptr;
  a.tail_tiles = tail ? pl.tail_tiles : 0;
  a.tail_split = tail ? pl.tail_split : 1;
  a.nfull = pl.tiles - a.tail_tiles;
  const int ktiles = ceil_div(K, pl.bk);
  a.k_chunk = ceil_div(ktiles, a.tail_split) * pl.bk;
  if (tail) a.tail_split = ceil_div(K, a.k_chunk);   // non-empty pieces only
  a.part = static_cast<float*>(ws);
  hipError_t e;
  if (dtype == kBF16) {
    if (pl.bm == 256) e = launch_dtl_layout<256, 256>(a, a_kc, b_kc, st);
    else e = launch_dtl_layout<128, 128>(a, a_kc, b_kc, st);
  } else {
    if (pl.bm == 128) e = launch_layout<float, 128, 128, 2, 2>(a, a_kc, b_kc, st);
    else e = launch_layout<float, 64, 64, 2, 2>(a, a_kc, b_kc, st);
  }
  if (e != hipSuccess || !tail) return e;
  const int64_t vec = (int64_t)a.tail_tiles * pl.bm * pl.bn / 8;
  const int blocks = (int)((vec + 255) / 256);
  if (pl.bm == 256)
    hipLaunchKernelGGL((tail_reduce_kernel<bf16_t, 256, 256>), dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((tail_reduce_kernel<bf16_t, 128, 128>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mtnlg
