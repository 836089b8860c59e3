// Tiled MFMA GEMM for gfx950: C[M,N] = op(A)[M,K] * op(B)[K,N] with an
// epilogue, fp32 accumulation.
//
// Every linear of the sliced layer maps onto this one kernel: the forward
// projections (X W: A K-contiguous, B N-contiguous), the input-gradient
// products (dY W^T: both K-contiguous) and the weight-gradient products
// (X^T dY: both M/N-contiguous), see the layer driver.
//
// Design (CDNA4, wave64):
//   * 256 threads = 4 waves in a 2x2 grid; each wave owns a (BM/2)x(BN/2)
//     sub-tile made of 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16 for bf16,
//     v_mfma_f32_32x32x2f32 for fp32).
//   * LDS holds both operand tiles as rows of K: 8 chunks of 16 bytes per
//     row (BK = 64 bf16 or 32 fp32), the chunk index XOR-ed with (row & 7)
//     so that the 32 rows one MFMA operand read touches spread over banks.
//   * K-contiguous operands are copied chunk by chunk; M/N-contiguous ones
//     are loaded as VECxVEC micro-blocks and transposed in registers, so the
//     MFMA loop is the same for all four layouts and HBM is read once.
//   * Two LDS stages: the global loads of tile k+1 are issued before the
//     MFMAs of tile k and written to the other stage afterwards.
//   * Workgroup ids are remapped so that each XCD (ids round-robin over 8
//     XCDs) gets a contiguous range of tiles, walked in groups of 8 tile rows
//     so that concurrently running tiles share operand panels in that XCD's L2.
//   * Optional split-K (grid.y) writes fp32 partials that a second kernel sums.
#include "common.hpp"
#include "kernels.hpp"

namespace mtnlg {

namespace {

constexpr int kCH = 8;        // 16-byte chunks per LDS row
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

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

  __device__ __forceinline__ void load(const T* __restrict__ p, int64_t ld, int r0, int rmax,
                                       int k0, int kend, int tid) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int id = tid + u * kThreads;
      if (KC) {
        const int row = id / kCH, ch = id % kCH;
        const int r = r0 + row, k = k0 + ch * VEC;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (id < UNITS && r < rmax && k < kend)
          v = *reinterpret_cast<const uint4*>(p + (int64_t)r * ld + k);
        st[u] = v;
      } else {
        const int kb = id / (R / VEC), rb = id % (R / VEC);
        const int r = r0 + rb * VEC;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int k = k0 + kb * VEC + j;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (id < UNITS && r < rmax && k < kend)
            v = *reinterpret_cast<const uint4*>(p + (int64_t)k * ld + r);
          st[u * VEC + j] = v;
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
        s[row * kCH + (ch ^ (row & 7))] = st[u];
      } else {
        const int kb = id / (R / VEC), rb = id % (R / VEC);
        uint4 t[VEC];
        transpose_block(&st[u * VEC], t, T());
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const int row = rb * VEC + i;
          s[row * kCH + (kb ^ (row & 7))] = t[i];
        }
      }
    }
  }
};

// Epilogue over a staged 32 x WN fp32 slab (row stride SROW floats): each lane
// takes 8-wide row vectors, applies the epilogue and stores 16 bytes (bf16) or
// 32 bytes (fp32). Not unrolled: it touches no register arrays.
template <typename T, int WN, int SROW>
__device__ __forceinline__ void epilogue_slab(const GemmArgs& p, const float* stage, int row0, int col0, int lane,
                                              int split) {
  using E = Elem<T>;
  constexpr int VPR = WN / 8;  // vectors per slab row
#pragma unroll 1
  for (int u = lane; u < 32 * VPR; u += kWave) {
    const int rr = u / VPR, cc = (u % VPR) * 8;
    const int row = row0 + rr, col = col0 + cc;
    if (row >= p.M || col >= p.N) continue;
    float v[8];
    const float4 a = *reinterpret_cast<const float4*>(stage + rr * SROW + cc);
    const float4 b = *reinterpret_cast<const float4*>(stage + rr * SROW + cc + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    const int64_t off = (int64_t)row * p.ldc + col;
    switch (p.epi) {
      case EPI_F32_PARTIAL:
        store8(static_cast<float*>(p.C) + (int64_t)split * p.M * p.N + (int64_t)row * p.N + col, v);
        break;
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
      default:
        store8(static_cast<T*>(p.C) + off, v);
    }
  }
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

template <typename T, int BM, int BN, bool A_KC, bool B_KC>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
  using E = Elem<T>;
  constexpr int VEC = E::VEC;
  constexpr int BK = kCH * VEC;
  constexpr int FM = BM / 64, FN = BN / 64;
  __shared__ uint4 smem[2 * (BM + BN) * kCH];
  uint4* const sA0 = smem;                        // two A stages, then two B stages
  uint4* const sB0 = smem + 2 * BM * kCH;

  // ---- tile id: XCD-contiguous ranges, grouped by 8 tile rows ----
  const int tiles = p.tiles_m * p.tiles_n;
  const int w = blockIdx.x;
  const int xcd = w & 7, idx = w >> 3;
  const int base = tiles >> 3, rem = tiles & 7;
  const int L = xcd * base + min(xcd, rem) + idx;
  const int group = kGroupM * p.tiles_n;
  const int g = L / group;
  const int first_m = g * kGroupM;
  const int gm = min(p.tiles_m - first_m, kGroupM);
  const int tm = first_m + (L % group) % gm;
  const int tn = (L % group) / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int split = blockIdx.y;
  const int kbeg = split * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);
  const int nk = (kend - kbeg + BK - 1) / BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, lg = lane >> 5;

  const T* __restrict__ Ap = static_cast<const T*>(p.A);
  const T* __restrict__ Bp = static_cast<const T*>(p.B);

  TileLoader<T, BM, A_KC> la;
  TileLoader<T, BN, B_KC> lb;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nk > 0) {
    la.load(Ap, p.lda, m0, p.M, kbeg, kend, tid);
    lb.load(Bp, p.ldb, n0, p.N, kbeg, kend, tid);
    la.store(sA0, tid);
    lb.store(sB0, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = kbeg + (kt + 1) * BK;
      la.load(Ap, p.lda, m0, p.M, k0, kend, tid);
      lb.load(Bp, p.ldb, n0, p.N, k0, kend, tid);
    }
    const uint4* a_s = sA0 + cur * BM * kCH;
    const uint4* b_s = sB0 + cur * BN * kCH;
#pragma unroll
    for (int s = 0; s < kCH / 2; ++s) {
      const int ch = 2 * s + lg;
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * (BM / 2) + i * 32 + lrow;
        af[i] = a_s[row * kCH + (ch ^ (row & 7))];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * (BN / 2) + j * 32 + lrow;
        bfr[j] = b_s[row * kCH + (ch ^ (row & 7))];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<T>::run(af[i], bfr[j], acc[i][j]);
    }
    if (more) {
      la.store(sA0 + (cur ^ 1) * BM * kCH, tid);
      lb.store(sB0 + (cur ^ 1) * BN * kCH, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: stage one 32-row slab of each wave's sub-tile in LDS (now
  // free), then write 8-wide row vectors; the MFMA output layout (lane: column
  // lrow, rows 8*blk + 4*lg + r) is turned into row-contiguous stores here.
  constexpr int WN = BN / 2;
  constexpr int SROW = WN + 4;  // padded so the two lane groups' rows hit different banks
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
    epilogue_slab<T, WN, SROW>(p, stage, m0 + wm * (BM / 2) + i * 32, n0 + wn * WN, lane, split);
    __syncthreads();
  }
}

// Sum of split-K partials [splits][M][N] f32 -> C (dtype), with optional bias.
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            int64_t MN, int N, const T* __restrict__ bias,
                                                            T* __restrict__ C) {
  const int64_t i8 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i8 >= MN) return;
  float s[8];
  load8(part + i8, s);
  for (int z = 1; z < splits; ++z) {
    float t[8];
    load8(part + (int64_t)z * MN + i8, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += t[e];
  }
  if (bias) {
    const int col = (int)(i8 % N);
    float b[8];
    load8(bias + col, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += b[e];
  }
  store8(C + i8, s);
}

template <typename T, int BM, int BN, bool AK, bool BKc>
hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
  dim3 grid(a.tiles_m * a.tiles_n, a.splits);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, AK, BKc>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename T, int BM, int BN>
hipError_t launch_layout(const GemmArgs& a, bool a_kc, bool b_kc, hipStream_t st) {
  if (a_kc && !b_kc) return launch_tile<T, BM, BN, true, false>(a, st);
  if (a_kc && b_kc) return launch_tile<T, BM, BN, true, true>(a, st);
  if (!a_kc && !b_kc) return launch_tile<T, BM, BN, false, false>(a, st);
  return launch_tile<T, BM, BN, false, true>(a, st);
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

GemmPlan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, bool allow_split) {
  GemmPlan pl;
  const int num_cu = 256;
  if (dtype == kBF16) {
    const int64_t big = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    if (big >= num_cu || (M >= 256 && N >= 256 && big * 4 >= 3 * num_cu)) {
      pl.bm = pl.bn = 256;
    } else {
      pl.bm = pl.bn = 128;
    }
    pl.bk = 64;
  } else {
    pl.bm = pl.bn = (M >= 1024 && N >= 1024) ? 128 : 64;
    pl.bk = 32;
  }
  const int64_t tiles = (int64_t)ceil_div(M, pl.bm) * ceil_div(N, pl.bn);
  pl.splits = 1;
  if (allow_split && tiles < num_cu) {
    // split K so that roughly one full wave of workgroups runs, keeping >= 8 K tiles each
    int s = (int)(num_cu / tiles);
    const int ktiles = ceil_div(K, pl.bk);
    while (s > 1 && ktiles / s < 8) --s;
    pl.splits = s < 1 ? 1 : s;
  }
  return pl;
}

size_t gemm_workspace_bytes(const GemmPlan& pl, int64_t M, int64_t N) {
  return pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
}

hipError_t gemm(int dtype, bool a_kc, bool b_kc, int64_t M, int64_t N, int64_t K, const void* A,
                int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int epi,
                const void* bias, void* C2, const void* aux, const GemmPlan& pl, void* ws,
                hipStream_t st) {
  GemmArgs a{};
  a.A = A; a.B = B; a.C = C;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc;
  a.bias = bias; a.C2 = C2; a.aux = aux;
  a.epi = epi;
  a.tiles_m = ceil_div(M, pl.bm);
  a.tiles_n = ceil_div(N, pl.bn);
  a.splits = pl.splits;
  const int ktiles = ceil_div(K, pl.bk);
  a.k_chunk = ceil_div(ktiles, pl.splits) * pl.bk;
  const bool split = pl.splits > 1;
  if (split) {
    // real number of non-empty splits
    a.splits = ceil_div(K, a.k_chunk);
    a.epi = EPI_F32_PARTIAL;
    a.C = ws;
  }
  hipError_t e;
  if (dtype == kBF16) {
    if (pl.bm == 256) e = launch_layout<bf16_t, 256, 256>(a, a_kc, b_kc, st);
    else e = launch_layout<bf16_t, 128, 128>(a, a_kc, b_kc, st);
  } else {
    if (pl.bm == 128) e = launch_layout<float, 128, 128>(a, a_kc, b_kc, st);
    else e = launch_layout<float, 64, 64>(a, a_kc, b_kc, st);
  }
  if (e != hipSuccess || !split) return e;
  const int64_t MN = M * N;
  const int blocks = ceil_div(MN / 8, 256);
  const bool with_bias = epi == EPI_BIAS;
  if (dtype == kBF16)
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(ws), a.splits, MN, (int)N,
                       with_bias ? static_cast<const bf16_t*>(bias) : nullptr, static_cast<bf16_t*>(C));
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(ws), a.splits, MN, (int)N,
                       with_bias ? static_cast<const float*>(bias) : nullptr, static_cast<float*>(C));
  return hipGetLastError();
}

}  // namespace mtnlg
