// dK and dV of the causal bf16 attention (gfx950). Built in its own
// translation unit because it keeps its MFMA accumulators in AGPRs (the
// forward and dQ kernels are built for VGPR accumulators); the method is
// described in attention_bf16.hip.
#include "attention_bf16.hpp"

namespace mtnlg {

namespace {

using namespace attn;

// --------------------------------------------------------- backward: dK, dV
// Wave (kg, qh): keys k0 + 32*kg + lane%32, queries 32*qh .. +31 of every
// query tile. S = Q K^T and dP = dO V^T put one key per lane column; P and dS
// feed dV^T += dO^T P and dK^T += Q^T dS without leaving registers. Each
// stage also holds the (L, D) pairs of the tile's 64 queries: wave w loads
// queries 16w .. 16w+15 into its own 1 KiB slot (lanes 8..63 load nothing
// but still write zeros, hence the slot).
template <int D, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_dkdv_bf16_kernel(const bf16_t* __restrict__ qkv,
                                                             const bf16_t* __restrict__ dout,
                                                             const float2* __restrict__ ldw,
                                                             bf16_t* __restrict__ dqkv, int seq, int nh,
                                                             int64_t tokens, int nbh, float scale,
                                                             float scale_log2, AttnDropout drop) {
  using TL = Tile<D>;
  constexpr int EB = TL::EB, SUB = TL::SUB;
  constexpr int LD_OFF = 2 * TL::BYTES, STAGE = 2 * TL::BYTES + 4096;
  __shared__ __align__(1024) char smem[kRing * STAGE];

  const int kb = (int)blockIdx.x / nbh;  // low key blocks see the most queries
  const int bh = (int)blockIdx.x % nbh;
  const int n = bh % nh, b = bh / nh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, g = lane >> 5;
  const int kg = wave & 1, qh = wave >> 1;
  const int64_t ld = 3LL * nh * D;
  const int64_t ldo = (int64_t)nh * D;
  const bf16_t* base = qkv + (int64_t)b * seq * ld;
  const bf16_t* dbase = dout + (int64_t)b * seq * ldo;
  const float2* lbase = ldw + (int64_t)n * tokens + (int64_t)b * seq;
  const i32x4_t rs_q = rsrc_words(base, (uint32_t)(seq * ld * 2));
  const i32x4_t rs_o = rsrc_words(dbase, (uint32_t)(seq * ldo * 2));
  const i32x4_t rs_l = rsrc_words(lbase, (uint32_t)(seq * 8));
  const int kw0 = kb * kRows + 32 * kg;
  const int kw = kw0 + lq;

  uint32_t voff_q[TL::IPW], voff_o[TL::IPW];
#pragma unroll
  for (int u = 0; u < TL::IPW; ++u) {
    voff_q[u] = tile_voff<D>(wave, u, lane, ld);
    voff_o[u] = tile_voff<D>(wave, u, lane, ldo);
  }
  const uint32_t voff_l = lane < 8 ? (uint32_t)((16 * wave + 2 * lane) * 8) : kOobOffset;
  const uint32_t col_q = (uint32_t)(n * D * 2);
  auto issue = [&](int t, int stage) {  // query tile kb + t
    char* st = smem + stage * STAGE;
    const int q0 = (kb + t) * kRows;
    issue_tile<D>(rs_q, voff_q, (uint32_t)q0 * (uint32_t)(ld * 2) + col_q, st, wave);
    issue_tile<D>(rs_o, voff_o, (uint32_t)q0 * (uint32_t)(ldo * 2) + col_q, st + TL::BYTES, wave);
    dtl16_so(rs_l, st + LD_OFF + wave * 1024, voff_l, (uint32_t)q0 * 8u);
  };

  // the first two query tiles are in flight while the key and value rows are read
  const int count = seq / kRows - kb;
  for (int t = 0; t < 2; ++t)
    if (t < count) issue(t, t);
  bf16x8_t kf[SUB], vf[SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    kf[s] = *reinterpret_cast<const bf16x8_t*>(base + (int64_t)kw * ld + (int64_t)(nh + n) * D + 16 * s + 8 * g);
    vf[s] = *reinterpret_cast<const bf16x8_t*>(base + (int64_t)kw * ld + (int64_t)(2 * nh + n) * D + 16 * s + 8 * g);
  }
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    settle(kf[s]);
    settle(vf[s]);
  }

  f32x16_t dk[EB], dv[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    zero(dk[e]);
    zero(dv[e]);
  }

  ring_walk<2 * TL::IPW + 1, kRing, 2>(count, issue, [&](int it, int stage) {
    const char* sq = smem + stage * STAGE;
    const char* so = sq + TL::BYTES;
    const char* sl = sq + LD_OFF;
    const int qw0 = (kb + it) * kRows + 32 * qh;
    if (kw0 > qw0) return;  // 32-aligned blocks: all of this half is masked
    // Every row fragment of the two chains is requested before the first
    // matrix instruction, the (L, D) pairs and the transposed fragments of
    // the first update half before the softmax arithmetic, and those of the
    // second half between the first half's matrix instructions, so that one
    // wave per SIMD does not wait out an LDS round trip per instruction;
    // scheduling barriers keep this source order.
    bf16x8_t fq[SUB], fo[SUB];
#pragma unroll
    for (int st = 0; st < SUB; ++st) fq[st] = frag_row(sq, 32 * qh + lq, st, g);
#pragma unroll
    for (int st = 0; st < SUB; ++st) fo[st] = frag_row(so, 32 * qh + lq, st, g);
    __builtin_amdgcn_sched_barrier(0);
    f32x16_t s, dp;
    zero(s);
    zero(dp);
#pragma unroll
    for (int st = 0; st < SUB; ++st) s = mma_f16(fq[st], kf[st], s);
#pragma unroll
    for (int st = 0; st < SUB; ++st) dp = mma(fo[st], vf[st], dp);
    // (L, D) of queries 32*qh + 8*(i2>>1) + 4*g + 2*(i2&1) + {0, 1}; these and
    // the first transposed fragments are read ahead except with dropout, whose
    // mask arithmetic needs the registers
    auto ld_pair = [&](int i2) {
      const int ql = 32 * qh + 8 * (i2 >> 1) + 4 * g + 2 * (i2 & 1);
      return *reinterpret_cast<const float4*>(sl + (ql >> 4) * 1024 + (ql & 15) * 8);
    };
    float4 pr[8];
    if constexpr (!DROP) {
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) pr[i2] = ld_pair(i2);
    }
    bf16x8_t tv[2][EB], tk[2][EB];
    if constexpr (!DROP) {
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        tv[0][e] = frag_tr(so, e, 32 * qh, 0, lane);
        tk[0][e] = frag_tr(sq, e, 32 * qh, 0, lane);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // dropout on the probabilities: dV takes P * keep * scale, and the
    // gradient reaching P is dO V^T * keep * scale (all ones without dropout)
    uint32_t keep = 0xFFFFu;
    if (DROP)
      keep = attn_keep_bits<true>(drop, (uint64_t)((qw0 >> 2) + 2 * (lq & 3) + g), (uint64_t)((kw0 >> 2) + (lq >> 2)),
                                  drop.head0 + n, b, lane);
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) {  // queries 32*qh + 8*(i>>2) + 4*g + (i&3), two at a time
      if constexpr (DROP) pr[i2] = ld_pair(i2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * i2 + j;
        const float p = fast_exp2(fmaf(s[i], scale_log2, -(j ? pr[i2].z : pr[i2].x)));
        if (DROP) {
          const bool kept = (keep >> i) & 1u;
          s[i] = kept ? p * drop.scale : 0.0f;
          dp[i] = p * ((kept ? dp[i] * drop.scale : 0.0f) - (j ? pr[i2].w : pr[i2].y));
        } else {
          s[i] = p;
          dp[i] = p * (dp[i] - (j ? pr[i2].w : pr[i2].y));
        }
      }
    }
    if (kw0 == qw0) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (lq > 8 * (i >> 2) + 4 * g + (i & 3)) {
          s[i] = 0.0f;
          dp[i] = 0.0f;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DROP) {
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        tv[0][e] = frag_tr(so, e, 32 * qh, 0, lane);
        tk[0][e] = frag_tr(sq, e, 32 * qh, 0, lane);
      }
    }
    {
      const bf16x8_t pb = pack_slots(s, 0);
      const bf16x8_t db = pack_slots_f16(dp, 0);
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        dv[e] = mma(tv[0][e], pb, dv[e]);
        dk[e] = mma_f16(tk[0][e], db, dk[e]);
        tv[1][e] = frag_tr(so, e, 32 * qh, 1, lane);
        tk[1][e] = frag_tr(sq, e, 32 * qh, 1, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {
      const bf16x8_t pb = pack_slots(s, 1);
      const bf16x8_t db = pack_slots_f16(dp, 1);
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        dv[e] = mma(tv[1][e], pb, dv[e]);
        dk[e] = mma_f16(tk[1][e], db, dk[e]);
      }
    }
  });

  __syncthreads();
  float* xs = reinterpret_cast<float*>(smem) + kg * (2 * EB * 16) * 64;
  if (qh == 1) {
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xs[(e * 16 + i) * 64 + lane] = dk[e][i];
        xs[((EB + e) * 16 + i) * 64 + lane] = dv[e][i];
      }
  }
  __syncthreads();
  if (qh == 0) {
    bf16_t* krow = dqkv + ((int64_t)b * seq + kw) * ld + (int64_t)(nh + n) * D;
    bf16_t* vrow = dqkv + ((int64_t)b * seq + kw) * ld + (int64_t)(2 * nh + n) * D;
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float a[4], c[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * blk + r;
          a[r] = (dk[e][i] + xs[(e * 16 + i) * 64 + lane]) * (scale * kDsUp);
          c[r] = (dv[e][i] + xs[((EB + e) * 16 + i) * 64 + lane]) * kDsUp;
        }
        store4(krow + e * 32 + 8 * blk + 4 * g, a[0], a[1], a[2], a[3]);
        store4(vrow + e * 32 + 8 * blk + 4 * g, c[0], c[1], c[2], c[3]);
      }
  }
}

template <int D>
hipError_t dkdv_launch(int batch, int seq, int heads, const void* qkv, const void* dout, const float2* ldw,
                       void* dqkv, const AttnDropout& drop, hipStream_t st) {
  const int nbh = batch * heads;
  const float scale = 1.0f / sqrtf((float)D);
  hipLaunchKernelGGL((drop.thr ? attn_dkdv_bf16_kernel<D, true> : attn_dkdv_bf16_kernel<D, false>),
                     dim3((unsigned)((seq / kRows) * nbh)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(qkv), static_cast<const bf16_t*>(dout), ldw,
                     static_cast<bf16_t*>(dqkv), seq, heads, (int64_t)batch * seq, nbh, scale, kLog2e * scale,
                     drop);
  return hipGetLastError();
}

}  // namespace

namespace attn {

hipError_t dkdv_bf16(int batch, int seq, int heads, int head_dim, const void* qkv, const void* dout,
                     const float2* ldw, void* dqkv, const AttnDropout& drop, hipStream_t st) {
  switch (head_dim) {
    case 64: return dkdv_launch<64>(batch, seq, heads, qkv, dout, ldw, dqkv, drop, st);
    case 128: return dkdv_launch<128>(batch, seq, heads, qkv, dout, ldw, dqkv, drop, st);
    case 160: return dkdv_launch<160>(batch, seq, heads, qkv, dout, ldw, dqkv, drop, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
}  // namespace mtnlg
