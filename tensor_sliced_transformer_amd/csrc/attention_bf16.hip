// Causal attention in bf16 on gfx950 matrix cores: forward, dQ and dK/dV.
//
// What is computed is the decoder self-attention of the Megatron-LM and
// MT-NLG pages (scores Q K^T / sqrt(head_dim), keys after the query masked,
// softmax over keys, weighted sum of values) for one slice's heads; the
// backward is the exact gradient of that map.
//
// Work split. A workgroup (4 waves) owns 64 rows of one (sequence, head): 64
// queries in the forward and dQ kernels, 64 keys in the dK/dV kernel, and
// walks the 64-row tiles of the other side that the causal mask leaves. The
// four waves are 2 x 2: two groups of 32 own rows, each split over the two
// 32-row halves of every tile. The two halves' partials (running max, sum and
// output for the forward; dQ, or dK and dV) are merged through LDS at the end,
// always in the same order, so the result is deterministic without atomics.
// Workgroups are numbered heaviest first (the forward and dQ blocks near the
// end of a sequence see the most keys, the dK/dV blocks near its start see the
// most queries); with one workgroup per CU the dispatcher then hands the
// lighter blocks to the CUs that finish first.
//
// Data movement. The streamed tiles go straight from memory into a 3-stage
// LDS ring with direct-to-LDS buffer loads, so the load of tile t+2 overlaps
// the math on tile t. A tile is 64 rows x head_dim bf16, stored as head_dim/32
// blocks of [64 rows][32 columns]; the four 16-byte chunks of a row sit at slot
// chunk ^ ((row >> 2) & 3), which keeps both read patterns below free of bank
// conflicts:
//   * row fragments (the A operand of S = X Y^T: lane = row, 8 head_dim
//     columns) are 16-byte reads;
//   * transposed fragments (the A operand of O^T = V^T P^T, dQ^T = K^T dS^T,
//     dV^T = dO^T P, dK^T = Q^T dS) come from ds_read_b64_tr_b16, which hands
//     each lane 4 consecutive rows of one column.
// The resident side (this block's 32 rows per wave) sits in registers as the B
// operand, and the score-like matrices (P, dS) never leave registers: an MFMA
// may take its 16 reduction slots in any order as long as both operands agree,
// so the accumulator layout of one product is used directly as the B operand
// of the next, with the transposed reads fetching the matching rows.
#include "attention_bf16.hpp"

namespace mtnlg {

namespace {

using namespace attn;

// ------------------------------------------------------------------ forward
// Wave (qg, kh): queries q0 + 32*qg + lane%32, keys 32*kh .. +31 of every tile.
// S^T = K Q^T puts one query per lane column, so the running max and sum are
// per lane (plus one exchange with lane^32).
//
// The running max m is a reference value, not necessarily the exact max: it
// is raised (and O, l rescaled) only when some query's max exceeds it by more
// than kSlack (in log2 units), so most tiles skip the rescale. Any reference
// gives the same softmax as long as the exponentials stay finite; here they
// stay below 2^kSlack.
constexpr float kSlack = 8.0f;

// Two ring stages and at most 256 registers per lane, so that two workgroups
// share a CU (two waves per SIMD): measured 8% faster than one workgroup with
// a three-stage ring at head_dim 160.
constexpr int kFwdRing = 2;

// The dQ kernel's ring: its pipelined walk reads tiles it+1 and it+2 during
// iteration it, and loads keep two iterations of lead.
constexpr int kDqRing = 4;

template <int D, bool DROP>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const bf16_t* __restrict__ qkv,
                                                               bf16_t* __restrict__ o, float* __restrict__ lse,
                                                               int seq, int nh, int64_t tokens, int nbh,
                                                               float scale_log2, AttnDropout drop) {
  using TL = Tile<D>;
  constexpr int EB = TL::EB, SUB = TL::SUB, STAGE = 2 * TL::BYTES;
  __shared__ __align__(1024) char smem[kFwdRing * STAGE];

  const int nqb = seq / kRows;
  const int qb = nqb - 1 - (int)blockIdx.x / nbh;
  const int bh = (int)blockIdx.x % nbh;
  const int n = bh % nh, b = bh / nh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, g = lane >> 5;
  const int qg = wave & 1, kh = wave >> 1;
  const int64_t ld = 3LL * nh * D;
  const bf16_t* base = qkv + (int64_t)b * seq * ld;
  const i32x4_t rs = rsrc_words(base, (uint32_t)(seq * ld * 2));
  const int q0 = qb * kRows;
  const int qw0 = q0 + 32 * qg;
  const int qw = qw0 + lq;

  uint32_t voff[TL::IPW];
#pragma unroll
  for (int u = 0; u < TL::IPW; ++u) voff[u] = tile_voff<D>(wave, u, lane, ld);
  const uint32_t row_bytes = (uint32_t)(ld * 2);
  const uint32_t col_k = (uint32_t)((nh + n) * D * 2), col_v = (uint32_t)((2 * nh + n) * D * 2);
  auto issue = [&](int t, int stage) {
    char* st = smem + stage * STAGE;
    const uint32_t r0 = (uint32_t)(t * kRows) * row_bytes;
    issue_tile<D>(rs, voff, r0 + col_k, st, wave);
    issue_tile<D>(rs, voff, r0 + col_v, st + TL::BYTES, wave);
  };

  // the first key tile is in flight while the query rows are read
  issue(0, 0);
  bf16x8_t qf[SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s)
    qf[s] = *reinterpret_cast<const bf16x8_t*>(base + (int64_t)qw * ld + (int64_t)n * D + 16 * s + 8 * g);
#pragma unroll
  for (int s = 0; s < SUB; ++s) settle(qf[s]);

  f32x16_t oacc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) zero(oacc[e]);
  float m = -INFINITY, l = 0.0f;

  ring_walk<2 * TL::IPW, kFwdRing, 1>(qb + 1, issue, [&](int it, int stage) {
    const char* sk = smem + stage * STAGE;
    const char* sv = sk + TL::BYTES;
    const int kw0 = it * kRows + 32 * kh;
    // key and query blocks are 32-aligned: either every query of this wave
    // sees key kw0, or none sees any key of the half
    if (kw0 > qw0) return;
    f32x16_t s;
    zero(s);
#pragma unroll
    for (int st = 0; st < SUB; ++st) s = mma_f16(frag_row(sk, 32 * kh + lq, st, g), qf[st], s);
    if (kw0 == qw0) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * g + (i & 3) > lq) s[i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    mx = fmaxf(mx, s[15]);
    mx = xor32_max(mx) * scale_log2;  // finite: key kw0 is visible here
    if (__builtin_amdgcn_ballot_w64(mx > m + kSlack)) {
      const float mn = fmaxf(m, mx);
      const float corr = fast_exp2(m - mn);
      m = mn;
      l *= corr;
#pragma unroll
      for (int e = 0; e < EB; ++e)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[e][i] *= corr;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[i], scale_log2, -m));
      l += p;  // the normaliser is the softmax's own, before dropout
      s[i] = p;
    }
    if (DROP) {
      const uint32_t keep = attn_keep_bits<false>(drop, (uint64_t)((qw0 >> 2) + (lq >> 2)),
                                                  (uint64_t)((kw0 >> 2) + 2 * (lq & 3) + g), drop.head0 + n, b, lane);
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = ((keep >> i) & 1u) ? s[i] * drop.scale : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8_t pb = pack_slots(s, t);
#pragma unroll
      for (int e = 0; e < EB; ++e) oacc[e] = mma(frag_tr(sv, e, 32 * kh, t, lane), pb, oacc[e]);
    }
  });

  // merge the two key halves: (m, l, O) of wave kh=1 into wave kh=0
  l = xor32_sum(l);
  __syncthreads();  // every load has been waited for and every wave is done with the ring
  static_assert(2 * (EB * 16 + 2) * 64 * 4 <= kFwdRing * STAGE, "merge staging exceeds the ring");
  float* xs = reinterpret_cast<float*>(smem) + qg * (EB * 16 + 2) * 64;
  if (kh == 1) {
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) xs[(e * 16 + i) * 64 + lane] = oacc[e][i];
    xs[(EB * 16) * 64 + lane] = m;
    xs[(EB * 16 + 1) * 64 + lane] = l;
  }
  __syncthreads();
  if (kh == 0) {
    const float m2 = xs[(EB * 16) * 64 + lane], l2 = xs[(EB * 16 + 1) * 64 + lane];
    const float mt = fmaxf(m, m2);  // m is finite (keys 0 .. 31 of the first tile)
    const float a1 = fast_exp2(m - mt), a2 = fast_exp2(m2 - mt);
    const float lt = l * a1 + l2 * a2;
    const float inv = 1.0f / lt;
    const float c1 = a1 * inv, c2 = a2 * inv;
    bf16_t* orow = o + ((int64_t)b * seq + qw) * (int64_t)(nh * D) + (int64_t)n * D;
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = oacc[e][4 * blk + r] * c1 + xs[(e * 16 + 4 * blk + r) * 64 + lane] * c2;
        store4(orow + e * 32 + 8 * blk + 4 * g, v[0], v[1], v[2], v[3]);
      }
    if (g == 0) lse[(int64_t)n * tokens + (int64_t)b * seq + qw] = (mt + log2f(lt)) * kLn2;
  }
}

// ------------------------------------------------------------- backward: dQ
// Same walk as the forward. Also computes, per query, D = rowsum(dO * O) and
// L = lse * log2(e), and stores the pair for the dK/dV kernel.
template <int D, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_dq_bf16_kernel(const bf16_t* __restrict__ qkv,
                                                           const bf16_t* __restrict__ o,
                                                           const bf16_t* __restrict__ dout,
                                                           const float* __restrict__ lse, float2* __restrict__ ldw,
                                                           bf16_t* __restrict__ dqkv, int seq, int nh,
                                                           int64_t tokens, int nbh, float scale, float scale_log2,
                                                           AttnDropout drop) {
  using TL = Tile<D>;
  constexpr int EB = TL::EB, SUB = TL::SUB, STAGE = 2 * TL::BYTES;
  __shared__ __align__(1024) char smem[kDqRing * STAGE];

  const int nqb = seq / kRows;
  const int qb = nqb - 1 - (int)blockIdx.x / nbh;
  const int bh = (int)blockIdx.x % nbh;
  const int n = bh % nh, b = bh / nh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, g = lane >> 5;
  const int qg = wave & 1, kh = wave >> 1;
  const int64_t ld = 3LL * nh * D;
  const int64_t ldo = (int64_t)nh * D;
  const bf16_t* base = qkv + (int64_t)b * seq * ld;
  const i32x4_t rs = rsrc_words(base, (uint32_t)(seq * ld * 2));
  const int q0 = qb * kRows;
  const int qw0 = q0 + 32 * qg;
  const int qw = qw0 + lq;
  const int64_t tq = (int64_t)b * seq + qw;  // token of this lane's query

  uint32_t voff[TL::IPW];
#pragma unroll
  for (int u = 0; u < TL::IPW; ++u) voff[u] = tile_voff<D>(wave, u, lane, ld);
  const uint32_t row_bytes = (uint32_t)(ld * 2);
  const uint32_t col_k = (uint32_t)((nh + n) * D * 2), col_v = (uint32_t)((2 * nh + n) * D * 2);
  auto issue = [&](int t, int stage) {
    char* st = smem + stage * STAGE;
    const uint32_t r0 = (uint32_t)(t * kRows) * row_bytes;
    issue_tile<D>(rs, voff, r0 + col_k, st, wave);
    issue_tile<D>(rs, voff, r0 + col_v, st + TL::BYTES, wave);
  };

  // The first two key tiles are in flight while this lane's query, output
  // gradient and output rows are read (the register loads' waits cover the
  // older tile loads too); tiles 2 and 3 follow once the register operands
  // have landed, so that no compiler-tracked load is pending in the loop.
  const int T = qb + 1;  // key tiles of this query block
  for (int t = 0; t < 2; ++t)
    if (t < T) issue(t, t);
  // All register operands are requested before the first wait, so that their
  // latencies overlap one another and the two tiles' loads.
  bf16x8_t qf[SUB], df[SUB], of[SUB];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    qf[s] = *reinterpret_cast<const bf16x8_t*>(base + (int64_t)qw * ld + (int64_t)n * D + 16 * s + 8 * g);
    const int64_t oo = tq * ldo + (int64_t)n * D + 16 * s + 8 * g;
    df[s] = *reinterpret_cast<const bf16x8_t*>(dout + oo);
    of[s] = *reinterpret_cast<const bf16x8_t*>(o + oo);
  }
  const float lse_q = lse[(int64_t)n * tokens + tq];
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    settle(qf[s]);
    settle(df[s]);
    settle(of[s]);
  }
  asm volatile("" : : "v"(lse_q));
  float dsum = 0.0f;
#pragma unroll
  for (int s = 0; s < SUB; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) dsum += (float)of[s][j] * (float)df[s][j];
  dsum = xor32_sum(dsum);
  // log2 of the softmax normaliser, plus the dS down-shift (kDsShift): P and
  // dS below are 2^-kDsShift times their values
  const float lrow = fmaf(lse_q, kLog2e, kDsShift);
  f32x16_t dq[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) zero(dq[e]);

  // Software-pipelined walk over the key tiles: iteration it computes S and
  // dP of tile it+1 on the matrix cores while the vector units turn tile
  // it's S and dP into dS, then accumulates dQ += dS K of tile it. Tiles
  // it+1 and it+2 are resident during iteration it; the ring's kDqRing
  // stages give every tile two iterations from the issue of its loads to
  // its first use.
  constexpr int NLD = 2 * TL::IPW;  // loads per wave per tile
  auto active = [&](int it) { return it * kRows + 32 * kh <= qw0; };  // some key of the half is visible
  f32x16_t sb[2], dpb[2];
  auto chains = [&](int it, int buf) {  // S and dP of tile it, alone (the first tile)
    const char* sk = smem + (it % kDqRing) * STAGE;
    const char* sv = sk + TL::BYTES;
    zero(sb[buf]);
    zero(dpb[buf]);
#pragma unroll
    for (int st = 0; st < SUB; ++st) {
      sb[buf] = mma_f16(frag_row(sk, 32 * kh + lq, st, g), qf[st], sb[buf]);
      dpb[buf] = mma(frag_row(sv, 32 * kh + lq, st, g), df[st], dpb[buf]);
    }
  };
  // dS of slot i from S and dP (2^-kDsShift scale)
  auto ds_slot = [&](f32x16_t& s, f32x16_t& dp, uint32_t keep, int i) {
    const float p = fast_exp2(fmaf(s[i], scale_log2, -lrow));
    if (DROP)  // the gradient reaching P is dO V^T * keep * scale
      dp[i] = p * ((((keep >> i) & 1u) ? dp[i] * drop.scale : 0.0f) - dsum);
    else
      dp[i] = p * (dp[i] - dsum);
  };

  // Fragment registers of two consecutive iterations: tile it+1's K and V
  // rows (S and dP) and tile it's transposed K (dQ), for iteration it.
  bf16x8_t kfr[2][SUB], vfr[2][SUB], ktr[2][2][EB];
  auto read_frags = [&](int it, int fb) {  // fragments of iteration it into set fb
    const char* sk = smem + (it % kDqRing) * STAGE;         // tile it
    const char* skn = smem + ((it + 1) % kDqRing) * STAGE;  // tile it+1 (past the last: stale, unused)
    const char* svn = skn + TL::BYTES;
#pragma unroll
    for (int st = 0; st < SUB; ++st) {
      kfr[fb][st] = frag_row(skn, 32 * kh + lq, st, g);
      vfr[fb][st] = frag_row(svn, 32 * kh + lq, st, g);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < EB; ++e) ktr[fb][t][e] = frag_tr(sk, e, 32 * kh, t, lane);
  };

  // One iteration; BUF = it & 1 is a template constant so that register sets
  // are never indexed at run time. The S and dP chains of tile it+1 run with
  // tile it's dS computed between their matrix instructions (source order,
  // kept by scheduling barriers); then a barrier publishes tile it+2, the
  // next iteration's fragments are read, and dQ += dS K of tile it covers
  // their latency.
  auto step = [&](int it, auto BUF_) {
    constexpr int buf = decltype(BUF_)::value;
    const int kw0 = it * kRows + 32 * kh;
    uint32_t keep = 0;
    if (DROP)
      keep = attn_keep_bits<false>(drop, (uint64_t)((qw0 >> 2) + (lq >> 2)), (uint64_t)((kw0 >> 2) + 2 * (lq & 3) + g),
                                   drop.head0 + n, b, lane);
    __builtin_amdgcn_sched_barrier(0);
    f32x16_t& sn = sb[buf ^ 1];
    f32x16_t& dpn = dpb[buf ^ 1];
    zero(sn);
    zero(dpn);
#pragma unroll
    for (int st = 0; st < SUB; ++st) {
      sn = mma_f16(kfr[buf][st], qf[st], sn);
      dpn = mma(vfr[buf][st], df[st], dpn);
#pragma unroll
      for (int i = 16 * st / SUB; i < 16 * (st + 1) / SUB; ++i) ds_slot(sb[buf], dpb[buf], keep, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Tile it+2 landed (tile it+3 may still be in flight), and every wave's
    // reads of tile it are done (its transposed K was read at the previous
    // barrier): tile it's stage takes tile it+kDqRing.
    wait_tiles<NLD>(min(T - 3 - it, kDqRing - 3));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __syncthreads();
    if (it + kDqRing < T) issue(it + kDqRing, it % kDqRing);
    read_frags(it + 1, buf ^ 1);
    f32x16_t& dp = dpb[buf];
    if (kw0 == qw0) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * g + (i & 3) > lq) dp[i] = 0.0f;
    }
    if (active(it)) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8_t db = pack_slots_f16(dp, t);
#pragma unroll
        for (int e = 0; e < EB; ++e) dq[e] = mma_f16(ktr[buf][t][e], db, dq[e]);
      }
    }
  };

  for (int t = 2; t < kDqRing; ++t)
    if (t < T) issue(t, t);
  wait_tiles<NLD>(min(T - 2, kDqRing - 2));  // tiles 0 and 1
  __syncthreads();
  chains(0, 0);
  read_frags(0, 0);
  for (int it = 0; it < T; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < T) step(it + 1, std::integral_constant<int, 1>{});
  }
  MTNLG_VMCNT(0);

  __syncthreads();
  float* xs = reinterpret_cast<float*>(smem) + qg * (EB * 16) * 64;
  if (kh == 1) {
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) xs[(e * 16 + i) * 64 + lane] = dq[e][i];
  }
  __syncthreads();
  if (kh == 0) {
    // stored after the loop so that no store is in flight among the ring's loads
    if (g == 0) ldw[(int64_t)n * tokens + tq] = make_float2(lrow, dsum);
    bf16_t* row = dqkv + tq * ld + (int64_t)n * D;
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = (dq[e][4 * blk + r] + xs[(e * 16 + 4 * blk + r) * 64 + lane]) * (scale * kDsUp);
        store4(row + e * 32 + 8 * blk + 4 * g, v[0], v[1], v[2], v[3]);
      }
  }
}

template <int D>
hipError_t fwd_launch(int batch, int seq, int heads, const void* qkv, void* o, float* lse, const AttnDropout& drop,
                      hipStream_t st) {
  const int nbh = batch * heads;
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((drop.thr ? attn_fwd_bf16_kernel<D, true> : attn_fwd_bf16_kernel<D, false>),
                     dim3((unsigned)((seq / kRows) * nbh)), dim3(256), 0, st, static_cast<const bf16_t*>(qkv),
                     static_cast<bf16_t*>(o), lse, seq, heads, (int64_t)batch * seq, nbh, scale_log2, drop);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_launch(int batch, int seq, int heads, const void* qkv, const void* o, const float* lse,
                      const void* dout, void* dqkv, float2* ldw, const AttnDropout& drop, hipStream_t st) {
  const int nbh = batch * heads;
  const int64_t tokens = (int64_t)batch * seq;
  const float scale = 1.0f / sqrtf((float)D);
  const float scale_log2 = kLog2e * scale;
  const dim3 grid((unsigned)((seq / kRows) * nbh));
  hipLaunchKernelGGL((drop.thr ? attn_dq_bf16_kernel<D, true> : attn_dq_bf16_kernel<D, false>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(qkv),
                     static_cast<const bf16_t*>(o), static_cast<const bf16_t*>(dout), lse, ldw,
                     static_cast<bf16_t*>(dqkv), seq, heads, tokens, nbh, scale, scale_log2, drop);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dkdv_bf16(batch, seq, heads, D, qkv, dout, ldw, dqkv, drop, st);
}

}  // namespace

hipError_t attention_fwd_bf16(int batch, int seq, int heads, int head_dim, const void* qkv, void* o, float* lse,
                              const AttnDropout& drop, hipStream_t st) {
  if (seq % kRows) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return fwd_launch<64>(batch, seq, heads, qkv, o, lse, drop, st);
    case 128: return fwd_launch<128>(batch, seq, heads, qkv, o, lse, drop, st);
    case 160: return fwd_launch<160>(batch, seq, heads, qkv, o, lse, drop, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t attention_bwd_bf16(int batch, int seq, int heads, int head_dim, const void* qkv, const void* o,
                              const float* lse, const void* dout, void* dqkv, void* ws, const AttnDropout& drop,
                              hipStream_t st) {
  if (seq % kRows) return hipErrorInvalidValue;
  float2* ldw = static_cast<float2*>(ws);
  switch (head_dim) {
    case 64: return bwd_launch<64>(batch, seq, heads, qkv, o, lse, dout, dqkv, ldw, drop, st);
    case 128: return bwd_launch<128>(batch, seq, heads, qkv, o, lse, dout, dqkv, ldw, drop, st);
    case 160: return bwd_launch<160>(batch, seq, heads, qkv, o, lse, dout, dqkv, ldw, drop, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtnlg
