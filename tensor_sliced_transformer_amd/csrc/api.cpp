// C ABI of the library (include/mtnlg.h): host-side validation, buffer
// layouts, and the launch sequences of the two halves of a layer slice.
//
// The halves follow the tensor-slicing example of the STRONGHOLD slide deck
// (slides 7-8): the first linear of each half is column-sliced (QKV by whole
// heads, MLP-up A by columns) and needs no communication; the second is
// row-sliced (attention output W_o, MLP-down B) and produces a partial that
// operator g sums across slices. Backward mirrors it: g's backward is the
// identity (every slice receives the same dy), f's backward sums the slices'
// input-gradient partials.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "../../include/mtnlg.h"
#include "abi_common.hpp"
#include "kernels.hpp"

using namespace mtnlg;
using namespace mtnlg::abi;

namespace {


struct Dims {
  int64_t T;      // tokens = batch*seq
  int64_t h;      // hidden
  int64_t d;      // head_dim
  int64_t nhl;    // local heads
  int64_t w;      // local attention width = nhl*d
  int64_t fl;     // local MLP width
  int dtype;
  size_t eb;      // element bytes
};

int validate_desc(const mtnlg_layer_desc* desc, int32_t half, Dims* out) {
  if (!desc) return fail(MTNLG_ERR_ARG, "desc is NULL");
  if (half != MTNLG_ATTN && half != MTNLG_MLP) return fail(MTNLG_ERR_ARG, "half must be 0 (ATTN) or 1 (MLP)");
  const mtnlg_layer_desc& D = *desc;
  if (D.dtype != MTNLG_F32 && D.dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", D.dtype);
  if (D.batch <= 0 || D.seq <= 0 || D.hidden <= 0 || D.heads <= 0 || D.ffn <= 0 || D.tp_size <= 0)
    return fail(MTNLG_ERR_SHAPE, "dimensions must be positive");
  if (D.tp_rank < 0 || D.tp_rank >= D.tp_size)
    return fail(MTNLG_ERR_ARG, "tp_rank %d outside [0, %d)", D.tp_rank, D.tp_size);
  if (D.hidden % D.heads) return fail(MTNLG_ERR_SHAPE, "hidden %% heads != 0");
  if (D.heads % D.tp_size) return fail(MTNLG_ERR_SHAPE, "heads %% tp_size != 0");
  if (D.ffn % D.tp_size) return fail(MTNLG_ERR_SHAPE, "ffn %% tp_size != 0");
  const int hd = D.hidden / D.heads;
  const bool hd_ok = D.dtype == MTNLG_BF16 ? (hd == 64 || hd == 128 || hd == 160) : (hd == 64 || hd == 128);
  if (!hd_ok) return fail(MTNLG_ERR_SHAPE, "head_dim %d unsupported for this dtype", hd);
  if (D.hidden % 16 || (D.ffn / D.tp_size) % 16) return fail(MTNLG_ERR_SHAPE, "hidden and ffn/tp must be multiples of 16");
  if (D.hidden > 32768) return fail(MTNLG_ERR_SHAPE, "hidden > 32768 unsupported");
  if (D.seq % 128) return fail(MTNLG_ERR_SHAPE, "seq must be a multiple of 128");
  if ((int64_t)D.seq * 3 * D.hidden / D.tp_size * (int64_t)elem_bytes(D.dtype) >= ((int64_t)1 << 31))
    return fail(MTNLG_ERR_SHAPE, "one sequence of the QKV activations must stay below 2 GiB");
  if (!(D.ln_eps > 0.0f) || !isfinite(D.ln_eps)) return fail(MTNLG_ERR_ARG, "ln_eps must be positive and finite");
  if (!(D.attn_dropout >= 0.0f && D.attn_dropout < 1.0f))
    return fail(MTNLG_ERR_ARG, "attn_dropout must be in [0, 1)");
  if (nearbyint((double)D.attn_dropout * 65536.0) >= 65536.0)
    return fail(MTNLG_ERR_ARG, "attn_dropout rounds to 1");
  if (D.attn_dropout > 0.0f && D.dtype != MTNLG_BF16)
    return fail(MTNLG_ERR_UNIMPLEMENTED, "dropout on the attention probabilities needs the BF16 path");
  const int64_t T = (int64_t)D.batch * D.seq;
  {
    // every GEMM operand of the layer (activations T x width, weights) must
    // stay below 2 GiB, the range of the GEMM's 32-bit buffer offsets
    const int64_t eb = elem_bytes(D.dtype), lim = (int64_t)1 << 31;
    const int64_t w3 = 3LL * (D.hidden / D.heads) * (D.heads / D.tp_size), fl = D.ffn / D.tp_size;
    const int64_t widest = std::max<int64_t>(std::max<int64_t>(D.hidden, w3), fl);
    if (T >= lim || T * widest * eb >= lim || (int64_t)D.hidden * std::max(w3, fl) * eb >= lim)
      return fail(MTNLG_ERR_SHAPE, "every GEMM operand (tokens x width, hidden x width) must stay below 2 GiB");
  }
  if (out) {
    out->T = T;
    out->h = D.hidden;
    out->d = hd;
    out->nhl = D.heads / D.tp_size;
    out->w = out->nhl * hd;
    out->fl = D.ffn / D.tp_size;
    out->dtype = D.dtype;
    out->eb = elem_bytes(D.dtype);
  }
  return MTNLG_OK;
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }
const char* at(const void* base, size_t off) { return static_cast<const char*>(base) + off; }

// ---- saved layout ----
struct SavedLayout {
  size_t ln_out, mean, rstd, a, b, c, total;  // ATTN: a=qkv b=o c=lse; MLP: a=u b=y
};

SavedLayout saved_layout(const Dims& d, int half) {
  SavedLayout L{};
  size_t off = 0;
  L.ln_out = off; off = align256(off + d.T * d.h * d.eb);
  L.mean = off;   off = align256(off + d.T * sizeof(float));
  L.rstd = off;   off = align256(off + d.T * sizeof(float));
  if (half == MTNLG_ATTN) {
    L.a = off; off = align256(off + d.T * 3 * d.w * d.eb);
    L.b = off; off = align256(off + d.T * d.w * d.eb);
    L.c = off; off = align256(off + d.nhl * d.T * sizeof(float));
  } else {
    L.a = off; off = align256(off + d.T * d.fl * d.eb);
    L.b = off; off = align256(off + d.T * d.fl * d.eb);
    L.c = off;
  }
  L.total = off;
  return L;
}

// Where the saved tensors of one half are: the fields of a `saved` region
// (the layer entry points), or fields placed elsewhere (a stage keeping
// every micro-batch's copy of a field back to back).
SavedPtrs saved_ptrs(const void* saved, const Dims& d, int half) {
  const SavedLayout L = saved_layout(d, half);
  char* b = const_cast<char*>(static_cast<const char*>(saved));
  SavedPtrs S;
  S.ln_out = b + L.ln_out;
  S.mean = reinterpret_cast<float*>(b + L.mean);
  S.rstd = reinterpret_cast<float*>(b + L.rstd);
  S.a = b + L.a;
  S.b = b + L.b;
  S.c = half == MTNLG_ATTN ? reinterpret_cast<float*>(b + L.c) : nullptr;
  return S;
}

// ---- GEMMs of each half: (M, N, K) of the forward and backward products ----
struct Shape3 { int64_t M, N, K; };
int half_gemms(const Dims& d, int half, Shape3* out) {
  if (half == MTNLG_ATTN) {
    const int64_t n3 = 3 * d.w;
    const Shape3 g[6] = {{d.T, n3, d.h}, {d.T, d.h, d.w}, {d.T, d.w, d.h},
                         {d.w, d.h, d.T}, {d.h, n3, d.T}, {d.T, d.h, n3}};
    for (int i = 0; i < 6; ++i) out[i] = g[i];
    return 6;
  }
  const Shape3 g[6] = {{d.T, d.fl, d.h}, {d.T, d.h, d.fl}, {d.T, d.fl, d.h},
                       {d.fl, d.h, d.T}, {d.h, d.fl, d.T}, {d.T, d.h, d.fl}};
  for (int i = 0; i < 6; ++i) out[i] = g[i];
  return 6;
}

// ---- workspace layout ----
// gemm: fp32 partials of a GEMM's tail tiles (one GEMM at a time; forward and
// backward); the rest is backward-only scratch.
struct WsLayout {
  size_t gemm, t1, t2, dln, lnp, cs, attn, total;
};

WsLayout ws_layout(const Dims& d, int half) {
  WsLayout L{};
  size_t off = 0;
  Shape3 g[6];
  const int ng = half_gemms(d, half, g);
  size_t gws = 0;
  for (int i = 0; i < ng; ++i)
    gws = std::max(gws, gemm_workspace_bytes(plan_gemm(d.dtype, g[i].M, g[i].N, g[i].K, true), g[i].M, g[i].N));
  L.gemm = off; off = align256(off + gws);
  if (half == MTNLG_ATTN) {
    L.t1 = off; off = align256(off + d.T * d.w * d.eb);        // dO
    L.t2 = off; off = align256(off + d.T * 3 * d.w * d.eb);    // dQKV
    L.attn = off; off = align256(off + attention_bwd_ws(1, (int)d.T, (int)d.nhl));
  } else {
    L.t1 = off; off = align256(off + d.T * d.fl * d.eb);       // dU
    L.t2 = off;
  }
  L.dln = off; off = align256(off + d.T * d.h * d.eb);
  L.lnp = off; off = align256(off + layernorm_bwd_ws(d.T, d.h));
  L.cs = off;  off = align256(off + colsum_ws(d.T, std::max<int64_t>(d.h, std::max<int64_t>(3 * d.w, d.fl))));
  L.total = off;
  return L;
}

// The attention-probability dropout of a layer call (thr 0: none).
AttnDropout attn_dropout(const mtnlg_layer_desc* desc, const Dims& d) {
  AttnDropout a{};
  a.thr = (uint32_t)nearbyint((double)desc->attn_dropout * 65536.0);
  a.scale = a.thr ? (float)(65536.0 / (65536.0 - (double)a.thr)) : 1.0f;
  a.seed = desc->attn_dropout_seed;
  a.site = desc->attn_dropout_site;
  a.head0 = desc->tp_rank * (int)d.nhl;
  return a;
}

// The forward of one half into its saved tensors S; the row-sliced output
// GEMM is skipped when y_partial is NULL (a recompute needs only what is
// saved).
int forward_into(const mtnlg_layer_desc* desc, const Dims& d, int half, const mtnlg_half_params* params,
                 const void* x, void* y_partial, const SavedPtrs& S, void* gws, hipStream_t st) {
  void* ln_out = S.ln_out;
  float* mean = S.mean;
  float* rstd = S.rstd;
  MTNLG_HIP(layernorm_fwd(d.dtype, d.T, d.h, x, params->ln_g, params->ln_b, desc->ln_eps, ln_out, mean, rstd, st),
            "layernorm_fwd");
  if (half == MTNLG_ATTN) {
    void* qkv = S.a;
    void* o = S.b;
    float* lse = S.c;
    const int64_t n3 = 3 * d.w;
    // bf16: Q and K leave the product in fp16 (see the attention kernels)
    const bool f16qk = d.dtype == MTNLG_BF16;
    MTNLG_HIP(gemm(d.dtype, true, false, d.T, n3, d.h, ln_out, d.h, params->w_in, n3, qkv, n3,
                   f16qk ? EPI_BIAS_F16LO : EPI_BIAS, params->b_in, nullptr, nullptr,
                   plan_gemm(d.dtype, d.T, n3, d.h, true), gws, st, f16qk ? (int)(2 * d.w) : 0),
              "qkv gemm");
    MTNLG_HIP(attention_fwd(d.dtype, desc->batch, desc->seq, (int)d.nhl, (int)d.d, qkv, o, lse,
                            attn_dropout(desc, d), st),
              "attention_fwd");
    if (y_partial)
      MTNLG_HIP(gemm(d.dtype, true, false, d.T, d.h, d.w, o, d.w, params->w_out, d.h, y_partial, d.h, EPI_STORE,
                     nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.T, d.h, d.w, true), gws, st),
                "out-proj gemm");
  } else {
    void* u = S.a;
    void* y = S.b;
    MTNLG_HIP(gemm(d.dtype, true, false, d.T, d.fl, d.h, ln_out, d.h, params->w_in, d.fl, u, d.fl, EPI_BIAS_GELU,
                   params->b_in, y, nullptr, plan_gemm(d.dtype, d.T, d.fl, d.h, true), gws, st),
              "mlp-up gemm");
    if (y_partial)
      MTNLG_HIP(gemm(d.dtype, true, false, d.T, d.h, d.fl, y, d.fl, params->w_out, d.h, y_partial, d.h, EPI_STORE,
                     nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.T, d.h, d.fl, true), gws, st),
                "mlp-down gemm");
  }
  return MTNLG_OK;
}


// The backward of one half from its saved tensors (workspace laid out by
// ws_layout). With `dd`, only the input gradient: the weight products and
// the bias column sums are skipped, dU (MLP) or dQKV (ATTN) is written to
// dd->g, and the LayerNorm's (dgamma, dbeta) partial rows to dd->lnp
// (weight_grads reduces them later); grads is unused then.
int backward_from(const mtnlg_layer_desc* desc, const Dims& d, int half, const mtnlg_half_params* params,
                  const void* x, const SavedPtrs& S, const void* dy, void* dx_partial, const mtnlg_half_grads* grads,
                  void* ws, hipStream_t st, const DataOnly* dd = nullptr) {
  const WsLayout W = ws_layout(d, half);
  const bool full = dd == nullptr;
  const void* ln_out = S.ln_out;
  const float* mean = S.mean;
  const float* rstd = S.rstd;
  void* dln = at(ws, W.dln);
  void* cs = at(ws, W.cs);
  void* gws = at(ws, W.gemm);

  if (full) MTNLG_HIP(colsum(d.dtype, d.T, d.h, dy, grads->b_out, cs, st), "b_out colsum");
  if (half == MTNLG_MLP) {
    const void* u = S.a;
    const void* y = S.b;
    void* du = full ? at(ws, W.t1) : dd->g;
    // dU = (dy B^T) * GeLU'(u)
    MTNLG_HIP(gemm(d.dtype, true, true, d.T, d.fl, d.h, dy, d.h, params->w_out, d.h, du, d.fl, EPI_GELU_GRAD,
                   nullptr, nullptr, u, plan_gemm(d.dtype, d.T, d.fl, d.h, true), gws, st),
              "mlp dY gemm");
    if (full) {
      // dB = Y^T dy
      MTNLG_HIP(gemm(d.dtype, false, false, d.fl, d.h, d.T, y, d.fl, dy, d.h, grads->w_out, d.h, EPI_STORE,
                     nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.fl, d.h, d.T, true), gws, st),
                "mlp dB gemm");
      MTNLG_HIP(colsum(d.dtype, d.T, d.fl, du, grads->b_in, cs, st), "mlp da colsum");
      // dA = LN2(x)^T dU
      MTNLG_HIP(gemm(d.dtype, false, false, d.h, d.fl, d.T, ln_out, d.h, du, d.fl, grads->w_in, d.fl, EPI_STORE,
                     nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.h, d.fl, d.T, true), gws, st),
                "mlp dA gemm");
    }
    // dLN = dU A^T
    MTNLG_HIP(gemm(d.dtype, true, true, d.T, d.h, d.fl, du, d.fl, params->w_in, d.fl, dln, d.h, EPI_STORE, nullptr,
                   nullptr, nullptr, plan_gemm(d.dtype, d.T, d.h, d.fl, true), gws, st),
              "mlp dX gemm");
  } else {
    const void* qkv = S.a;
    const void* o = S.b;
    const float* lse = S.c;
    void* dO = at(ws, W.t1);
    void* dqkv = full ? at(ws, W.t2) : dd->g;
    const int64_t n3 = 3 * d.w;
    // dO = dy W_o^T (short N: split K)
    MTNLG_HIP(gemm(d.dtype, true, true, d.T, d.w, d.h, dy, d.h, params->w_out, d.h, dO, d.w, EPI_STORE, nullptr,
                   nullptr, nullptr, plan_gemm(d.dtype, d.T, d.w, d.h, true), gws, st),
              "attn dO gemm");
    // dW_o = O^T dy
    if (full)
      MTNLG_HIP(gemm(d.dtype, false, false, d.w, d.h, d.T, o, d.w, dy, d.h, grads->w_out, d.h, EPI_STORE, nullptr,
                     nullptr, nullptr, plan_gemm(d.dtype, d.w, d.h, d.T, true), gws, st),
                "attn dWo gemm");
    MTNLG_HIP(attention_bwd(d.dtype, desc->batch, desc->seq, (int)d.nhl, (int)d.d, qkv, o, lse, dO, dqkv,
                            at(ws, W.attn), attn_dropout(desc, d), st),
              "attention_bwd");
    if (full) {
      MTNLG_HIP(colsum(d.dtype, d.T, n3, dqkv, grads->b_in, cs, st), "attn dbqkv colsum");
      // dW_qkv = LN1(x)^T dQKV
      MTNLG_HIP(gemm(d.dtype, false, false, d.h, n3, d.T, ln_out, d.h, dqkv, n3, grads->w_in, n3, EPI_STORE,
                     nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.h, n3, d.T, true), gws, st),
                "attn dWqkv gemm");
    }
    // dLN = dQKV W_qkv^T
    MTNLG_HIP(gemm(d.dtype, true, true, d.T, d.h, n3, dqkv, n3, params->w_in, n3, dln, d.h, EPI_STORE, nullptr,
                   nullptr, nullptr, plan_gemm(d.dtype, d.T, d.h, n3, true), gws, st),
              "attn dX gemm");
  }
  if (full)
    MTNLG_HIP(layernorm_bwd(d.dtype, d.dtype, d.T, d.h, dln, x, mean, rstd, params->ln_g, dx_partial, grads->ln_g,
                            grads->ln_b, at(ws, W.lnp), st),
              "layernorm_bwd");
  else
    MTNLG_HIP(layernorm_bwd_partials(d.dtype, d.dtype, d.T, d.h, dln, x, mean, rstd, params->ln_g, dx_partial,
                                     dd->lnp, st),
              "layernorm_bwd");
  return MTNLG_OK;
}

// ---- weight and bias gradients over several micro-batches at once ----
// R = mb * T rows: every operand below holds the micro-batches' rows back to
// back. Workspace: the products' tail partials, then the column sums'.
struct WgLayout {
  size_t gemm, cs, total;
};

WgLayout wg_layout(const Dims& d, int half, int64_t R) {
  const int64_t n_in = half == MTNLG_ATTN ? 3 * d.w : d.fl;  // w_in columns
  const int64_t n_out = half == MTNLG_ATTN ? d.w : d.fl;     // w_out rows
  const Shape3 g[2] = {{n_out, d.h, R}, {d.h, n_in, R}};
  size_t gws = 0;
  for (const Shape3& s : g)
    gws = std::max(gws, gemm_workspace_bytes(plan_gemm(d.dtype, s.M, s.N, s.K, true), s.M, s.N));
  WgLayout L{};
  L.gemm = 0;
  L.cs = align256(gws);
  L.total = L.cs + align256(colsum_ws(R, std::max(d.h, n_in)));
  return L;
}

int weight_grads(const Dims& d, int half, int mb, const SavedPtrs& S, const void* dy_all, const void* g_all,
                 const float* lnp_all, const mtnlg_half_grads* grads, void* ws, hipStream_t st) {
  const int64_t R = (int64_t)mb * d.T;
  const WgLayout W = wg_layout(d, half, R);
  void* gws = at(ws, W.gemm);
  void* cs = at(ws, W.cs);
  MTNLG_HIP(colsum(d.dtype, R, d.h, dy_all, grads->b_out, cs, st), "b_out colsum");
  if (half == MTNLG_MLP) {
    // dB = Y^T dy, db_A = colsum(dU), dA = LN2(x)^T dU over all R rows
    MTNLG_HIP(gemm(d.dtype, false, false, d.fl, d.h, R, S.b, d.fl, dy_all, d.h, grads->w_out, d.h, EPI_STORE,
                   nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.fl, d.h, R, true), gws, st),
              "mlp dB gemm");
    MTNLG_HIP(colsum(d.dtype, R, d.fl, g_all, grads->b_in, cs, st), "mlp da colsum");
    MTNLG_HIP(gemm(d.dtype, false, false, d.h, d.fl, R, S.ln_out, d.h, g_all, d.fl, grads->w_in, d.fl, EPI_STORE,
                   nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.h, d.fl, R, true), gws, st),
              "mlp dA gemm");
  } else {
    const int64_t n3 = 3 * d.w;
    // dW_o = O^T dy, db_qkv = colsum(dQKV), dW_qkv = LN1(x)^T dQKV over all R rows
    MTNLG_HIP(gemm(d.dtype, false, false, d.w, d.h, R, S.b, d.w, dy_all, d.h, grads->w_out, d.h, EPI_STORE,
                   nullptr, nullptr, nullptr, plan_gemm(d.dtype, d.w, d.h, R, true), gws, st),
              "attn dWo gemm");
    MTNLG_HIP(colsum(d.dtype, R, n3, g_all, grads->b_in, cs, st), "attn dbqkv colsum");
    MTNLG_HIP(gemm(d.dtype, false, false, d.h, n3, R, S.ln_out, d.h, g_all, n3, grads->w_in, n3, EPI_STORE, nullptr,
                   nullptr, nullptr, plan_gemm(d.dtype, d.h, n3, R, true), gws, st),
              "attn dWqkv gemm");
  }
  MTNLG_HIP(layernorm_bwd_reduce(d.dtype, mb * layernorm_bwd_blocks(d.T), d.h, lnp_all, grads->ln_g, grads->ln_b,
                                 st),
            "layernorm grads");
  return MTNLG_OK;
}

}  // namespace

// ---- entry points for the pipeline stage (abi_common.hpp) ----
namespace mtnlg {
namespace abi {

int half_saved_sizes(const mtnlg_layer_desc* desc, int half, SavedSizes* out) {
  Dims d;
  const int s = validate_desc(desc, half, &d);
  if (s != MTNLG_OK) return s;
  out->ln_out = (size_t)(d.T * d.h) * d.eb;
  out->stats = (size_t)d.T * sizeof(float);
  out->a = (size_t)(d.T * (half == MTNLG_ATTN ? 3 * d.w : d.fl)) * d.eb;
  out->b = (size_t)(d.T * (half == MTNLG_ATTN ? d.w : d.fl)) * d.eb;
  out->c = half == MTNLG_ATTN ? (size_t)(d.nhl * d.T) * sizeof(float) : 0;
  out->g = out->a;  // dU or dQKV: the shape of a
  out->lnp = (size_t)layernorm_bwd_blocks(d.T) * 2 * (size_t)d.h * sizeof(float);
  out->widest = (size_t)std::max<int64_t>(d.h, std::max<int64_t>(3 * d.w, d.fl)) * d.eb;
  return MTNLG_OK;
}

size_t half_bwd_ws_bytes(const mtnlg_layer_desc* desc, int half) {
  Dims d;
  if (validate_desc(desc, half, &d) != MTNLG_OK) return 0;
  return ws_layout(d, half).total;
}

size_t half_weight_grads_ws_bytes(const mtnlg_layer_desc* desc, int half, int mb) {
  Dims d;
  if (validate_desc(desc, half, &d) != MTNLG_OK) return 0;
  return wg_layout(d, half, (int64_t)mb * d.T).total;
}

int half_fwd(const mtnlg_layer_desc* desc, int half, const mtnlg_half_params* params, const void* x,
             void* y_partial, const SavedPtrs& S, void* ws, hipStream_t st) {
  Dims d;
  const int s = validate_desc(desc, half, &d);
  if (s != MTNLG_OK) return s;
  return forward_into(desc, d, half, params, x, y_partial, S, at(ws, ws_layout(d, half).gemm), st);
}

int half_bwd_data(const mtnlg_layer_desc* desc, int half, const mtnlg_half_params* params, const void* x,
                  const SavedPtrs& S, const void* dy, void* dx_partial, void* g_out, float* lnp_out, void* ws,
                  hipStream_t st) {
  Dims d;
  const int s = validate_desc(desc, half, &d);
  if (s != MTNLG_OK) return s;
  const DataOnly dd{g_out, lnp_out};
  return backward_from(desc, d, half, params, x, S, dy, dx_partial, nullptr, ws, st, &dd);
}

int half_weight_grads(const mtnlg_layer_desc* desc, int half, int mb, const SavedPtrs& S, const void* dy_all,
                      const void* g_all, const float* lnp_all, const mtnlg_half_grads* grads, void* ws,
                      hipStream_t st) {
  Dims d;
  const int s = validate_desc(desc, half, &d);
  if (s != MTNLG_OK) return s;
  return weight_grads(d, half, mb, S, dy_all, g_all, lnp_all, grads, ws, st);
}

}  // namespace abi
}  // namespace mtnlg

namespace {
}  // namespace

extern "C" {

const char* mtnlg_status_str(int32_t status) {
  switch (status) {
    case MTNLG_OK: return "ok";
    case MTNLG_ERR_ARG: return "invalid argument";
    case MTNLG_ERR_SHAPE: return "unsupported or inconsistent shape";
    case MTNLG_ERR_DTYPE: return "unsupported dtype";
    case MTNLG_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MTNLG_ERR_WORKSPACE: return "workspace too small";
    case MTNLG_ERR_HIP: return "HIP error";
    case MTNLG_ERR_UNIMPLEMENTED: return "unimplemented";
    default: return "unknown status";
  }
}

const char* mtnlg_last_error(void) { return g_last_error; }

size_t mtnlg_saved_bytes(const mtnlg_layer_desc* desc, int32_t half) {
  Dims d;
  if (validate_desc(desc, half, &d) != MTNLG_OK) return 0;
  return saved_layout(d, half).total;
}

size_t mtnlg_workspace_bytes(const mtnlg_layer_desc* desc, int32_t half) {
  Dims d;
  if (validate_desc(desc, half, &d) != MTNLG_OK) return 0;
  return ws_layout(d, half).total;
}

int mtnlg_layer_fwd(const mtnlg_layer_desc* desc, int32_t half, const mtnlg_half_params* params, const void* x,
                    void* y_partial, void* saved, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  Dims d;
  int s = validate_desc(desc, half, &d);
  if (s != MTNLG_OK) return s;
  if (!params) return fail(MTNLG_ERR_ARG, "params is NULL");
  CHECK_PTR(params->ln_g);
  CHECK_PTR(params->ln_b);
  CHECK_PTR(params->w_in);
  CHECK_PTR(params->b_in);
  CHECK_PTR(params->w_out);
  CHECK_PTR(x);
  CHECK_PTR(y_partial);
  CHECK_PTR(saved);
  const WsLayout W = ws_layout(d, half);
  const size_t need = W.t1;  // the forward uses only the GEMM partial region, which comes first
  if (need > 0) {
    CHECK_PTR(ws);
    if (ws_bytes < need) return fail(MTNLG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  }
  void* gws = need > 0 ? at(ws, W.gemm) : nullptr;
  return forward_into(desc, d, half, params, x, y_partial, saved_ptrs(saved, d, half), gws,
                      static_cast<hipStream_t>(stream));
}

int mtnlg_layer_bwd(const mtnlg_layer_desc* desc, int32_t half, const mtnlg_half_params* params, const void* x,
                    const void* saved, const void* dy, void* dx_partial, const mtnlg_half_grads* grads, void* ws,
                    size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  Dims d;
  int s = validate_desc(desc, half, &d);
  if (s != MTNLG_OK) return s;
  if (!params) return fail(MTNLG_ERR_ARG, "params is NULL");
  if (!grads) return fail(MTNLG_ERR_ARG, "grads is NULL");
  CHECK_PTR(params->ln_g);
  CHECK_PTR(params->ln_b);
  CHECK_PTR(params->w_in);
  CHECK_PTR(params->b_in);
  CHECK_PTR(params->w_out);
  CHECK_PTR(grads->ln_g);
  CHECK_PTR(grads->ln_b);
  CHECK_PTR(grads->w_in);
  CHECK_PTR(grads->b_in);
  CHECK_PTR(grads->w_out);
  CHECK_PTR(grads->b_out);
  CHECK_PTR(x);
  CHECK_PTR(saved);
  CHECK_PTR(dy);
  CHECK_PTR(dx_partial);
  CHECK_PTR(ws);
  const WsLayout W = ws_layout(d, half);
  if (ws_bytes < W.total)
    return fail(MTNLG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, W.total);
  return backward_from(desc, d, half, params, x, saved_ptrs(saved, d, half), dy, dx_partial, grads, ws,
                       static_cast<hipStream_t>(stream));
}

size_t mtnlg_recompute_workspace_bytes(const mtnlg_layer_desc* desc, int32_t half) {
  Dims d;
  if (validate_desc(desc, half, &d) != MTNLG_OK) return 0;
  return align256(saved_layout(d, half).total) + ws_layout(d, half).total;
}

int mtnlg_layer_bwd_recompute(const mtnlg_layer_desc* desc, int32_t half, const mtnlg_half_params* params,
                              const void* x, const void* dy, void* dx_partial, const mtnlg_half_grads* grads,
                              void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  Dims d;
  int s = validate_desc(desc, half, &d);
  if (s != MTNLG_OK) return s;
  if (!params) return fail(MTNLG_ERR_ARG, "params is NULL");
  if (!grads) return fail(MTNLG_ERR_ARG, "grads is NULL");
  CHECK_PTR(params->ln_g);
  CHECK_PTR(params->ln_b);
  CHECK_PTR(params->w_in);
  CHECK_PTR(params->b_in);
  CHECK_PTR(params->w_out);
  CHECK_PTR(grads->ln_g);
  CHECK_PTR(grads->ln_b);
  CHECK_PTR(grads->w_in);
  CHECK_PTR(grads->b_in);
  CHECK_PTR(grads->w_out);
  CHECK_PTR(grads->b_out);
  CHECK_PTR(x);
  CHECK_PTR(dy);
  CHECK_PTR(dx_partial);
  CHECK_PTR(ws);
  const size_t sv = align256(saved_layout(d, half).total);
  const WsLayout W = ws_layout(d, half);
  if (ws_bytes < sv + W.total)
    return fail(MTNLG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, sv + W.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* saved = ws;
  void* rest = at(ws, sv);
  const SavedPtrs S = saved_ptrs(saved, d, half);
  s = forward_into(desc, d, half, params, x, nullptr, S, at(rest, W.gemm), st);
  if (s != MTNLG_OK) return s;
  return backward_from(desc, d, half, params, x, S, dy, dx_partial, grads, rest, st);
}

int mtnlg_reduce_partials(int64_t rows, int64_t cols, int32_t dtype, const void* const* partials, int32_t n,
                          const void* residual, const void* bias, void* out, void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (rows < 0 || cols <= 0 || cols % 8) return fail(MTNLG_ERR_SHAPE, "rows >= 0 and cols a positive multiple of 8");
  if (n < 1 || n > kMaxPartials) return fail(MTNLG_ERR_ARG, "n must be in [1, %d]", kMaxPartials);
  if (!partials) return fail(MTNLG_ERR_ARG, "partials is NULL");
  for (int j = 0; j < n; ++j) {
    int st = check_ptr(partials[j], "partials[j]");
    if (st != MTNLG_OK) return st;
  }
  if (residual) CHECK_PTR(residual);
  if (bias) CHECK_PTR(bias);
  CHECK_PTR(out);
  MTNLG_HIP(reduce_partials(dtype, rows, cols, partials, n, residual, bias, out, static_cast<hipStream_t>(stream)),
            "reduce_partials");
  return MTNLG_OK;
}

static int dropout_thr(const mtnlg_dropout* dr, uint32_t* thr) {
  if (!dr) return fail(MTNLG_ERR_ARG, "dropout is NULL");
  if (!(dr->p >= 0.0f && dr->p < 1.0f)) return fail(MTNLG_ERR_ARG, "dropout rate must be in [0, 1)");
  *thr = (uint32_t)nearbyint((double)dr->p * 65536.0);
  if (*thr >= 65536u) return fail(MTNLG_ERR_ARG, "dropout rate rounds to 1");
  return MTNLG_OK;
}

int mtnlg_reduce_partials_dropout(int64_t rows, int64_t cols, int32_t dtype, const void* const* partials, int32_t n,
                                  const void* residual, const void* bias, const mtnlg_dropout* dropout, void* out,
                                  void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return fail(MTNLG_ERR_SHAPE, "rows >= 0, cols > 0 and cols %% 8 == 0");
  if (!partials || n < 1 || n > kMaxPartials) return fail(MTNLG_ERR_ARG, "1 <= n <= %d partials", kMaxPartials);
  uint32_t thr;
  int s = dropout_thr(dropout, &thr);
  if (s != MTNLG_OK) return s;
  for (int j = 0; j < n; ++j) {
    s = check_ptr(partials[j], "partials[j]");
    if (s != MTNLG_OK) return s;
  }
  if (residual) CHECK_PTR(residual);
  if (bias) CHECK_PTR(bias);
  CHECK_PTR(out);
  MTNLG_HIP(reduce_partials_dropout(dtype, rows, cols, partials, n, residual, bias, out, dropout->seed,
                                    dropout->site, thr, static_cast<hipStream_t>(stream)),
            "reduce_partials_dropout");
  return MTNLG_OK;
}

int mtnlg_dropout_bwd(int64_t rows, int64_t cols, int32_t dtype, const void* dy, const mtnlg_dropout* dropout,
                      void* dz, void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return fail(MTNLG_ERR_SHAPE, "rows >= 0, cols > 0 and cols %% 8 == 0");
  uint32_t thr;
  int s = dropout_thr(dropout, &thr);
  if (s != MTNLG_OK) return s;
  CHECK_PTR(dy);
  CHECK_PTR(dz);
  MTNLG_HIP(dropout_bwd(dtype, rows * cols, dy, dz, dropout->seed, dropout->site, thr,
                        static_cast<hipStream_t>(stream)),
            "dropout_bwd");
  return MTNLG_OK;
}

int mtnlg_grad_accumulate(int64_t n, int32_t dtype, const void* grad, float* acc, int32_t overwrite, void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (n < 0) return fail(MTNLG_ERR_SHAPE, "n < 0");
  if (n == 0) return MTNLG_OK;
  CHECK_PTR(grad);
  CHECK_PTR(acc);
  MTNLG_HIP(grad_accumulate(n, dtype, grad, acc, overwrite != 0, static_cast<hipStream_t>(stream)),
            "grad_accumulate");
  return MTNLG_OK;
}

size_t mtnlg_adam_workspace_bytes(int64_t n) { return n < 0 ? 0 : adam_ws(n); }

}  // extern "C"

namespace mtnlg {
namespace abi {
int adam_args(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v, const float* grad,
              void* w_bf16, float* stats, const void* ws, size_t ws_bytes, AdamScalars* c) {
  if (!cfg) return fail(MTNLG_ERR_ARG, "cfg is NULL");
  if (n < 0) return fail(MTNLG_ERR_SHAPE, "n < 0");
  if (cfg->step < 1) return fail(MTNLG_ERR_ARG, "step must be >= 1");
  if (!(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f) || !(cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f))
    return fail(MTNLG_ERR_ARG, "betas must be in [0, 1)");
  if (!(cfg->eps > 0.0f) || !(cfg->lr >= 0.0f) || !(cfg->weight_decay >= 0.0f) || !isfinite(cfg->inv_loss_scale))
    return fail(MTNLG_ERR_ARG, "eps > 0, lr >= 0, weight_decay >= 0 and a finite inv_loss_scale are required");
  CHECK_PTR(master);
  CHECK_PTR(m);
  CHECK_PTR(v);
  CHECK_PTR(grad);
  CHECK_PTR(stats);
  if (ws != kNoWorkspace) {
    CHECK_PTR(ws);
    if (ws_bytes < adam_ws(n)) return fail(MTNLG_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, adam_ws(n));
  }
  if (w_bf16) CHECK_PTR(w_bf16);
  c->lr = cfg->lr;
  c->beta1 = cfg->beta1;
  c->beta2 = cfg->beta2;
  c->eps = cfg->eps;
  c->weight_decay = cfg->weight_decay;
  c->max_grad_norm = cfg->max_grad_norm;
  c->inv_loss_scale = cfg->inv_loss_scale;
  c->inv_bc1 = (float)(1.0 / (1.0 - pow((double)cfg->beta1, (double)cfg->step)));
  c->inv_bc2 = (float)(1.0 / (1.0 - pow((double)cfg->beta2, (double)cfg->step)));
  return MTNLG_OK;
}
}  // namespace abi
}  // namespace mtnlg

extern "C" {

int mtnlg_adam_step(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v, const float* grad,
                    void* w_bf16, float* stats, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  AdamScalars c{};
  const int s = adam_args(cfg, n, master, m, v, grad, w_bf16, stats, ws, ws_bytes, &c);
  if (s != MTNLG_OK) return s;
  MTNLG_HIP(adam_step(c, n, master, m, v, grad, w_bf16, stats, ws, static_cast<hipStream_t>(stream)), "adam_step");
  return MTNLG_OK;
}

size_t mtnlg_adam_static_scratch_bytes(void) { return adam_static_scratch_bytes(); }

int mtnlg_adam_step_noalloc(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v,
                            const float* grad, void* w_bf16, float* stats, void* stream) {
  g_last_error[0] = 0;
  AdamScalars c{};
  const int s = adam_args(cfg, n, master, m, v, grad, w_bf16, stats, kNoWorkspace, 0, &c);
  if (s != MTNLG_OK) return s;
  MTNLG_HIP(adam_step_static(c, n, master, m, v, grad, w_bf16, stats, static_cast<hipStream_t>(stream)),
            "adam_step_static");
  return MTNLG_OK;
}

int mtnlg_grad_accumulate_norm(int64_t n, int32_t dtype, const void* grad, float* acc, int32_t overwrite,
                               float inv_loss_scale, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (n < 0) return fail(MTNLG_ERR_SHAPE, "n < 0");
  if (!isfinite(inv_loss_scale)) return fail(MTNLG_ERR_ARG, "inv_loss_scale must be finite");
  if (n > 0) {
    CHECK_PTR(grad);
    CHECK_PTR(acc);
  }
  CHECK_PTR(ws);
  if (ws_bytes < adam_ws(n)) return fail(MTNLG_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, adam_ws(n));
  MTNLG_HIP(grad_accumulate_norm(n, dtype, grad, acc, overwrite != 0, inv_loss_scale, ws,
                                 static_cast<hipStream_t>(stream)),
            "grad_accumulate_norm");
  return MTNLG_OK;
}

int mtnlg_adam_update(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v, const float* grad,
                      void* w_bf16, float* stats, const void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  AdamScalars c{};
  const int s = adam_args(cfg, n, master, m, v, grad, w_bf16, stats, ws, ws_bytes, &c);
  if (s != MTNLG_OK) return s;
  MTNLG_HIP(adam_update(c, n, master, m, v, grad, w_bf16, stats, ws, static_cast<hipStream_t>(stream)),
            "adam_update");
  return MTNLG_OK;
}

int mtnlg_adam_stream_reference(int64_t n, float* master, float* m, float* v, const float* grad, void* w_bf16,
                                void* stream) {
  g_last_error[0] = 0;
  if (n < 0) return fail(MTNLG_ERR_SHAPE, "n < 0");
  if (n == 0) return MTNLG_OK;
  CHECK_PTR(master);
  CHECK_PTR(m);
  CHECK_PTR(v);
  CHECK_PTR(grad);
  if (w_bf16) CHECK_PTR(w_bf16);
  MTNLG_HIP(adam_streams(n, master, m, v, grad, w_bf16, static_cast<hipStream_t>(stream)), "adam_streams");
  return MTNLG_OK;
}

static bool gemm_shape_ok(int32_t dtype, int64_t M, int64_t N, int64_t K) {
  // every operand must stay below 2 GiB: the kernels address operands through
  // 32-bit buffer offsets and mark out-of-range elements with offset 2^31
  const int64_t eb = elem_bytes(dtype), lim = (int64_t)1 << 31;
  return M >= 8 && N >= 8 && K >= 8 && M % 8 == 0 && N % 8 == 0 && K % 8 == 0 && M < lim && N < lim && K < lim &&
         M * K * eb < lim && K * N * eb < lim && M * N * eb < lim;
}

size_t mtnlg_gemm_workspace_bytes(int32_t dtype, int64_t M, int64_t N, int64_t K) {
  if ((dtype != MTNLG_F32 && dtype != MTNLG_BF16) || !gemm_shape_ok(dtype, M, N, K)) return 0;
  return gemm_workspace_bytes(plan_gemm(dtype, M, N, K, true), M, N);
}

int mtnlg_gemm(int32_t dtype, int32_t trans_a, int32_t trans_b, int64_t M, int64_t N, int64_t K, const void* A,
               const void* B, void* C, const void* bias, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (!gemm_shape_ok(dtype, M, N, K))
    return fail(MTNLG_ERR_SHAPE, "M, N, K must be positive multiples of 8 with operands below 2 GiB");
  CHECK_PTR(A);
  CHECK_PTR(B);
  CHECK_PTR(C);
  if (bias) CHECK_PTR(bias);
  const GemmPlan pl = plan_gemm(dtype, M, N, K, true);
  const size_t need = gemm_workspace_bytes(pl, M, N);
  if (need > 0) {
    CHECK_PTR(ws);
    if (ws_bytes < need) return fail(MTNLG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  }
  const bool a_kc = trans_a == 0, b_kc = trans_b != 0;
  const int64_t lda = a_kc ? K : M;
  const int64_t ldb = b_kc ? K : N;
  MTNLG_HIP(gemm(dtype, a_kc, b_kc, M, N, K, A, lda, B, ldb, C, N, bias ? EPI_BIAS : EPI_STORE, bias, nullptr,
                 nullptr, pl, need > 0 ? ws : nullptr, static_cast<hipStream_t>(stream)),
            "gemm");
  return MTNLG_OK;
}

int mtnlg_layernorm_fwd(int32_t dtype, int64_t rows, int64_t cols, const void* x, const void* gamma,
                        const void* beta, float eps, void* y, float* mean, float* rstd, void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (rows < 0 || cols < 8 || cols % 8 || cols > 32768) return fail(MTNLG_ERR_SHAPE, "bad rows/cols");
  if (!(eps > 0.0f)) return fail(MTNLG_ERR_ARG, "eps must be positive");
  if (rows == 0) return MTNLG_OK;
  CHECK_PTR(x);
  CHECK_PTR(gamma);
  CHECK_PTR(beta);
  CHECK_PTR(y);
  CHECK_PTR(mean);
  CHECK_PTR(rstd);
  MTNLG_HIP(layernorm_fwd(dtype, rows, cols, x, gamma, beta, eps, y, mean, rstd, static_cast<hipStream_t>(stream)),
            "layernorm_fwd");
  return MTNLG_OK;
}

size_t mtnlg_layernorm_bwd_workspace_bytes(int64_t rows, int64_t cols) {
  return rows <= 0 || cols <= 0 ? 0 : layernorm_bwd_ws(rows, cols);
}

int mtnlg_layernorm_bwd(int32_t dtype, int64_t rows, int64_t cols, const void* gy, const void* x, const float* mean,
                        const float* rstd, const void* gamma, void* dx, void* dgamma, void* dbeta, void* ws,
                        size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (rows <= 0 || cols < 8 || cols % 8 || cols > 32768) return fail(MTNLG_ERR_SHAPE, "bad rows/cols");
  CHECK_PTR(gy);
  CHECK_PTR(x);
  CHECK_PTR(mean);
  CHECK_PTR(rstd);
  CHECK_PTR(gamma);
  CHECK_PTR(dx);
  CHECK_PTR(dgamma);
  CHECK_PTR(dbeta);
  CHECK_PTR(ws);
  if (ws_bytes < layernorm_bwd_ws(rows, cols)) return fail(MTNLG_ERR_WORKSPACE, "workspace too small");
  MTNLG_HIP(layernorm_bwd(dtype, dtype, rows, cols, gy, x, mean, rstd, gamma, dx, dgamma, dbeta, ws,
                          static_cast<hipStream_t>(stream)),
            "layernorm_bwd");
  return MTNLG_OK;
}

static int validate_attn(int32_t dtype, int32_t batch, int32_t seq, int32_t heads, int32_t head_dim) {
  if (dtype != MTNLG_F32 && dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "dtype %d unsupported", dtype);
  if (batch <= 0 || seq <= 0 || heads <= 0) return fail(MTNLG_ERR_SHAPE, "dimensions must be positive");
  if (seq % 128) return fail(MTNLG_ERR_SHAPE, "seq must be a multiple of 128");
  const bool ok = dtype == MTNLG_BF16 ? (head_dim == 64 || head_dim == 128 || head_dim == 160)
                                      : (head_dim == 64 || head_dim == 128);
  if (!ok) return fail(MTNLG_ERR_SHAPE, "head_dim %d unsupported", head_dim);
  if ((int64_t)seq * 3 * heads * head_dim * (int64_t)elem_bytes(dtype) >= ((int64_t)1 << 31))
    return fail(MTNLG_ERR_SHAPE, "one sequence of qkv must stay below 2 GiB");
  return MTNLG_OK;
}

int mtnlg_attention_fwd(int32_t dtype, int32_t batch, int32_t seq, int32_t heads, int32_t head_dim, const void* qkv,
                        void* o, float* lse, void* stream) {
  g_last_error[0] = 0;
  int s = validate_attn(dtype, batch, seq, heads, head_dim);
  if (s != MTNLG_OK) return s;
  CHECK_PTR(qkv);
  CHECK_PTR(o);
  CHECK_PTR(lse);
  MTNLG_HIP(attention_fwd(dtype, batch, seq, heads, head_dim, qkv, o, lse, AttnDropout{},
                          static_cast<hipStream_t>(stream)),
            "attention_fwd");
  return MTNLG_OK;
}

size_t mtnlg_attention_bwd_workspace_bytes(int32_t batch, int32_t seq, int32_t heads) {
  return batch <= 0 || seq <= 0 || heads <= 0 ? 0 : attention_bwd_ws(batch, seq, heads);
}

int mtnlg_attention_bwd(int32_t dtype, int32_t batch, int32_t seq, int32_t heads, int32_t head_dim, const void* qkv,
                        const void* o, const float* lse, const void* do_, void* dqkv, void* ws, size_t ws_bytes,
                        void* stream) {
  g_last_error[0] = 0;
  int s = validate_attn(dtype, batch, seq, heads, head_dim);
  if (s != MTNLG_OK) return s;
  CHECK_PTR(qkv);
  CHECK_PTR(o);
  CHECK_PTR(lse);
  CHECK_PTR(do_);
  CHECK_PTR(dqkv);
  CHECK_PTR(ws);
  if (ws_bytes < attention_bwd_ws(batch, seq, heads)) return fail(MTNLG_ERR_WORKSPACE, "workspace too small");
  MTNLG_HIP(attention_bwd(dtype, batch, seq, heads, head_dim, qkv, o, lse, do_, dqkv, ws, AttnDropout{},
                          static_cast<hipStream_t>(stream)),
            "attention_bwd");
  return MTNLG_OK;
}

}  // extern "C"
