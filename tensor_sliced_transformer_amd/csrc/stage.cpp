// One pipeline stage of chained layer slices on one GPU (include/mtnlg.h,
// "One pipeline stage on one GPU"): the host-side schedule that runs the
// micro-batches through the layer-half entry points, accumulates the flat
// gradient, and takes the Adam step on the norm folded into the last
// accumulation.
//
// In MT-NLG 530B the 105 layers are split over 35 pipeline stages with 8-way
// tensor slicing inside each (jiqizhixin MT-NLG article, system paragraph), so
// one GPU holds 3 layer slices, and gradients of several micro-batches are
// accumulated before each step (Elamur summary, Key points). Each micro-batch
// runs forward then backward before the next starts: with no neighbouring
// stage this is the order a one-forward-one-backward schedule gives.
//
// Gradients over the micro-batches: the sum over micro-batches of X_k^T dY_k
// is X^T dY with the micro-batches' rows stacked, so by default (saved
// tensors kept) the backward of each micro-batch computes only the input
// gradients and keeps what the weight gradients need (each half's saved
// tensors, its output gradient, its dU or dQKV and its LayerNorm partial
// rows, every micro-batch's copy of a field back to back in HBM); after the
// last micro-batch's backward of a layer, each of its weight gradients is one
// product over micro_batches * T rows, with fp32 accumulation throughout, and
// each bias gradient one column sum. The products then run with a K of
// micro_batches * T instead of T (fewer tile epilogues per FLOP) and no
// per-micro-batch accumulation pass is left. The recompute schedule (which
// keeps only each half's input) and per_micro_batch_grads = 1 instead
// accumulate every micro-batch's gradient into the fp32 accumulator.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "abi_common.hpp"

using namespace mtnlg;
using namespace mtnlg::abi;

namespace {

constexpr int kTensors = 6;  // ln_g, ln_b, w_in, b_in, w_out, b_out

struct StageDims {
  int64_t T, h, act;          // rows, hidden, elements of one [T, h] activation
  int64_t win[2], wout[2];    // columns of w_in and rows of w_out per half
  int64_t per_layer;          // parameter elements of one layer
};

int stage_dims(const mtnlg_stage_desc* sd, StageDims* o) {
  if (!sd) return fail(MTNLG_ERR_ARG, "stage desc is NULL");
  if (sd->layers < 1 || sd->micro_batches < 1) return fail(MTNLG_ERR_SHAPE, "layers and micro_batches must be >= 1");
  if (sd->recompute != 0 && sd->recompute != 1) return fail(MTNLG_ERR_ARG, "recompute must be 0 or 1");
  if (sd->per_micro_batch_grads != 0 && sd->per_micro_batch_grads != 1)
    return fail(MTNLG_ERR_ARG, "per_micro_batch_grads must be 0 or 1");
  if (!(sd->dropout_p >= 0.0f && sd->dropout_p < 1.0f) || nearbyint((double)sd->dropout_p * 65536.0) >= 65536.0)
    return fail(MTNLG_ERR_ARG, "dropout_p must be in [0, 1)");
  const mtnlg_layer_desc& L = sd->layer;
  if (L.dtype != MTNLG_BF16) return fail(MTNLG_ERR_DTYPE, "a stage runs bf16 layers (mixed precision)");
  if (mtnlg_saved_bytes(&L, MTNLG_ATTN) == 0 || mtnlg_saved_bytes(&L, MTNLG_MLP) == 0)
    return fail(MTNLG_ERR_SHAPE, "invalid layer descriptor");
  o->T = (int64_t)L.batch * L.seq;
  o->h = L.hidden;
  o->wout[MTNLG_ATTN] = (int64_t)(L.heads / L.tp_size) * (L.hidden / L.heads);  // local heads * head_dim
  o->win[MTNLG_ATTN] = 3 * o->wout[MTNLG_ATTN];                                   // q, k and v
  o->win[MTNLG_MLP] = o->wout[MTNLG_MLP] = (int64_t)L.ffn / L.tp_size;
  o->act = o->T * o->h;
  o->per_layer = 0;
  for (int half = 0; half < 2; ++half)
    o->per_layer += 2 * o->h + o->h * o->win[half] + o->win[half] + o->wout[half] * o->h + o->h;
  return MTNLG_OK;
}

void layer_offsets(const StageDims& d, int layer, int64_t off[2][kTensors]) {
  int64_t p = (int64_t)layer * d.per_layer;
  for (int half = 0; half < 2; ++half) {
    const int64_t sizes[kTensors] = {d.h, d.h, d.h * d.win[half], d.win[half], d.wout[half] * d.h, d.h};
    for (int t = 0; t < kTensors; ++t) {
      off[half][t] = p;
      p += sizes[t];
    }
  }
}

// Batched weight gradients (saved tensors kept, per_micro_batch_grads = 0):
// per layer and half, each saved field, the half's output gradient, its dU
// or dQKV and its LayerNorm partial rows, every micro-batch's copy of a field
// back to back, so that a weight gradient is one product over mb * T rows.
// Off when a batched operand would reach the GEMM's 2 GiB operand bound.
bool stage_batched(const mtnlg_stage_desc* sd) {
  if (sd->recompute || sd->per_micro_batch_grads) return false;
  SavedSizes z;
  if (half_saved_sizes(&sd->layer, MTNLG_ATTN, &z) != MTNLG_OK) return false;
  const int64_t T = (int64_t)sd->layer.batch * sd->layer.seq;
  return (int64_t)sd->micro_batches * T * (int64_t)z.widest < ((int64_t)1 << 31);
}

struct HalfBlock {  // byte offsets within one (layer, half) block of the batched region
  size_t ln_out, mean, rstd, a, b, c, dy, g, lnp, total;
  SavedSizes sz;
};

HalfBlock half_block(const mtnlg_stage_desc* sd, int half) {
  HalfBlock B{};
  half_saved_sizes(&sd->layer, half, &B.sz);
  const size_t mb = (size_t)sd->micro_batches;
  const size_t act = (size_t)sd->layer.batch * sd->layer.seq * sd->layer.hidden * 2;
  size_t p = 0;
  B.ln_out = p; p += align256(mb * B.sz.ln_out);
  B.mean = p;   p += align256(mb * B.sz.stats);
  B.rstd = p;   p += align256(mb * B.sz.stats);
  B.a = p;      p += align256(mb * B.sz.a);
  B.b = p;      p += align256(mb * B.sz.b);
  B.c = p;      p += align256(mb * B.sz.c);
  B.dy = p;     p += align256(mb * act);
  B.g = p;      p += align256(mb * B.sz.g);
  B.lnp = p;    p += align256(mb * B.sz.lnp);
  B.total = p;
  return B;
}

// Workspace regions, each on a 256-byte boundary.
struct StageWs {
  size_t adam, xin, mid, part, g1, g2, dz, saved, layer, wg, total;
  size_t saved_a, saved_m;  // bytes of one layer's saved tensors per half
  size_t block[2];          // batched: bytes of one layer's block per half
};

StageWs stage_ws(const mtnlg_stage_desc* sd, const StageDims& d, int64_t n) {
  const mtnlg_layer_desc* L = &sd->layer;
  const size_t act = align256((size_t)d.act * 2);
  StageWs w{};
  w.saved_a = align256(mtnlg_saved_bytes(L, MTNLG_ATTN));
  w.saved_m = align256(mtnlg_saved_bytes(L, MTNLG_MLP));
  size_t p = 0;
  w.adam = p;
  p += align256(mtnlg_adam_workspace_bytes(n));
  w.xin = p;  // inputs of layers 1 .. layers-1 (layer 0 reads the caller's x)
  p += act * (size_t)(sd->layers - 1);
  w.mid = p;  // each layer's MLP-half input X1
  p += act * (size_t)sd->layers;
  w.part = p;  // one slice partial (forward) or input-gradient partial (backward)
  p += act;
  w.g1 = p;
  p += act;
  w.g2 = p;
  p += act;
  w.dz = p;  // the masked gradient a half's backward starts from (dropout only)
  p += sd->dropout_p > 0.0f ? act : 0;
  w.saved = p;  // every layer's saved tensors, or one scratch set when recomputing
  const bool batched = stage_batched(sd);
  if (batched) {
    // every layer's and micro-batch's, as per-(layer, half) blocks
    for (int half = 0; half < 2; ++half) w.block[half] = half_block(sd, half).total;
    p += (w.block[0] + w.block[1]) * (size_t)sd->layers;
  } else {
    p += sd->recompute ? std::max(w.saved_a, w.saved_m) : (w.saved_a + w.saved_m) * (size_t)sd->layers;
  }
  w.wg = p;  // the weight-gradient products' and column sums' scratch (batched)
  if (batched)
    p += align256(std::max(half_weight_grads_ws_bytes(L, MTNLG_ATTN, sd->micro_batches),
                           half_weight_grads_ws_bytes(L, MTNLG_MLP, sd->micro_batches)));
  w.layer = p;
  const size_t lw = sd->recompute
                        ? std::max(mtnlg_recompute_workspace_bytes(L, MTNLG_ATTN),
                                   mtnlg_recompute_workspace_bytes(L, MTNLG_MLP))
                        : std::max(mtnlg_workspace_bytes(L, MTNLG_ATTN), mtnlg_workspace_bytes(L, MTNLG_MLP));
  p += align256(lw);
  w.total = p;
  return w;
}

// Events that order the stage step's two streams, created on first use and
// kept, per thread and device, until the process ends: a step records and
// waits on them in issue order, and a later step on the same thread records
// them again (a stream wait refers to the record made before it, so the reuse
// is safe). Only a step with more layers than any before it on this thread
// and device creates events; the others allocate nothing on the host.
constexpr int kMaxDevices = 64;
struct EventPool {
  std::vector<hipEvent_t> ev[kMaxDevices];
  // 2 * layers events of the current device: [0, layers) "backward done",
  // [layers, 2 * layers) "accumulation done"
  hipError_t get(int layers, hipEvent_t** out) {
    int dev = 0;
    hipError_t r = hipGetDevice(&dev);
    if (r != hipSuccess) return r;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::vector<hipEvent_t>& v = ev[dev];
    while (v.size() < (size_t)(2 * layers)) {
      hipEvent_t e;
      r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
      v.push_back(e);
    }
    *out = v.data();
    return hipSuccess;
  }
};
thread_local EventPool t_events;

#define STAGE_CALL(call)          \
  do {                            \
    const int s_ = (call);        \
    if (s_ != MTNLG_OK) return s_; \
  } while (0)

}  // namespace

extern "C" {

int64_t mtnlg_stage_param_count(const mtnlg_stage_desc* desc) {
  StageDims d;
  if (stage_dims(desc, &d) != MTNLG_OK) return -1;
  return d.per_layer * desc->layers;
}

int mtnlg_stage_param_offsets(const mtnlg_stage_desc* desc, int64_t* off) {
  g_last_error[0] = 0;
  StageDims d;
  STAGE_CALL(stage_dims(desc, &d));
  if (!off) return fail(MTNLG_ERR_ARG, "off is NULL");
  for (int l = 0; l < desc->layers; ++l) {
    int64_t o[2][kTensors];
    layer_offsets(d, l, o);
    memcpy(off + (size_t)l * 2 * kTensors, o, sizeof(o));
  }
  return MTNLG_OK;
}

size_t mtnlg_stage_workspace_bytes(const mtnlg_stage_desc* desc) {
  StageDims d;
  if (stage_dims(desc, &d) != MTNLG_OK) return 0;
  return stage_ws(desc, d, d.per_layer * desc->layers).total;
}

int mtnlg_stage_step(const mtnlg_stage_desc* desc, const mtnlg_adam_cfg* cfg, void* w, float* master, float* m,
                     float* v, void* grad, float* acc, const void* x, const void* dy, void* y, void* dx,
                     float* stats, void* ws, size_t ws_bytes, void* stream, void* aux_stream) {
  g_last_error[0] = 0;
  StageDims d;
  STAGE_CALL(stage_dims(desc, &d));
  const int64_t n = d.per_layer * desc->layers;
  // everything is checked before the first launch
  AdamScalars sc;
  STAGE_CALL(adam_args(cfg, n, master, m, v, acc, w, stats, ws, ws_bytes, &sc));
  CHECK_PTR(grad);
  CHECK_PTR(x);
  CHECK_PTR(dy);
  CHECK_PTR(y);
  CHECK_PTR(dx);
  const StageWs W = stage_ws(desc, d, n);
  if (ws_bytes < W.total) return fail(MTNLG_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, W.total);

  // With a second stream, each layer's gradient of micro-batch k < last is
  // accumulated on it as soon as that layer's backward is done, overlapping the
  // HBM-bound accumulation with the MFMA-bound work of the following layers and
  // micro-batches; the next micro-batch's backward of that layer waits for it.
  const int nl = desc->layers, mb = desc->micro_batches;
  hipStream_t S = static_cast<hipStream_t>(stream), A = static_cast<hipStream_t>(aux_stream);
  const bool overlap = A != nullptr && A != S && mb > 1 && !stage_batched(desc);
  hipEvent_t* events = nullptr;
  if (overlap) MTNLG_HIP(t_events.get(nl, &events), "hipEventCreateWithFlags");
  hipEvent_t* const bwd_done = events;
  hipEvent_t* const acc_done = events ? events + nl : nullptr;

  const mtnlg_layer_desc* L = &desc->layer;
  const size_t act = (size_t)d.act * 2;
  const size_t act_al = align256(act);
  char* base = static_cast<char*>(ws);
  char* part = base + W.part;
  char* g1 = base + W.g1;
  char* g2 = base + W.g2;
  char* lws = base + W.layer;
  const size_t lws_bytes = ws_bytes - W.layer;
  char* wb = static_cast<char*>(w);
  char* gb = static_cast<char*>(grad);
  auto xin = [&](int l, int k) -> const void* {
    return l == 0 ? static_cast<const char*>(x) + (size_t)k * act : base + W.xin + (size_t)(l - 1) * act_al;
  };
  auto xout = [&](int l, int k) -> void* {
    return l == desc->layers - 1 ? static_cast<char*>(y) + (size_t)k * act : base + W.xin + (size_t)l * act_al;
  };
  auto mid = [&](int l) -> void* { return base + W.mid + (size_t)l * act_al; };
  const bool drop = desc->dropout_p > 0.0f;
  auto site = [&](int k, int l, int half) -> uint64_t {
    return ((uint64_t)k * (uint64_t)desc->layers + (uint64_t)l) * 2u + (uint64_t)half;
  };
  // layer l of micro-batch k: its own attention-probability mask
  auto layer_of = [&](int k, int l) -> mtnlg_layer_desc {
    mtnlg_layer_desc Lk = *L;
    Lk.attn_dropout_site += (uint64_t)k * (uint64_t)desc->layers + (uint64_t)l;
    return Lk;
  };
  auto saved = [&](int l, int half) -> void* {
    if (desc->recompute) return base + W.saved;
    return base + W.saved + (size_t)l * (W.saved_a + W.saved_m) + (half == MTNLG_MLP ? W.saved_a : 0);
  };

  if (stage_batched(desc)) {
    // ---- batched weight gradients ----
    const HalfBlock HB[2] = {half_block(desc, MTNLG_ATTN), half_block(desc, MTNLG_MLP)};
    auto block = [&](int l, int half) -> char* {
      return base + W.saved + (size_t)l * (W.block[0] + W.block[1]) + (half == MTNLG_MLP ? W.block[0] : 0);
    };
    auto fields = [&](int l, int half, int k) -> SavedPtrs {  // micro-batch k's saved tensors
      const HalfBlock& B = HB[half];
      char* b = block(l, half);
      SavedPtrs f;
      f.ln_out = b + B.ln_out + (size_t)k * B.sz.ln_out;
      f.mean = reinterpret_cast<float*>(b + B.mean + (size_t)k * B.sz.stats);
      f.rstd = reinterpret_cast<float*>(b + B.rstd + (size_t)k * B.sz.stats);
      f.a = b + B.a + (size_t)k * B.sz.a;
      f.b = b + B.b + (size_t)k * B.sz.b;
      f.c = half == MTNLG_ATTN ? reinterpret_cast<float*>(b + B.c + (size_t)k * B.sz.c) : nullptr;
      return f;
    };
    // the half's output gradient as its weight gradients use it (after the
    // dropout backward); without dropout it is the residual-path gradient
    // itself, which the previous half's partial sum writes there directly
    // (the top layer's MLP half: the caller's dy)
    auto dy_kept = [&](int l, int half) -> char* {
      if (!drop && l == nl - 1 && half == MTNLG_MLP) return static_cast<char*>(const_cast<void*>(dy));
      return block(l, half) + HB[half].dy;
    };
    char* wgws = base + W.wg;
    for (int k = 0; k < mb; ++k) {
      for (int l = 0; l < nl; ++l) {
        int64_t o[2][kTensors];
        layer_offsets(d, l, o);
        const void* in[2] = {xin(l, k), mid(l)};
        void* out[2] = {mid(l), xout(l, k)};
        const mtnlg_layer_desc Lk = layer_of(k, l);
        for (int half = 0; half < 2; ++half) {
          const int64_t* t = o[half];
          const mtnlg_half_params p = {wb + 2 * t[0], wb + 2 * t[1], wb + 2 * t[2], wb + 2 * t[3], wb + 2 * t[4]};
          STAGE_CALL(half_fwd(&Lk, half, &p, in[half], part, fields(l, half, k), lws, S));
          const void* parts[1] = {part};
          if (drop) {
            const mtnlg_dropout dr = {desc->dropout_seed, site(k, l, half), desc->dropout_p};
            STAGE_CALL(mtnlg_reduce_partials_dropout(d.T, d.h, MTNLG_BF16, parts, 1, in[half], wb + 2 * t[5], &dr,
                                                     out[half], stream));
          } else {
            STAGE_CALL(mtnlg_reduce_partials(d.T, d.h, MTNLG_BF16, parts, 1, in[half], wb + 2 * t[5], out[half],
                                             stream));
          }
        }
      }
      const void* gcur = static_cast<const char*>(dy) + (size_t)k * act;
      for (int l = nl - 1; l >= 0; --l) {
        int64_t o[2][kTensors];
        layer_offsets(d, l, o);
        const void* in[2] = {xin(l, k), mid(l)};
        const mtnlg_layer_desc Lk = layer_of(k, l);
        for (int half = 1; half >= 0; --half) {
          const int64_t* t = o[half];
          const mtnlg_half_params p = {wb + 2 * t[0], wb + 2 * t[1], wb + 2 * t[2], wb + 2 * t[3], wb + 2 * t[4]};
          const void* dyh = gcur;
          if (drop) {
            const mtnlg_dropout dr = {desc->dropout_seed, site(k, l, half), desc->dropout_p};
            void* dz = dy_kept(l, half) + (size_t)k * act;
            STAGE_CALL(mtnlg_dropout_bwd(d.T, d.h, MTNLG_BF16, gcur, &dr, dz, stream));
            dyh = dz;
          }
          const HalfBlock& B = HB[half];
          STAGE_CALL(half_bwd_data(&Lk, half, &p, in[half], fields(l, half, k), dyh, part,
                                   block(l, half) + B.g + (size_t)k * B.sz.g,
                                   reinterpret_cast<float*>(block(l, half) + B.lnp + (size_t)k * B.sz.lnp), lws, S));
          // dx of the half = dy (residual path) + the slice's partial, written
          // where the next half keeps its output gradient
          void* dst;
          if (half == MTNLG_MLP)
            dst = drop ? g1 : dy_kept(l, MTNLG_ATTN) + (size_t)k * act;
          else if (l == 0)
            dst = static_cast<char*>(dx) + (size_t)k * act;
          else
            dst = drop ? g2 : dy_kept(l - 1, MTNLG_MLP) + (size_t)k * act;
          const void* parts[1] = {part};
          STAGE_CALL(mtnlg_reduce_partials(d.T, d.h, MTNLG_BF16, parts, 1, gcur, nullptr, dst, stream));
          gcur = dst;
        }
        if (k == mb - 1) {
          // layer l's every micro-batch is through its backward: its weight,
          // bias and LayerNorm gradients, each over mb * T rows
          for (int half = 1; half >= 0; --half) {
            const int64_t* t = o[half];
            const mtnlg_half_grads g = {gb + 2 * t[0], gb + 2 * t[1], gb + 2 * t[2],
                                        gb + 2 * t[3], gb + 2 * t[4], gb + 2 * t[5]};
            const HalfBlock& B = HB[half];
            STAGE_CALL(half_weight_grads(L, half, mb, fields(l, half, 0), dy_kept(l, half), block(l, half) + B.g,
                                         reinterpret_cast<const float*>(block(l, half) + B.lnp), &g, wgws, S));
          }
        }
      }
    }
    // grad holds the whole step's gradient: the norm pass and the update read
    // it as it is (acc is left untouched; an fp32 copy would only add 6 bytes
    // per parameter of traffic for the same values)
    MTNLG_HIP(grad_norm_bf16(n, grad, cfg->inv_loss_scale, base + W.adam, S), "grad_norm_bf16");
    MTNLG_HIP(adam_update_bf16(sc, n, master, m, v, grad, w, stats, base + W.adam, S), "adam_update_bf16");
    return MTNLG_OK;
  }

  for (int k = 0; k < desc->micro_batches; ++k) {
    for (int l = 0; l < desc->layers; ++l) {
      int64_t o[2][kTensors];
      layer_offsets(d, l, o);
      const void* in[2] = {xin(l, k), mid(l)};
      void* out[2] = {mid(l), xout(l, k)};
      const mtnlg_layer_desc Lk = layer_of(k, l);
      for (int half = 0; half < 2; ++half) {
        const int64_t* t = o[half];
        const mtnlg_half_params p = {wb + 2 * t[0], wb + 2 * t[1], wb + 2 * t[2], wb + 2 * t[3], wb + 2 * t[4]};
        STAGE_CALL(mtnlg_layer_fwd(&Lk, half, &p, in[half], part, saved(l, half), lws, lws_bytes, stream));
        const void* parts[1] = {part};
        if (drop) {
          const mtnlg_dropout dr = {desc->dropout_seed, site(k, l, half), desc->dropout_p};
          STAGE_CALL(mtnlg_reduce_partials_dropout(d.T, d.h, MTNLG_BF16, parts, 1, in[half], wb + 2 * t[5], &dr,
                                                   out[half], stream));
        } else {
          STAGE_CALL(mtnlg_reduce_partials(d.T, d.h, MTNLG_BF16, parts, 1, in[half], wb + 2 * t[5], out[half],
                                           stream));
        }
      }
    }
    const void* gcur = static_cast<const char*>(dy) + (size_t)k * act;
    for (int l = desc->layers - 1; l >= 0; --l) {
      int64_t o[2][kTensors];
      layer_offsets(d, l, o);
      // layer l's gradient buffer is rewritten below: the previous micro-batch's
      // accumulation of it must be done
      if (overlap && k > 0) MTNLG_HIP(hipStreamWaitEvent(S, acc_done[l], 0), "hipStreamWaitEvent");
      const void* in[2] = {xin(l, k), mid(l)};
      const mtnlg_layer_desc Lk = layer_of(k, l);
      for (int half = 1; half >= 0; --half) {
        const int64_t* t = o[half];
        const mtnlg_half_params p = {wb + 2 * t[0], wb + 2 * t[1], wb + 2 * t[2], wb + 2 * t[3], wb + 2 * t[4]};
        const mtnlg_half_grads g = {gb + 2 * t[0], gb + 2 * t[1], gb + 2 * t[2],
                                    gb + 2 * t[3], gb + 2 * t[4], gb + 2 * t[5]};
        // the half's output gradient: gcur, or its dropout-masked copy
        const void* dyh = gcur;
        if (drop) {
          const mtnlg_dropout dr = {desc->dropout_seed, site(k, l, half), desc->dropout_p};
          STAGE_CALL(mtnlg_dropout_bwd(d.T, d.h, MTNLG_BF16, gcur, &dr, base + W.dz, stream));
          dyh = base + W.dz;
        }
        if (desc->recompute)
          STAGE_CALL(mtnlg_layer_bwd_recompute(&Lk, half, &p, in[half], dyh, part, &g, lws, lws_bytes, stream));
        else
          STAGE_CALL(mtnlg_layer_bwd(&Lk, half, &p, in[half], saved(l, half), dyh, part, &g, lws, lws_bytes,
                                     stream));
        // dx of the half = dy (residual path) + the slice's partial
        void* dst = half == MTNLG_MLP ? g1 : (l == 0 ? static_cast<char*>(dx) + (size_t)k * act : g2);
        const void* parts[1] = {part};
        STAGE_CALL(mtnlg_reduce_partials(d.T, d.h, MTNLG_BF16, parts, 1, gcur, nullptr, dst, stream));
        gcur = dst;
      }
      if (overlap && k + 1 < mb) {
        const int64_t lo = (int64_t)l * d.per_layer;
        MTNLG_HIP(hipEventRecord(bwd_done[l], S), "hipEventRecord");
        MTNLG_HIP(hipStreamWaitEvent(A, bwd_done[l], 0), "hipStreamWaitEvent");
        STAGE_CALL(mtnlg_grad_accumulate(d.per_layer, MTNLG_BF16, gb + 2 * lo, acc + lo, k == 0, A));
        MTNLG_HIP(hipEventRecord(acc_done[l], A), "hipEventRecord");
      }
    }
    const bool first = k == 0;
    if (k + 1 < mb) {
      if (!overlap) STAGE_CALL(mtnlg_grad_accumulate(n, MTNLG_BF16, grad, acc, first, stream));
    } else {
      // every earlier accumulation is ordered before this one: S waited for each
      // layer's before rewriting that layer's gradient
      STAGE_CALL(mtnlg_grad_accumulate_norm(n, MTNLG_BF16, grad, acc, first, cfg->inv_loss_scale, base + W.adam,
                                            W.xin - W.adam, stream));
    }
  }
  return mtnlg_adam_update(cfg, n, master, m, v, acc, w, stats, base + W.adam, W.xin - W.adam, stream);
}

}  // extern "C"
