/*
 * mtnlg.h -- C ABI of the MI355X (gfx950) library for one GPU's tensor slice of
 * an MT-NLG decoder layer and its mixed-precision Adam step.
 *
 * What is computed (sources are web pages about MT-NLG 530B; cited by title
 * and section):
 *   - A dense left-to-right transformer decoder layer ("Using DeepSpeed and
 *     Megatron to Train Megatron-Turing NLG 530B", Elamur summary page,
 *     Summary; jiqizhixin MT-NLG article, model paragraph: 105 layers,
 *     hidden 20480, 128 heads).
 *   - Tensor slicing as in the Megatron example of the STRONGHOLD slide deck
 *     (slides 7-8): the first MLP weight A is split by columns, so slice i
 *     computes Y_i = GeLU(X A_i) alone; the second weight B is split by rows,
 *     so slice i produces Z_i = Y_i B_i and the layer output needs the sum of
 *     the Z_i (operator g: all-reduce forward, identity backward; operator f:
 *     identity forward, all-reduce backward). Attention is split the same way
 *     by whole heads: QKV by columns, the output projection by rows.
 *   - Mixed-precision Adam at about 20 bytes per parameter, with gradients of
 *     micro-batches accumulated before the step (Elamur summary, Key points).
 *
 * Readings where the pages are silent (same as the CPU oracle): pre-LN block,
 * LayerNorm eps given in the descriptor (1e-5 by default) with biased
 * variance, exact-erf GeLU, every linear has a bias, row-sliced biases are
 * added once after the sum, dropout 0, attention scale 1/sqrt(head_dim),
 * causal mask inside each sequence, QKV columns ordered (q/k/v, local head,
 * dim).
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers into memory the caller
 *     allocated (the library never allocates or frees on these paths and keeps
 *     no mutable global state). Descriptor / config structs and the array of
 *     partial pointers in mtnlg_reduce_partials are HOST memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; nothing synchronises the host.
 *   - Layout is row-major. Activations are [batch*seq, width] with rows
 *     ordered (sequence, position). Weights are in math form [in, out], so a
 *     linear is Y = X W (+ b).
 *   - Element type is given by mtnlg_dtype: F32 = IEEE binary32, BF16 =
 *     bfloat16 bit patterns (uint16). bf16 paths accumulate in fp32 and round
 *     results to nearest even.
 *   - Inputs and outputs must not alias. Every device pointer must be 16-byte
 *     aligned.
 *   - Errors: arguments are validated on the host BEFORE anything is
 *     enqueued; a negative mtnlg_status is returned and nothing is launched.
 *     A failed launch returns MTNLG_ERR_HIP. mtnlg_last_error() gives a
 *     thread-local text for the last failure. Numerical events (a non-finite
 *     gradient) are data, not errors.
 */
#ifndef MTNLG_H
#define MTNLG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTNLG_OK = 0,
  MTNLG_ERR_ARG = -1,          /* null pointer or out-of-range scalar          */
  MTNLG_ERR_SHAPE = -2,        /* dimensions inconsistent or unsupported        */
  MTNLG_ERR_DTYPE = -3,        /* unsupported element type                      */
  MTNLG_ERR_ALIGN = -4,        /* a device pointer is not 16-byte aligned       */
  MTNLG_ERR_WORKSPACE = -5,    /* workspace smaller than the size query returns */
  MTNLG_ERR_HIP = -6,          /* a HIP launch or runtime call failed           */
  MTNLG_ERR_UNIMPLEMENTED = -7
} mtnlg_status;

typedef enum { MTNLG_F32 = 0, MTNLG_BF16 = 1 } mtnlg_dtype;

/* The two halves of a layer, each ending in a row-sliced linear whose partial
 * output feeds an all-reduce (g). */
typedef enum { MTNLG_ATTN = 0, MTNLG_MLP = 1 } mtnlg_half;

/* Full-layer dimensions plus the slicing factor t (tp_size) and the index of
 * the slice this call computes (tp_rank). The slice sees heads/tp_size heads
 * of width hidden/heads and ffn/tp_size MLP columns.
 * Supported: hidden % heads == 0; heads % tp_size == 0; ffn % tp_size == 0;
 * 0 <= tp_rank < tp_size; head_dim in {64, 128, 160} (bf16) or {64, 128}
 * (f32); hidden and ffn/tp_size multiples of 16; hidden <= 32768; seq a
 * multiple of 128; one sequence of the slice's QKV activations
 * (seq * 3 * hidden/tp_size elements) below 2 GiB; every GEMM operand of the
 * slice below 2 GiB in bytes of dtype (batch*seq tokens x the widest of
 * hidden, 3*hidden/tp_size and ffn/tp_size; hidden x the wider of
 * 3*hidden/tp_size and ffn/tp_size), the range of the GEMM's 32-bit buffer
 * offsets (bf16 at hidden 20480: at most 52428 tokens); dtype F32 or BF16;
 * ln_eps > 0 and finite. Violations return MTNLG_ERR_SHAPE, MTNLG_ERR_DTYPE
 * or MTNLG_ERR_ARG before any launch.
 *
 * Dropout on the attention probabilities (ATTN half; the MLP half ignores
 * these fields): attn_dropout = rate p, 0 <= p < 1 (0: none; p must round to
 * a threshold below 65536 as for mtnlg_reduce_partials_dropout), BF16 only
 * (MTNLG_ERR_UNIMPLEMENTED for F32 with p > 0). The softmax normaliser is
 * taken before dropout: O = (P * keep * scale) V with scale = 65536 /
 * (65536 - thr), thr = round(p * 65536). Element (b, head, q, k) -- b the
 * sequence, head the GLOBAL head index tp_rank * heads/tp_size + local head,
 * q and k positions in the sequence -- is kept when the 16-bit draw at bits
 * 16 * (k % 4) of word q % 4 of Philox4x64-10 at counter (q/4, k/4, head, b)
 * under key (attn_dropout_seed, attn_dropout_site) is >= thr. This reading
 * is the library's: the pages name dropout only on the row-sliced output
 * (STRONGHOLD slide deck, slide 8). layer_bwd (and the recompute variant)
 * regenerate the same mask from the same fields, so the forward and backward
 * of one micro-batch must pass equal values; callers vary the site per layer
 * and micro-batch. */
typedef struct {
  int32_t batch, seq, hidden, heads, ffn;
  int32_t tp_size, tp_rank;
  int32_t dtype;       /* mtnlg_dtype */
  float ln_eps;
  float attn_dropout;          /* rate on the attention probabilities (0: none) */
  uint64_t attn_dropout_seed;  /* generator key, first word */
  uint64_t attn_dropout_site;  /* generator key, second word */
} mtnlg_layer_desc;

/* Parameters of one slice of one half, all in desc->dtype:
 *   ATTN: ln_g, ln_b = gamma1, beta1 [hidden] (replicated);
 *         w_in = W_qkv,i [hidden, 3*w] (columns (q/k/v, local head, dim));
 *         b_in = b_qkv,i [3*w]; w_out = W_o,i [w, hidden]; w = local heads*head_dim
 *   MLP:  ln_g, ln_b = gamma2, beta2 [hidden]; w_in = A_i [hidden, f];
 *         b_in = a_i [f]; w_out = B_i [f, hidden]; f = ffn/tp_size
 * The row-sliced output bias (b_o or b_B) is not here: it is added once, by
 * the reduction of the partials. */
typedef struct { const void *ln_g, *ln_b, *w_in, *b_in, *w_out; } mtnlg_half_params;

/* Gradients of one slice of one half, same shapes and dtype as the
 * parameters; OVERWRITTEN (not accumulated). ln_g and ln_b are this slice's
 * partial sums (the replicated gamma/beta gradient is their sum over slices);
 * b_out [hidden] is the gradient of the row-sliced output bias = column sums
 * of dy, identical on every slice. */
typedef struct { void *ln_g, *ln_b, *w_in, *b_in, *w_out, *b_out; } mtnlg_half_grads;

/* Size in bytes of the `saved` buffer that layer_fwd fills and layer_bwd
 * reads for this descriptor and half; 0 if the descriptor is invalid.
 * Layout (each region starts on a 256-byte boundary, in this order):
 *   ATTN: ln_out [T, hidden] dtype | mean [T] f32 | rstd [T] f32 |
 *         qkv [T, 3w] (F32: f32; BF16: the Q and K columns [0, 2w) as IEEE
 *         binary16, the V columns as bf16) | o [T, w] dtype |
 *         lse [local heads, T] f32
 *   MLP:  ln_out [T, hidden] dtype | mean [T] f32 | rstd [T] f32 |
 *         u [T, f] dtype (pre-activation) | y [T, f] dtype (GeLU(u))
 * with T = batch*seq. lse is the natural log of the softmax normaliser of
 * each query row (scores already scaled by 1/sqrt(head_dim)). */
size_t mtnlg_saved_bytes(const mtnlg_layer_desc* desc, int32_t half);

/* Size in bytes of the scratch workspace layer_fwd / layer_bwd need for
 * this descriptor and half (one size serves both); 0 if invalid. */
size_t mtnlg_workspace_bytes(const mtnlg_layer_desc* desc, int32_t half);

/* Forward of one slice of one half. Defined by the Megatron example of the
 * STRONGHOLD slide deck (slides 7-8): the half's first linear is split by
 * columns (QKV by whole heads, MLP-up A by columns, Y_i = GeLU(X A_i)), its
 * second by rows (W_o, MLP-down B: Z_i = Y_i B_i), so one slice runs
 * LayerNorm, its column slice, attention over its heads or GeLU, and its row
 * slice, whose output is the partial that operator g sums; the left-to-right
 * decoder (Elamur summary, Summary) makes the attention causal.
 *   x          [T, hidden] dtype: the half's input (X for ATTN, X1 for MLP)
 *   y_partial  [T, hidden] dtype: this slice's row-parallel output WITHOUT
 *              bias or residual -- ATTN: Attn_i(LN1(x)) W_o,i;
 *              MLP: GeLU(LN2(x) A_i + a_i) B_i. The caller's reduction adds
 *              residual + bias + the sum over slices once (on a real
 *              multi-GPU run this is the g all-reduce).
 *   saved      mtnlg_saved_bytes(desc, half) bytes, written here.
 *   ws         mtnlg_workspace_bytes(desc, half) bytes of scratch. */
int mtnlg_layer_fwd(const mtnlg_layer_desc* desc, int32_t half, const mtnlg_half_params* params,
                    const void* x, void* y_partial, void* saved, void* ws, size_t ws_bytes,
                    void* stream);

/* Backward of one slice of one half for L = <output, dy>. The conjugate
 * operators of the STRONGHOLD slide deck (slides 7-8) fix what each slice
 * receives and returns: g's backward is the identity, so every slice gets the
 * same dy; f's backward is an all-reduce, so each slice returns its own
 * input-gradient partial. The gradients are those of the forward above.
 *   x          the same input that was passed to layer_fwd (unchanged)
 *   saved      what layer_fwd wrote for the same x and params
 *   dy         [T, hidden] dtype: gradient of the half's output (g's
 *              backward is the identity, so every slice gets the same dy)
 *   dx_partial [T, hidden] dtype: this slice's contribution to dL/dx through
 *              LayerNorm. The caller forms dx = dy + sum of the partials
 *              (f's backward all-reduce); LayerNorm backward is linear in its
 *              upstream gradient, so applying it per slice is exact.
 *   grads      overwritten, see mtnlg_half_grads. */
int mtnlg_layer_bwd(const mtnlg_layer_desc* desc, int32_t half, const mtnlg_half_params* params,
                    const void* x, const void* saved, const void* dy, void* dx_partial,
                    const mtnlg_half_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* Backward of one half with activation recomputation: the caller keeps only
 * the half's input x (no `saved` buffer between forward and backward). The
 * call first recomputes, into its workspace, everything mtnlg_layer_fwd saves
 * (LayerNorm, the QKV or MLP-up product and, for ATTN, the attention output
 * and lse; the row-sliced output product is not needed and is skipped), then
 * runs exactly the mtnlg_layer_bwd of that half. All kernels are
 * deterministic, so dx_partial and the grads are bit-identical to those of
 * mtnlg_layer_fwd + mtnlg_layer_bwd on the same inputs. This trades one more
 * forward for the activation memory that the MT-NLG paper summary (Key
 * points) budgets per micro-batch.
 * ws: at least mtnlg_recompute_workspace_bytes(desc, half) bytes, owned by
 * the caller; its first part holds the recomputed saved tensors, the rest is
 * the backward's scratch. Argument meaning, layouts, overwrite semantics and
 * errors are those of mtnlg_layer_bwd (MTNLG_ERR_WORKSPACE if ws is too small). */
size_t mtnlg_recompute_workspace_bytes(const mtnlg_layer_desc* desc, int32_t half);
int mtnlg_layer_bwd_recompute(const mtnlg_layer_desc* desc, int32_t half, const mtnlg_half_params* params,
                              const void* x, const void* dy, void* dx_partial, const mtnlg_half_grads* grads,
                              void* ws, size_t ws_bytes, void* stream);

/* out = residual + bias + sum_{j<n} partials[j], summed in fp32 and rounded
 * once (the g all-reduce, or f's backward, done locally on one device). The
 * sum of the row slices' partials is the layer output in the STRONGHOLD
 * slide deck's Megatron example (slides 7-8: Z = sum_i Y_i B_i); the
 * residual and the row-sliced bias are added here, once.
 *   partials   HOST array of n DEVICE pointers, each [rows, cols] dtype; 1 <= n <= 16
 *   residual   [rows, cols] dtype, nullable (treated as zero)
 *   bias       [cols] dtype, nullable
 *   out        [rows, cols] dtype; must not alias the inputs.
 * cols must be a multiple of 8. */
int mtnlg_reduce_partials(int64_t rows, int64_t cols, int32_t dtype, const void* const* partials,
                          int32_t n, const void* residual, const void* bias, void* out,
                          void* stream);

/* Dropout at the end of a half (STRONGHOLD slides, slide 8: the row-sliced
 * linear's output goes through dropout, Z = Dropout(Y B), i.e. after operator
 * g has summed the slices; the attention half is treated the same way). The
 * keep mask is drawn from Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) so that the
 * backward regenerates it instead of storing it: element e of the row-major
 * [rows, cols] tensor takes 16 bits of the generator's block at counter
 * (e / 16, 0, 0, 0) under key (seed, site) -- bits 16 * (e % 4) of word
 * (e % 16) / 4 -- and is kept when those bits, as an integer, are
 * >= thr = nearbyint((double)p * 65536) (ties to even); kept values are
 * scaled by 65536 / (65536 - thr). `site` distinguishes the dropout sites of
 * one step (layer, half, micro-batch). 0 <= p < 1 (p = 0 keeps everything);
 * otherwise MTNLG_ERR_ARG. */
typedef struct {
  uint64_t seed, site;
  float p;
} mtnlg_dropout;

/* out = residual + keep * scale * (sum_{j<n} partials[j] + bias): the partial
 * sum of mtnlg_reduce_partials with dropout applied to the half's output
 * before the residual. Arguments, layouts and errors as mtnlg_reduce_partials. */
int mtnlg_reduce_partials_dropout(int64_t rows, int64_t cols, int32_t dtype, const void* const* partials,
                                  int32_t n, const void* residual, const void* bias,
                                  const mtnlg_dropout* dropout, void* out, void* stream);

/* The backward of that dropout: dz = keep * scale * dy with the same mask
 * (same rows, cols and dropout struct). dz is the dy the half's backward
 * (mtnlg_layer_bwd) takes; the residual path keeps dy itself.
 *   dy, dz [rows, cols] dtype, must not alias. cols a positive multiple of 8. */
int mtnlg_dropout_bwd(int64_t rows, int64_t cols, int32_t dtype, const void* dy,
                      const mtnlg_dropout* dropout, void* dz, void* stream);

/* Gradient accumulation over micro-batches (Elamur summary, Key points):
 * acc[i] = (overwrite ? 0 : acc[i]) + grad[i] for i < n, in fp32.
 *   grad  [n] dtype (BF16 for the mixed-precision path, F32 allowed)
 *   acc   [n] f32.  n >= 0 (0 is a no-op). */
int mtnlg_grad_accumulate(int64_t n, int32_t dtype, const void* grad, float* acc,
                          int32_t overwrite, void* stream);

/* Adam hyper-parameters of one step. step is the 1-based index of the step
 * being taken (bias corrections use beta^step). max_grad_norm <= 0 turns
 * clipping off. inv_loss_scale multiplies the accumulated gradient first. */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay, max_grad_norm, inv_loss_scale;
  int64_t step;
} mtnlg_adam_cfg;

/* Scratch bytes mtnlg_adam_step needs for n parameters. */
size_t mtnlg_adam_workspace_bytes(int64_t n);

/* Fused mixed-precision Adam step over one GPU's flat share of n params, the
 * fp32 master weights and two fp32 moments of the mixed-precision Adam that
 * the Elamur summary (Key points) counts at about 20 bytes per parameter,
 * with Adam as in its References (Kingma and Ba):
 *   g_hat = grad * inv_loss_scale; norm = ||g_hat||_2 over all n;
 *   found_inf = any non-finite g_hat; coef = max_norm / (norm + 1e-6) if
 *   that is below 1, else 1. If found_inf, NOTHING is written except
 *   stats. Otherwise with g = g_hat * coef: p *= (1 - lr*wd) when wd > 0;
 *   m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
 *   p -= lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps);
 *   w_bf16 = bf16 round-to-nearest-even of p.
 *   master, m, v [n] f32 (updated in place); grad [n] f32 (the accumulator);
 *   w_bf16 [n] bf16, nullable (skipped); stats DEVICE f32[3] written with
 *   {norm, coef, found_inf (0 or 1)}; ws >= mtnlg_adam_workspace_bytes(n).
 * The whole decision (norm, clip, skip) stays on the device: no host sync. */
int mtnlg_adam_step(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v,
                    const float* grad, void* w_bf16, float* stats, void* ws, size_t ws_bytes,
                    void* stream);

/* mtnlg_adam_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and result, bit for bit, with no workspace argument. The
 * norm pass's per-workgroup partials go to the library's own static scratch
 * of mtnlg_adam_static_scratch_bytes() bytes (96 KiB: one fp64 partial and
 * one flag for each of at most 8192 norm workgroups; every n fits, as the
 * norm pass never launches more), one copy per GPU, held until the process
 * ends. Its device address is looked up once per device, on the first call
 * with that device current. Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (on different streams, or from different
 * threads) race and give wrong results; calls on one stream are ordered.
 * Nothing in the scratch needs to start at zero (every partial the finish
 * reads is written first by the same call). The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine). Arguments,
 * semantics and errors as mtnlg_adam_step without ws and ws_bytes. */
size_t mtnlg_adam_static_scratch_bytes(void);
int mtnlg_adam_step_noalloc(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v,
                            const float* grad, void* w_bf16, float* stats, void* stream);

/* The optimizer's norm pass folded into the last micro-batch's accumulation
 * (Elamur summary, Key points: micro-batch gradient accumulation; the norm and
 * clip are this library's reading): one pass does
 *   acc[i] = (overwrite ? 0 : acc[i]) + grad[i]   (as mtnlg_grad_accumulate)
 * and leaves in ws, per workgroup, the fp64 sum of (acc[i]*inv_loss_scale)^2
 * and a non-finite flag. mtnlg_adam_update then takes the step without
 * reading acc a second time for the norm (4 bytes per parameter less).
 *   grad [n] dtype, acc [n] f32 (may be NULL only when n == 0);
 *   ws >= mtnlg_adam_workspace_bytes(n), device memory the caller owns; its
 *   contents are consumed by the next mtnlg_adam_update on the same stream.
 * n >= 0 (n == 0 writes an empty norm). Errors as mtnlg_grad_accumulate,
 * plus MTNLG_ERR_WORKSPACE and MTNLG_ERR_ARG for a non-finite inv_loss_scale. */
int mtnlg_grad_accumulate_norm(int64_t n, int32_t dtype, const void* grad, float* acc,
                               int32_t overwrite, float inv_loss_scale, void* ws,
                               size_t ws_bytes, void* stream);

/* mtnlg_adam_step without its own norm pass: the norm, clip coefficient and
 * found_inf come from the partials that mtnlg_grad_accumulate_norm left in
 * ws. Same arguments, semantics and errors as mtnlg_adam_step, with three
 * conditions the caller keeps: grad is that call's acc, n is that call's n,
 * and cfg->inv_loss_scale equals that call's inv_loss_scale (the update
 * scales by it; the norm was formed with it). ws is only read. */
int mtnlg_adam_update(const mtnlg_adam_cfg* cfg, int64_t n, float* master, float* m, float* v,
                      const float* grad, void* w_bf16, float* stats, const void* ws,
                      size_t ws_bytes, void* stream);

/* Measurement reference for the optimizer step (not part of training): the
 * memory traffic of mtnlg_adam_update's element pass -- master, m, v and grad
 * read, master, m, v and (if w_bf16 is not NULL) the bf16 copy written, 30
 * bytes per parameter as the mixed-precision Adam state of the Elamur summary
 * (Key points) is laid out here -- with the same launch and access order but
 * no optimizer arithmetic: master, m and v are written back unchanged and
 * w_bf16 receives bf16(master). Its rate is the memory system's rate for that
 * access mix, the ceiling of the update.
 *   master, m, v [n] f32 (rewritten with their own values), grad [n] f32
 *   (read only), w_bf16 [n] bf16 or NULL; device memory, 16-byte aligned.
 * n >= 0 (n == 0 does nothing). MTNLG_ERR_SHAPE for n < 0, MTNLG_ERR_ARG for a
 * NULL pointer, MTNLG_ERR_ALIGN, MTNLG_ERR_HIP. */
int mtnlg_adam_stream_reference(int64_t n, float* master, float* m, float* v, const float* grad,
                                void* w_bf16, void* stream);

/* ---- One pipeline stage on one GPU ----
 *
 * A stage is `layers` consecutive decoder layers, each held as the same slice
 * (desc.layer.tp_rank of desc.layer.tp_size) -- in MT-NLG 530B, 105 layers in
 * 35 pipeline stages of 3 (jiqizhixin MT-NLG article, system paragraph) --
 * trained on `micro_batches` micro-batches whose gradients are accumulated
 * before one optimizer step (Elamur summary, Key points). On one GPU the
 * all-reduces that join the slices (operators f and g) are the identity:
 * each layer's partial is summed alone, with its residual and output bias,
 * by mtnlg_reduce_partials; on a real tensor-sliced run this is where the
 * all-reduce would be. Only BF16 layers (mixed precision) are supported. */
typedef struct {
  mtnlg_layer_desc layer;  /* shape and slice of every layer; batch sequences per micro-batch */
  int32_t layers;          /* >= 1 */
  int32_t micro_batches;   /* >= 1 */
  int32_t recompute;       /* 0: keep each layer's saved tensors from forward to backward;
                              1: keep only each half's input and recompute in the backward */
  float dropout_p;         /* dropout on each half's output, 0 <= p < 1 (0: none), as
                              mtnlg_reduce_partials_dropout */
  uint64_t dropout_seed;   /* the generator key's first word; the site of micro-batch k,
                              layer l, half h is (k * layers + l) * 2 + h */
  int32_t per_micro_batch_grads; /* with recompute = 0: 0 computes every layer's weight and
                              bias gradients once, over all micro-batches' tokens, after the
                              last micro-batch's backward of that layer (the saved tensors
                              and output gradients of every micro-batch are kept); 1
                              computes them per micro-batch and accumulates as with
                              recompute = 1. Ignored (per micro-batch) when recompute = 1,
                              and when a batched operand (micro_batches * T rows of the
                              widest activation) would reach 2 GiB. */
} mtnlg_stage_desc;
/* layer.attn_dropout > 0 also drops attention probabilities: micro-batch k,
 * layer l keys its mask with (layer.attn_dropout_seed,
 * layer.attn_dropout_site + k * layers + l), in its forward and its backward. */

/* The stage's parameters live in ONE flat element array (the bf16 weights,
 * the bf16 gradients and the fp32 master, m, v and accumulator all share this
 * layout), layer after layer, each layer as ATTN then MLP, each half as
 *   ln_g [h] | ln_b [h] | w_in [h, win] | b_in [win] | w_out [win, h] | b_out [h]
 * with win = 3 * local heads * head_dim (ATTN) or ffn / tp_size (MLP), shapes
 * and meaning as in mtnlg_half_params / mtnlg_half_grads (b_out is b_o or
 * b_B). Every tensor starts on a multiple of 8 elements.
 * mtnlg_stage_param_count: total elements, or -1 if the descriptor is invalid.
 * mtnlg_stage_param_offsets: writes layers*2*6 element offsets (HOST array
 * `off`, order layer, half, tensor as listed); MTNLG_ERR_* if invalid. */
int64_t mtnlg_stage_param_count(const mtnlg_stage_desc* desc);
int mtnlg_stage_param_offsets(const mtnlg_stage_desc* desc, int64_t* off);

/* Scratch bytes of mtnlg_stage_step; 0 if the descriptor is invalid. */
size_t mtnlg_stage_workspace_bytes(const mtnlg_stage_desc* desc);

/* One training step of the stage: for each micro-batch k in order, the
 * forward through every layer, then the backward in reverse order (with
 * dropout_p > 0 each half's output goes through mtnlg_reduce_partials_dropout
 * and its backward starts from mtnlg_dropout_bwd of the same site).
 * Per-micro-batch gradients (recompute = 1 or per_micro_batch_grads = 1):
 * each micro-batch's flat gradient is accumulated into acc (overwritten by
 * k = 0, added for k > 0; the last accumulation carries the norm pass, see
 * mtnlg_grad_accumulate_norm). Batched gradients (the default with
 * recompute = 0): the backward of every micro-batch computes only the input
 * gradients, keeping each half's output gradient, its dU or dQKV and its
 * LayerNorm partial sums; after the last micro-batch's backward of a layer,
 * that layer's weight gradients are single products over micro_batches * T
 * rows (fp32 accumulation inside the product, one bf16 rounding into grad)
 * and its bias and LayerNorm gradients single column sums; the norm pass
 * and the update then read grad as it is (no fp32 copy: 6 bytes per
 * parameter less traffic, and the same result bit for bit as overwriting acc
 * with grad through mtnlg_grad_accumulate_norm and updating from acc).
 * Either way the update is mtnlg_adam_update's, with cfg.
 *   w       [n] bf16 flat weights; read by every layer and rewritten by the
 *           step as bf16(master)
 *   master, m, v  [n] f32 optimizer state (updated in place)
 *   grad    [n] bf16 scratch: one micro-batch's gradient (batched: the sum over
 *           all micro-batches)
 *   acc     [n] f32: per-micro-batch gradients: the accumulated gradient (left
 *           holding it); batched gradients: not used (left untouched)
 *   x       [micro_batches, T, h] bf16: stage input (T = batch * seq)
 *   dy      [micro_batches, T, h] bf16: gradient of the stage output
 *   y       [micro_batches, T, h] bf16: stage output, written
 *   dx      [micro_batches, T, h] bf16: gradient of the stage input, written
 *   stats   DEVICE f32[3]: {norm, coef, found_inf} of the step
 *   ws      >= mtnlg_stage_workspace_bytes(desc)
 *   aux_stream  nullable second hipStream_t. When given (and different from
 *           stream), the per-micro-batch gradient of each layer of every
 *           micro-batch but the last is accumulated on it as soon as that
 *           layer's backward is done, overlapping the accumulation with the
 *           rest of the work (batched gradients leave it unused); ordering
 *           between the two streams uses 2 * layers events that the library
 *           creates on first use and keeps, per calling thread and device,
 *           until the process ends (a later call on the same thread records
 *           them again; a stream wait refers to the record
 *           made before it, so reuse does not change the ordering). Results are
 *           identical with and without it. All of the step's work is
 *           complete once `stream` has passed it.
 * n = mtnlg_stage_param_count(desc). All arguments are validated before
 * anything is enqueued; errors as the calls it makes (MTNLG_ERR_HIP also
 * when an event cannot be created). */
int mtnlg_stage_step(const mtnlg_stage_desc* desc, const mtnlg_adam_cfg* cfg, void* w, float* master,
                     float* m, float* v, void* grad, float* acc, const void* x, const void* dy, void* y,
                     void* dx, float* stats, void* ws, size_t ws_bytes, void* stream,
                     void* aux_stream);

/* ---- Component entry points (the kernels the layer calls, one at a time) ---- */

/* C[M,N] = op(A) op(B) (+ bias[n]) in dtype, fp32 accumulation -- the GEMM
 * every linear of the layer runs on.
 *   trans_a = 0: A is [M, K] row-major; 1: A is stored [K, M] (op(A) = A^T).
 *   trans_b = 0: B is [K, N] row-major; 1: B is stored [N, K] (op(B) = B^T).
 *   bias nullable. M, N, K multiples of 8; each operand (A, B and C) below
 *   2 GiB in bytes of dtype, else MTNLG_ERR_SHAPE (operands are addressed
 *   through 32-bit buffer offsets).
 *   ws: mtnlg_gemm_workspace_bytes(...) bytes (fp32 partials of the tiles
 *   that are split along K to fill the last round of workgroups); may be NULL
 *   when that size is 0. */
size_t mtnlg_gemm_workspace_bytes(int32_t dtype, int64_t M, int64_t N, int64_t K);
int mtnlg_gemm(int32_t dtype, int32_t trans_a, int32_t trans_b, int64_t M, int64_t N, int64_t K,
               const void* A, const void* B, void* C, const void* bias, void* ws, size_t ws_bytes,
               void* stream);

/* Row LayerNorm of x [rows, cols] (the oracle's layernorm_fwd):
 * y = gamma*(x-mean)*rstd + beta; mean, rstd [rows] f32. cols multiple of 8. */
int mtnlg_layernorm_fwd(int32_t dtype, int64_t rows, int64_t cols, const void* x,
                        const void* gamma, const void* beta, float eps, void* y, float* mean,
                        float* rstd, void* stream);

/* LayerNorm backward for upstream gradient gy (the oracle's layernorm_bwd):
 * dx [rows, cols] dtype, dgamma / dbeta [cols] dtype. gy is dtype.
 * ws >= mtnlg_layernorm_bwd_workspace_bytes(rows, cols). */
size_t mtnlg_layernorm_bwd_workspace_bytes(int64_t rows, int64_t cols);
int mtnlg_layernorm_bwd(int32_t dtype, int64_t rows, int64_t cols, const void* gy, const void* x,
                        const float* mean, const float* rstd, const void* gamma, void* dx,
                        void* dgamma, void* dbeta, void* ws, size_t ws_bytes, void* stream);

/* Causal attention of `heads` heads of width head_dim over batch sequences
 * of length seq, reading qkv [batch*seq, 3*heads*head_dim] (columns
 * (q/k/v, head, dim)) and writing o [batch*seq, heads*head_dim] (columns
 * (head, dim)) and lse [heads, batch*seq] f32 (natural log of each query's
 * softmax normaliser). Scores are scaled by 1/sqrt(head_dim); query r sees
 * keys 0..r of its own sequence (the left-to-right decoder of the MT-NLG
 * paper summary, Summary, and of the STRONGHOLD slides, slide 8).
 * Requires seq % 128 == 0, head_dim in {64, 128, 160} (bf16) or {64, 128}
 * (f32), and seq*3*heads*head_dim elements below 2 GiB.
 * BF16: the Q and K columns of qkv hold IEEE binary16 values (the V columns
 * bf16), as the layer's QKV product stores them: with scores of standard
 * deviation near 8 (the MT-NLG slice at its initialisation) the softmax
 * magnifies the rounding of Q and K, and binary16 carries three more
 * fraction bits; |Q|, |K| must stay below 65504, binary16's largest finite
 * value. S = Q K^T runs on the fp16 matrix cores; o, do_ and dqkv are bf16. */
int mtnlg_attention_fwd(int32_t dtype, int32_t batch, int32_t seq, int32_t heads,
                        int32_t head_dim, const void* qkv, void* o, float* lse, void* stream);

/* Backward of mtnlg_attention_fwd: dqkv [batch*seq, 3*heads*head_dim] from
 * qkv, o, lse and do_ [batch*seq, heads*head_dim]. Every element of dqkv is
 * written (no accumulation); the result is deterministic.
 * ws >= mtnlg_attention_bwd_workspace_bytes(...) (two floats per token and
 * head: lse*log2(e) and rowsum(dO*O)). */
size_t mtnlg_attention_bwd_workspace_bytes(int32_t batch, int32_t seq, int32_t heads);
int mtnlg_attention_bwd(int32_t dtype, int32_t batch, int32_t seq, int32_t heads,
                        int32_t head_dim, const void* qkv, const void* o, const float* lse,
                        const void* do_, void* dqkv, void* ws, size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* mtnlg_status_str(int32_t status);
/* Thread-local text describing the last failure on this thread ("" if none). */
const char* mtnlg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MTNLG_H */
