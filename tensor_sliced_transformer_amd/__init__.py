"""MI355X (gfx950) library for one GPU's tensor slice of an MT-NLG decoder layer.

Python binding over the C ABI of ``include/mtnlg.h`` (libmtnlg.so). Every
function here only marshals arguments: device pointers of torch tensors (torch
is used for device memory and streams) and the current HIP stream are handed to
the library, whose hand-written HIP kernels do all the arithmetic. A missing
library raises on first use; nothing falls back to PyTorch or the CPU.

Tensors: bf16 path -> torch.bfloat16, fp32 path -> torch.float32, all on the
GPU, contiguous, 16-byte aligned (any fresh torch allocation is).
"""
from __future__ import annotations

import ctypes
from . import _lib
from ._lib import ATTN, MLP, BF16, F32, AdamCfg, HalfGrads, HalfParams, LayerDesc, MtnlgError, StageDesc, check, load

__all__ = ["ATTN", "MLP", "BF16", "F32", "LayerDesc", "AdamCfg", "MtnlgError", "load", "make_desc",
           "saved_bytes", "workspace_bytes", "layer_fwd", "layer_bwd", "reduce_partials",
           "grad_accumulate", "adam_workspace_bytes", "adam_step", "adam_static_scratch_bytes", "adam_step_noalloc",
           "grad_accumulate_norm", "adam_update", "adam_stream_reference",
           "reduce_partials_dropout", "dropout_bwd",
           "recompute_workspace_bytes", "layer_bwd_recompute", "StageDesc", "make_stage_desc",
           "stage_param_count", "stage_param_offsets", "stage_workspace_bytes", "stage_step", "gemm", "gemm_workspace_bytes", "layernorm_fwd",
           "layernorm_bwd_workspace_bytes", "layernorm_bwd", "attention_fwd",
           "attention_bwd_workspace_bytes", "attention_bwd", "torch_dtype"]


def _torch():
    import torch
    return torch


def torch_dtype(dtype: int):
    t = _torch()
    return t.bfloat16 if dtype == BF16 else t.float32


def _code(tensor) -> int:
    t = _torch()
    if tensor.dtype == t.bfloat16:
        return BF16
    if tensor.dtype == t.float32:
        return F32
    raise TypeError(f"unsupported tensor dtype {tensor.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    t = _torch()
    s = stream if stream is not None else t.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(batch, seq, hidden, heads, ffn, tp_size=1, tp_rank=0, dtype=BF16, ln_eps=1e-5,
              attn_dropout=0.0, attn_dropout_seed=0, attn_dropout_site=0) -> LayerDesc:
    """mtnlg_layer_desc; attn_dropout > 0 drops attention probabilities (BF16)."""
    return LayerDesc(batch, seq, hidden, heads, ffn, tp_size, tp_rank, dtype, ln_eps, attn_dropout,
                     attn_dropout_seed, attn_dropout_site)


def saved_bytes(desc: LayerDesc, half: int) -> int:
    return int(load().mtnlg_saved_bytes(ctypes.byref(desc), half))


def workspace_bytes(desc: LayerDesc, half: int) -> int:
    return int(load().mtnlg_workspace_bytes(ctypes.byref(desc), half))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _expect(name, t, shape, dtype) -> None:
    """Size checks on the host side of the boundary: the C ABI takes bare
    pointers, so a tensor smaller than the descriptor implies would be written
    past its end on the device."""
    if t is None:
        raise ValueError(f"{name} is None")
    if tuple(t.shape) != tuple(shape) and t.numel() != _prod(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _prod(shape) -> int:
    n = 1
    for s in shape:
        n *= int(s)
    return n


def _half_shapes(desc: LayerDesc, half: int) -> dict:
    h = desc.hidden
    if half == ATTN:
        w = desc.heads // desc.tp_size * (desc.hidden // desc.heads)
        win, wout = 3 * w, w
    else:
        win = wout = desc.ffn // desc.tp_size
    return {"ln_g": (h,), "ln_b": (h,), "w_in": (h, win), "b_in": (win,), "w_out": (wout, h), "b_out": (h,)}


def _check_half(desc, half, params=None, grads=None, acts=(), saved=None, ws=None, ws_need=None):
    dt = torch_dtype(desc.dtype)
    shapes = _half_shapes(desc, half)
    if params is not None:
        for k in ("ln_g", "ln_b", "w_in", "b_in", "w_out"):
            _expect(f"params[{k}]", params[k], shapes[k], dt)
    if grads is not None:
        for k, s in shapes.items():
            _expect(f"grads[{k}]", grads[k], s, dt)
    tok = (desc.batch * desc.seq, desc.hidden)
    for name, t in acts:
        _expect(name, t, tok, dt)
    if saved is not None and _nbytes(saved) < saved_bytes(desc, half):
        raise ValueError(f"saved: {_nbytes(saved)} bytes < {saved_bytes(desc, half)} required")
    if ws_need is not None and (0 if ws is None else _nbytes(ws)) < ws_need:
        raise ValueError(f"ws: {0 if ws is None else _nbytes(ws)} bytes < {ws_need} required")


def _params(p: dict) -> HalfParams:
    return HalfParams(*(_ptr(p[k]) for k in ("ln_g", "ln_b", "w_in", "b_in", "w_out")))


def _grads(g: dict) -> HalfGrads:
    return HalfGrads(*(_ptr(g[k]) for k in ("ln_g", "ln_b", "w_in", "b_in", "w_out", "b_out")))


def layer_fwd(desc, half, params: dict, x, y_partial, saved, ws=None, stream=None) -> None:
    """One slice's half forward (mtnlg_layer_fwd); params keys ln_g ln_b w_in b_in w_out."""
    _check_half(desc, half, params=params, acts=(("x", x), ("y_partial", y_partial)), saved=saved)
    p = _params(params)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().mtnlg_layer_fwd(ctypes.byref(desc), half, ctypes.byref(p), _ptr(x), _ptr(y_partial),
                                 _ptr(saved), _ptr(ws), ws_bytes, _stream(stream)), "mtnlg_layer_fwd")


def layer_bwd(desc, half, params: dict, x, saved, dy, dx_partial, grads: dict, ws, stream=None) -> None:
    """One slice's half backward (mtnlg_layer_bwd); grads keys ln_g ln_b w_in b_in w_out b_out."""
    _check_half(desc, half, params=params, grads=grads, acts=(("x", x), ("dy", dy), ("dx_partial", dx_partial)),
                saved=saved)
    p = _params(params)
    g = _grads(grads)
    check(load().mtnlg_layer_bwd(ctypes.byref(desc), half, ctypes.byref(p), _ptr(x), _ptr(saved), _ptr(dy),
                                 _ptr(dx_partial), ctypes.byref(g), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "mtnlg_layer_bwd")


def recompute_workspace_bytes(desc: LayerDesc, half: int) -> int:
    return int(load().mtnlg_recompute_workspace_bytes(ctypes.byref(desc), half))


def layer_bwd_recompute(desc, half, params: dict, x, dy, dx_partial, grads: dict, ws, stream=None) -> None:
    """One slice's half backward that first recomputes its saved activations from x
    (mtnlg_layer_bwd_recompute); ws of recompute_workspace_bytes(desc, half) bytes."""
    _check_half(desc, half, params=params, grads=grads, acts=(("x", x), ("dy", dy), ("dx_partial", dx_partial)))
    p = _params(params)
    g = _grads(grads)
    check(load().mtnlg_layer_bwd_recompute(ctypes.byref(desc), half, ctypes.byref(p), _ptr(x), _ptr(dy),
                                           _ptr(dx_partial), ctypes.byref(g), _ptr(ws),
                                           ws.numel() * ws.element_size(), _stream(stream)),
          "mtnlg_layer_bwd_recompute")


def _check_reduce(partials, out, residual, bias) -> None:
    rows, cols = out.shape
    for j, t in enumerate(partials):
        _expect(f"partials[{j}]", t, (rows, cols), out.dtype)
    if residual is not None:
        _expect("residual", residual, (rows, cols), out.dtype)
    if bias is not None:
        _expect("bias", bias, (cols,), out.dtype)


def reduce_partials(partials, out, residual=None, bias=None, stream=None) -> None:
    """out = residual + bias + sum(partials) (mtnlg_reduce_partials)."""
    rows, cols = out.shape
    _check_reduce(partials, out, residual, bias)
    arr = (ctypes.c_void_p * len(partials))(*[p.data_ptr() for p in partials])
    for p in partials:
        _ptr(p)
    check(load().mtnlg_reduce_partials(rows, cols, _code(out), arr, len(partials), _ptr(residual), _ptr(bias),
                                       _ptr(out), _stream(stream)), "mtnlg_reduce_partials")


def reduce_partials_dropout(partials, out, p: float, seed: int, site: int, residual=None, bias=None,
                            stream=None) -> None:
    """out = residual + keep * scale * (sum(partials) + bias) (mtnlg_reduce_partials_dropout)."""
    rows, cols = out.shape
    _check_reduce(partials, out, residual, bias)
    arr = (ctypes.c_void_p * len(partials))(*[t.data_ptr() for t in partials])
    for t in partials:
        _ptr(t)
    d = _lib.Dropout(seed, site, p)
    check(load().mtnlg_reduce_partials_dropout(rows, cols, _code(out), arr, len(partials), _ptr(residual),
                                               _ptr(bias), ctypes.byref(d), _ptr(out), _stream(stream)),
          "mtnlg_reduce_partials_dropout")


def dropout_bwd(dy, dz, p: float, seed: int, site: int, stream=None) -> None:
    """dz = keep * scale * dy with the mask of the same (p, seed, site) (mtnlg_dropout_bwd)."""
    rows, cols = dy.shape
    d = _lib.Dropout(seed, site, p)
    check(load().mtnlg_dropout_bwd(rows, cols, _code(dy), _ptr(dy), ctypes.byref(d), _ptr(dz), _stream(stream)),
          "mtnlg_dropout_bwd")


def grad_accumulate(grad, acc, overwrite: bool, stream=None) -> None:
    check(load().mtnlg_grad_accumulate(grad.numel(), _code(grad), _ptr(grad), _ptr(acc), int(overwrite),
                                       _stream(stream)), "mtnlg_grad_accumulate")


def adam_workspace_bytes(n: int) -> int:
    return int(load().mtnlg_adam_workspace_bytes(n))


def adam_step(cfg: AdamCfg, master, m, v, grad, w_bf16, stats, ws, stream=None) -> None:
    check(load().mtnlg_adam_step(ctypes.byref(cfg), master.numel(), _ptr(master), _ptr(m), _ptr(v), _ptr(grad),
                                 _ptr(w_bf16), _ptr(stats), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "mtnlg_adam_step")


def adam_static_scratch_bytes() -> int:
    return int(load().mtnlg_adam_static_scratch_bytes())


def adam_step_noalloc(cfg: AdamCfg, master, m, v, grad, w_bf16, stats, stream=None) -> None:
    """adam_step with its scratch in the library's static per-GPU buffer
    (mtnlg_adam_step_noalloc): allocates nothing; overlapping calls on one GPU race."""
    check(load().mtnlg_adam_step_noalloc(ctypes.byref(cfg), master.numel(), _ptr(master), _ptr(m), _ptr(v),
                                         _ptr(grad), _ptr(w_bf16), _ptr(stats), _stream(stream)),
          "mtnlg_adam_step_noalloc")


def grad_accumulate_norm(grad, acc, overwrite: bool, inv_loss_scale: float, ws, stream=None) -> None:
    """acc (+)= grad and, in the same pass, the norm partials of acc * inv_loss_scale
    left in ws for adam_update (mtnlg_grad_accumulate_norm)."""
    check(load().mtnlg_grad_accumulate_norm(acc.numel(), _code(grad), _ptr(grad), _ptr(acc), int(overwrite),
                                            float(inv_loss_scale), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)), "mtnlg_grad_accumulate_norm")


def adam_update(cfg: AdamCfg, master, m, v, grad, w_bf16, stats, ws, stream=None) -> None:
    """The Adam step on the norm partials grad_accumulate_norm left in ws (mtnlg_adam_update)."""
    check(load().mtnlg_adam_update(ctypes.byref(cfg), master.numel(), _ptr(master), _ptr(m), _ptr(v), _ptr(grad),
                                   _ptr(w_bf16), _ptr(stats), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "mtnlg_adam_update")


def adam_stream_reference(master, m, v, grad, w_bf16=None, stream=None) -> None:
    """The Adam update's reads and writes with no optimizer arithmetic (master, m,
    v rewritten unchanged, w_bf16 = bf16(master)): a measurement reference for the
    update's rate (mtnlg_adam_stream_reference)."""
    torch = _torch()
    n = master.numel()
    for name, t in (("master", master), ("m", m), ("v", v), ("grad", grad)):
        _expect(name, t, (n,), torch.float32)
    if w_bf16 is not None:
        _expect("w_bf16", w_bf16, (n,), torch.bfloat16)
    check(load().mtnlg_adam_stream_reference(n, _ptr(master), _ptr(m), _ptr(v), _ptr(grad),
                                             _ptr(w_bf16) if w_bf16 is not None else None, _stream(stream)),
          "mtnlg_adam_stream_reference")


STAGE_TENSORS = ("ln_g", "ln_b", "w_in", "b_in", "w_out", "b_out")


def make_stage_desc(layer: LayerDesc, layers: int, micro_batches: int, recompute: bool = False,
                    dropout_p: float = 0.0, dropout_seed: int = 0, per_micro_batch_grads: bool = False) -> StageDesc:
    return StageDesc(layer, layers, micro_batches, int(recompute), dropout_p, dropout_seed,
                     int(per_micro_batch_grads))


def stage_param_count(sd: StageDesc) -> int:
    n = int(load().mtnlg_stage_param_count(ctypes.byref(sd)))
    if n < 0:
        raise MtnlgError("invalid stage descriptor")
    return n


def stage_param_offsets(sd: StageDesc) -> list:
    """[layer][half] -> {tensor name: element offset} in the flat parameter array."""
    off = (ctypes.c_int64 * (sd.layers * 2 * 6))()
    check(load().mtnlg_stage_param_offsets(ctypes.byref(sd), off), "mtnlg_stage_param_offsets")
    return [[{k: int(off[(l * 2 + h) * 6 + i]) for i, k in enumerate(STAGE_TENSORS)} for h in range(2)]
            for l in range(sd.layers)]


def stage_workspace_bytes(sd: StageDesc) -> int:
    return int(load().mtnlg_stage_workspace_bytes(ctypes.byref(sd)))


def stage_step(sd: StageDesc, cfg: AdamCfg, w, master, m, v, grad, acc, x, dy, y, dx, stats, ws,
               stream=None, aux_stream=None) -> None:
    """One training step of a pipeline stage (mtnlg_stage_step); aux_stream, a second
    torch stream, lets the gradient accumulation overlap the compute."""
    aux = ctypes.c_void_p(aux_stream.cuda_stream) if aux_stream is not None else None
    check(load().mtnlg_stage_step(ctypes.byref(sd), ctypes.byref(cfg), _ptr(w), _ptr(master), _ptr(m), _ptr(v),
                                  _ptr(grad), _ptr(acc), _ptr(x), _ptr(dy), _ptr(y), _ptr(dx), _ptr(stats),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream), aux),
          "mtnlg_stage_step")


def gemm_workspace_bytes(dtype: int, M: int, N: int, K: int) -> int:
    return int(load().mtnlg_gemm_workspace_bytes(dtype, M, N, K))


def gemm(a, b, c, trans_a=False, trans_b=False, bias=None, ws=None, stream=None) -> None:
    """c = op(a) op(b) (+ bias) (mtnlg_gemm). ws: a uint8 tensor of at least
    gemm_workspace_bytes(...) bytes, or None when that is 0."""
    M, N = c.shape
    K = a.shape[0] if trans_a else a.shape[1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().mtnlg_gemm(_code(c), int(trans_a), int(trans_b), M, N, K, _ptr(a), _ptr(b), _ptr(c), _ptr(bias),
                            _ptr(ws), ws_bytes, _stream(stream)), "mtnlg_gemm")


def layernorm_fwd(x, gamma, beta, eps, y, mean, rstd, stream=None) -> None:
    rows, cols = x.shape
    check(load().mtnlg_layernorm_fwd(_code(x), rows, cols, _ptr(x), _ptr(gamma), _ptr(beta), eps, _ptr(y),
                                     _ptr(mean), _ptr(rstd), _stream(stream)), "mtnlg_layernorm_fwd")


def layernorm_bwd_workspace_bytes(rows: int, cols: int) -> int:
    return int(load().mtnlg_layernorm_bwd_workspace_bytes(rows, cols))


def layernorm_bwd(gy, x, mean, rstd, gamma, dx, dgamma, dbeta, ws, stream=None) -> None:
    rows, cols = x.shape
    check(load().mtnlg_layernorm_bwd(_code(x), rows, cols, _ptr(gy), _ptr(x), _ptr(mean), _ptr(rstd), _ptr(gamma),
                                     _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "mtnlg_layernorm_bwd")


def attention_fwd(qkv, o, lse, batch, seq, heads, head_dim, stream=None) -> None:
    check(load().mtnlg_attention_fwd(_code(qkv), batch, seq, heads, head_dim, _ptr(qkv), _ptr(o), _ptr(lse),
                                     _stream(stream)), "mtnlg_attention_fwd")


def attention_bwd_workspace_bytes(batch, seq, heads) -> int:
    return int(load().mtnlg_attention_bwd_workspace_bytes(batch, seq, heads))


def attention_bwd(qkv, o, lse, do, dqkv, ws, batch, seq, heads, head_dim, stream=None) -> None:
    check(load().mtnlg_attention_bwd(_code(qkv), batch, seq, heads, head_dim, _ptr(qkv), _ptr(o), _ptr(lse),
                                     _ptr(do), _ptr(dqkv), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "mtnlg_attention_bwd")
