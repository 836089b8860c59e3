"""ctypes declarations of the C ABI in include/mtnlg.h.

Loading fails loudly (RuntimeError) when libmtnlg.so has not been built: there
is no fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p, c_char_p, POINTER

HERE = os.path.dirname(os.path.abspath(__file__))
# MTNLG_LIBRARY may name another build of the same sources (the host-sanitizer
# build that the host ABI tests run against); the default is the in-tree build.
LIB_PATH = os.environ.get("MTNLG_LIBRARY") or os.path.join(HERE, "libmtnlg.so")

MTNLG_OK = 0
STATUS = {0: "MTNLG_OK", -1: "MTNLG_ERR_ARG", -2: "MTNLG_ERR_SHAPE", -3: "MTNLG_ERR_DTYPE",
          -4: "MTNLG_ERR_ALIGN", -5: "MTNLG_ERR_WORKSPACE", -6: "MTNLG_ERR_HIP",
          -7: "MTNLG_ERR_UNIMPLEMENTED"}
F32, BF16 = 0, 1
ATTN, MLP = 0, 1


class LayerDesc(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("seq", c_int32), ("hidden", c_int32), ("heads", c_int32),
                ("ffn", c_int32), ("tp_size", c_int32), ("tp_rank", c_int32), ("dtype", c_int32),
                ("ln_eps", c_float), ("attn_dropout", c_float), ("attn_dropout_seed", ctypes.c_uint64),
                ("attn_dropout_site", ctypes.c_uint64)]


class StageDesc(ctypes.Structure):
    _fields_ = [("layer", LayerDesc), ("layers", c_int32), ("micro_batches", c_int32), ("recompute", c_int32),
                ("dropout_p", c_float), ("dropout_seed", ctypes.c_uint64), ("per_micro_batch_grads", c_int32)]


class Dropout(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("site", ctypes.c_uint64), ("p", c_float)]


class HalfParams(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("ln_g", "ln_b", "w_in", "b_in", "w_out")]


class HalfGrads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("ln_g", "ln_b", "w_in", "b_in", "w_out", "b_out")]


class AdamCfg(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("max_grad_norm", c_float), ("inv_loss_scale", c_float),
                ("step", c_int64)]


# name -> (restype, argtypes)
SIGNATURES = {
    "mtnlg_saved_bytes": (c_size_t, [POINTER(LayerDesc), c_int32]),
    "mtnlg_workspace_bytes": (c_size_t, [POINTER(LayerDesc), c_int32]),
    "mtnlg_layer_fwd": (c_int32, [POINTER(LayerDesc), c_int32, POINTER(HalfParams), c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_size_t, c_void_p]),
    "mtnlg_layer_bwd": (c_int32, [POINTER(LayerDesc), c_int32, POINTER(HalfParams), c_void_p, c_void_p,
                                  c_void_p, c_void_p, POINTER(HalfGrads), c_void_p, c_size_t, c_void_p]),
    "mtnlg_recompute_workspace_bytes": (c_size_t, [POINTER(LayerDesc), c_int32]),
    "mtnlg_layer_bwd_recompute": (c_int32, [POINTER(LayerDesc), c_int32, POINTER(HalfParams), c_void_p, c_void_p,
                                            c_void_p, POINTER(HalfGrads), c_void_p, c_size_t, c_void_p]),
    "mtnlg_reduce_partials": (c_int32, [c_int64, c_int64, c_int32, POINTER(c_void_p), c_int32, c_void_p,
                                        c_void_p, c_void_p, c_void_p]),
    "mtnlg_reduce_partials_dropout": (c_int32, [c_int64, c_int64, c_int32, POINTER(c_void_p), c_int32, c_void_p,
                                                c_void_p, POINTER(Dropout), c_void_p, c_void_p]),
    "mtnlg_dropout_bwd": (c_int32, [c_int64, c_int64, c_int32, c_void_p, POINTER(Dropout), c_void_p, c_void_p]),
    "mtnlg_grad_accumulate": (c_int32, [c_int64, c_int32, c_void_p, c_void_p, c_int32, c_void_p]),
    "mtnlg_adam_workspace_bytes": (c_size_t, [c_int64]),
    "mtnlg_adam_step": (c_int32, [POINTER(AdamCfg), c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mtnlg_adam_static_scratch_bytes": (c_size_t, []),
    "mtnlg_adam_step_noalloc": (c_int32, [POINTER(AdamCfg), c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_void_p]),
    "mtnlg_grad_accumulate_norm": (c_int32, [c_int64, c_int32, c_void_p, c_void_p, c_int32, c_float, c_void_p,
                                             c_size_t, c_void_p]),
    "mtnlg_adam_update": (c_int32, [POINTER(AdamCfg), c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mtnlg_adam_stream_reference": (c_int32, [c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p]),
    "mtnlg_stage_param_count": (c_int64, [POINTER(StageDesc)]),
    "mtnlg_stage_param_offsets": (c_int32, [POINTER(StageDesc), POINTER(c_int64)]),
    "mtnlg_stage_workspace_bytes": (c_size_t, [POINTER(StageDesc)]),
    "mtnlg_stage_step": (c_int32, [POINTER(StageDesc), POINTER(AdamCfg), c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p, c_void_p]),
    "mtnlg_gemm_workspace_bytes": (c_size_t, [c_int32, c_int64, c_int64, c_int64]),
    "mtnlg_gemm": (c_int32, [c_int32, c_int32, c_int32, c_int64, c_int64, c_int64, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mtnlg_layernorm_fwd": (c_int32, [c_int32, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_float,
                                      c_void_p, c_void_p, c_void_p, c_void_p]),
    "mtnlg_layernorm_bwd_workspace_bytes": (c_size_t, [c_int64, c_int64]),
    "mtnlg_layernorm_bwd": (c_int32, [c_int32, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mtnlg_attention_fwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                      c_void_p, c_void_p]),
    "mtnlg_attention_bwd_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "mtnlg_attention_bwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mtnlg_status_str": (c_char_p, [c_int32]),
    "mtnlg_last_error": (c_char_p, []),
}

_LIB = None


def load() -> ctypes.CDLL:
    """The loaded library (declared once). Raises RuntimeError if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m tensor_sliced_transformer_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


class MtnlgError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


def check(status: int, where: str) -> None:
    if status != MTNLG_OK:
        lib = load()
        detail = lib.mtnlg_last_error().decode(errors="replace")
        raise MtnlgError(status, where, detail)
