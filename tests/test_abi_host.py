"""Host-side checks of the C ABI that need no GPU: the built library loads, it
exports every function include/mtnlg.h declares, size queries follow the
documented layouts, and invalid arguments are rejected before any launch.

Only validation paths are called here (they return before touching HIP); no
test passes a fake pointer to a path that would launch a kernel.
"""
import ctypes
import os
import re

import pytest

from tensor_sliced_transformer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtnlg.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libmtnlg.so not built (python -m tensor_sliced_transformer_amd.build)")

A = 1 << 20          # a fake, 16-byte aligned, non-null address (never dereferenced)
ODD = A + 4          # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtnlg_[a-z_0-9]+)\s*\(", text)))


def lib():
    return _lib.load()


def desc(**kw):
    d = dict(batch=1, seq=2048, hidden=20480, heads=128, ffn=81920, tp_size=8, tp_rank=0, dtype=_lib.BF16,
             ln_eps=1e-5)
    d.update(kw)
    return _lib.LayerDesc(**d)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 17
    missing = [n for n in names if not hasattr(lib(), n)]
    assert not missing, missing
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings():
    L = lib()
    for code in _lib.STATUS:
        assert L.mtnlg_status_str(code)
    assert L.mtnlg_status_str(12345) == b"unknown status"


def align256(x):
    return (x + 255) & ~255


def test_saved_bytes_mtnlg_shard():
    """ATTN: ln_out | mean | rstd | qkv | o | lse; MLP: ln_out | mean | rstd | u | y (256-byte aligned)."""
    L = lib()
    T, h, w, f, nh = 2048, 20480, 2560, 10240, 16
    d = desc()
    attn = 0
    for nbytes in (T * h * 2, T * 4, T * 4, T * 3 * w * 2, T * w * 2, nh * T * 4):
        attn = align256(attn + nbytes)
    mlp = 0
    for nbytes in (T * h * 2, T * 4, T * 4, T * f * 2, T * f * 2):
        mlp = align256(mlp + nbytes)
    assert L.mtnlg_saved_bytes(ctypes.byref(d), _lib.ATTN) == attn
    assert L.mtnlg_saved_bytes(ctypes.byref(d), _lib.MLP) == mlp
    assert L.mtnlg_workspace_bytes(ctypes.byref(d), _lib.ATTN) > T * h * 2
    assert L.mtnlg_workspace_bytes(ctypes.byref(d), _lib.MLP) > T * h * 2


@pytest.mark.parametrize("bad,status", [
    (dict(dtype=7), -3),
    (dict(tp_rank=8), -1),
    (dict(tp_rank=-1), -1),
    (dict(heads=100), -2),           # hidden % heads
    (dict(heads=128, tp_size=3), -2),
    (dict(hidden=20480, heads=80), -2),   # head_dim 256 unsupported
    (dict(seq=100), -2),
    (dict(ln_eps=0.0), -1),
    (dict(batch=0), -2),
    (dict(batch=26), -2),            # 53248 tokens x hidden 20480 x 2 B >= 2 GiB (32-bit GEMM offsets)
    (dict(dtype=_lib.F32, hidden=16384, heads=128, ffn=65536, batch=16), -2),   # 32768 x 16384 x 4 B = 2 GiB
])
def test_invalid_descriptor_rejected(bad, status):
    L = lib()
    d = desc(**bad)
    assert L.mtnlg_saved_bytes(ctypes.byref(d), _lib.ATTN) == 0
    p = _lib.HalfParams(A, A, A, A, A)
    st = L.mtnlg_layer_fwd(ctypes.byref(d), _lib.ATTN, ctypes.byref(p), A, A, A, None, 0, None)
    assert st == status, L.mtnlg_last_error()
    assert L.mtnlg_last_error()


def test_largest_layer_accepted():
    """25 sequences of 2048 at hidden 20480 keep every GEMM operand of the slice below 2 GiB."""
    L = lib()
    d = desc(batch=25)
    assert L.mtnlg_saved_bytes(ctypes.byref(d), _lib.ATTN) > 0
    assert L.mtnlg_saved_bytes(ctypes.byref(d), _lib.MLP) > 0


def test_gemm_operands_of_2_gib_rejected():
    """The GEMM addresses operands through 32-bit buffer offsets: an operand of
    2 GiB or more (counted in bytes of its dtype) is a shape error."""
    L = lib()
    assert L.mtnlg_gemm(_lib.F32, 0, 0, 65536, 256, 8192, A, A, A, None, None, 0, None) == -2    # A: 2 GiB fp32
    assert L.mtnlg_gemm(_lib.BF16, 0, 0, 65536, 256, 16384, A, A, A, None, None, 0, None) == -2  # A: 2 GiB bf16
    assert L.mtnlg_gemm(_lib.BF16, 0, 1, 256, 65536, 16384, A, A, A, None, None, 0, None) == -2  # B: 2 GiB
    assert L.mtnlg_gemm(_lib.F32, 0, 0, 32768, 16384, 64, A, A, A, None, None, 0, None) == -2    # C: 2 GiB fp32
    assert b"2 GiB" in L.mtnlg_last_error()


def test_null_and_misaligned_pointers():
    L = lib()
    d = desc()
    p = _lib.HalfParams(A, A, None, A, A)
    assert L.mtnlg_layer_fwd(ctypes.byref(d), _lib.MLP, ctypes.byref(p), A, A, A, None, 0, None) == -1
    assert b"w_in" in L.mtnlg_last_error()
    p = _lib.HalfParams(A, A, ODD, A, A)
    assert L.mtnlg_layer_fwd(ctypes.byref(d), _lib.MLP, ctypes.byref(p), A, A, A, None, 0, None) == -4
    assert L.mtnlg_layer_fwd(None, _lib.MLP, ctypes.byref(p), A, A, A, None, 0, None) == -1
    assert L.mtnlg_layer_fwd(ctypes.byref(d), 2, ctypes.byref(p), A, A, A, None, 0, None) == -1


def test_small_workspace_rejected():
    L = lib()
    d = desc()
    p = _lib.HalfParams(A, A, A, A, A)
    g = _lib.HalfGrads(A, A, A, A, A, A)
    need = L.mtnlg_workspace_bytes(ctypes.byref(d), _lib.ATTN)
    st = L.mtnlg_layer_bwd(ctypes.byref(d), _lib.ATTN, ctypes.byref(p), A, A, A, A, ctypes.byref(g), A,
                           need - 1, None)
    assert st == -5
    g2 = _lib.HalfGrads(A, A, A, None, A, A)
    st = L.mtnlg_layer_bwd(ctypes.byref(d), _lib.ATTN, ctypes.byref(p), A, A, A, A, ctypes.byref(g2), A,
                           need, None)
    assert st == -1


def test_recompute_workspace_and_validation():
    """The recompute backward's workspace is the saved tensors (256-aligned) plus the
    ordinary backward workspace; it validates like mtnlg_layer_bwd."""
    L = lib()
    d = desc()
    p = _lib.HalfParams(A, A, A, A, A)
    g = _lib.HalfGrads(A, A, A, A, A, A)
    for half in (_lib.ATTN, _lib.MLP):
        need = L.mtnlg_recompute_workspace_bytes(ctypes.byref(d), half)
        assert need == align256(L.mtnlg_saved_bytes(ctypes.byref(d), half)) + \
            L.mtnlg_workspace_bytes(ctypes.byref(d), half)
        st = L.mtnlg_layer_bwd_recompute(ctypes.byref(d), half, ctypes.byref(p), A, A, A, ctypes.byref(g), A,
                                         need - 1, None)
        assert st == -5
        st = L.mtnlg_layer_bwd_recompute(ctypes.byref(d), half, ctypes.byref(p), None, A, A, ctypes.byref(g), A,
                                         need, None)
        assert st == -1
    assert L.mtnlg_recompute_workspace_bytes(ctypes.byref(desc(seq=100)), _lib.ATTN) == 0


def test_dropout_entry_points_validate():
    L = lib()
    arr = (ctypes.c_void_p * 1)(A)
    for p in (-0.1, 1.0, float("nan"), 0.99999999):
        d = _lib.Dropout(1, 2, p)
        assert L.mtnlg_reduce_partials_dropout(4, 16, _lib.BF16, arr, 1, None, None, ctypes.byref(d), A, None) == -1
        assert L.mtnlg_dropout_bwd(4, 16, _lib.BF16, A, ctypes.byref(d), A, None) == -1
    d = _lib.Dropout(1, 2, 0.5)
    assert L.mtnlg_reduce_partials_dropout(4, 12, _lib.BF16, arr, 1, None, None, ctypes.byref(d), A, None) == -2
    assert L.mtnlg_reduce_partials_dropout(4, 16, 9, arr, 1, None, None, ctypes.byref(d), A, None) == -3
    assert L.mtnlg_reduce_partials_dropout(4, 16, _lib.BF16, arr, 1, None, None, None, A, None) == -1
    assert L.mtnlg_dropout_bwd(4, 16, _lib.BF16, ODD, ctypes.byref(d), A, None) == -4
    assert L.mtnlg_dropout_bwd(4, 16, _lib.BF16, A, ctypes.byref(d), None, None) == -1


def test_other_entry_points_validate():
    L = lib()
    arr = (ctypes.c_void_p * 2)(A, A)
    assert L.mtnlg_reduce_partials(4, 12, _lib.BF16, arr, 2, None, None, A, None) == -2      # cols % 8
    assert L.mtnlg_reduce_partials(4, 16, _lib.BF16, arr, 0, None, None, A, None) == -1      # n
    assert L.mtnlg_reduce_partials(4, 16, _lib.BF16, arr, 17, None, None, A, None) == -1
    assert L.mtnlg_reduce_partials(4, 16, 5, arr, 2, None, None, A, None) == -3
    assert L.mtnlg_grad_accumulate(-1, _lib.BF16, A, A, 1, None) == -2
    assert L.mtnlg_grad_accumulate(0, _lib.BF16, None, None, 1, None) == 0                   # empty: no-op
    assert L.mtnlg_grad_accumulate(16, _lib.BF16, ODD, A, 1, None) == -4
    cfg = _lib.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 0)
    assert L.mtnlg_adam_step(ctypes.byref(cfg), 16, A, A, A, A, None, A, A, 1 << 20, None) == -1   # step 0
    cfg = _lib.AdamCfg(1e-4, 1.0, 0.95, 1e-8, 0.0, 1.0, 1.0, 1)
    assert L.mtnlg_adam_step(ctypes.byref(cfg), 16, A, A, A, A, None, A, A, 1 << 20, None) == -1   # beta1
    cfg = _lib.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 1)
    assert L.mtnlg_adam_step(ctypes.byref(cfg), 16, A, A, A, A, None, A, A, 8, None) == -5
    assert L.mtnlg_adam_update(ctypes.byref(cfg), 16, A, A, A, A, None, A, A, 8, None) == -5
    assert L.mtnlg_grad_accumulate_norm(16, _lib.BF16, A, A, 1, 1.0, A, 8, None) == -5
    assert L.mtnlg_grad_accumulate_norm(16, _lib.BF16, A, A, 1, float("inf"), A, 1 << 20, None) == -1
    assert L.mtnlg_grad_accumulate_norm(16, _lib.BF16, None, A, 1, 1.0, A, 1 << 20, None) == -1
    assert L.mtnlg_grad_accumulate_norm(16, 7, A, A, 1, 1.0, A, 1 << 20, None) == -3
    assert L.mtnlg_adam_stream_reference(-1, A, A, A, A, None, None) == -2
    assert L.mtnlg_adam_stream_reference(0, None, None, None, None, None, None) == 0      # empty: no-op
    assert L.mtnlg_adam_stream_reference(16, A, None, A, A, None, None) == -1
    assert L.mtnlg_adam_stream_reference(16, A, A, A, ODD, None, None) == -4
    assert L.mtnlg_adam_stream_reference(16, A, A, A, A, ODD, None) == -4
    assert L.mtnlg_gemm(_lib.BF16, 0, 0, 12, 16, 16, A, A, A, None, None, 0, None) == -2
    assert L.mtnlg_gemm(_lib.BF16, 0, 0, 16, 16, 16, None, A, A, None, None, 0, None) == -1
    # 2048 x 10240 tiles: the leftover round is split along K, so a workspace is required
    need = L.mtnlg_gemm_workspace_bytes(_lib.BF16, 2048, 10240, 20480)
    assert need == 64 * 4 * 256 * 256 * 4
    assert L.mtnlg_gemm(_lib.BF16, 0, 0, 2048, 10240, 20480, A, A, A, None, A, need - 1, None) == -5
    assert L.mtnlg_gemm_workspace_bytes(_lib.BF16, 2048, 7680, 20480) == 0     # 240 tiles: one round
    assert L.mtnlg_layernorm_fwd(_lib.BF16, 4, 12, A, A, A, 1e-5, A, A, A, None) == -2
    assert L.mtnlg_attention_fwd(_lib.F32, 1, 128, 2, 160, A, A, A, None) == -2               # f32 hd 160
    assert L.mtnlg_attention_fwd(_lib.BF16, 1, 96, 2, 128, A, A, A, None) == -2
    assert L.mtnlg_attention_bwd(_lib.BF16, 1, 128, 2, 128, A, A, A, A, A, A, 0, None) == -5


def _stage(layers=3, mb=4, recompute=0, per_mb=1, **kw):
    return _lib.StageDesc(desc(**kw), layers, mb, recompute, 0.0, 0, per_mb)


def test_stage_layout_follows_header():
    """Flat layout: per layer ATTN then MLP, each ln_g | ln_b | w_in | b_in | w_out | b_out."""
    L = lib()
    sd = _stage()
    h, wl, fl = 20480, 16 * 160, 10240
    sizes = {0: [h, h, h * 3 * wl, 3 * wl, wl * h, h], 1: [h, h, h * fl, fl, fl * h, h]}
    per_layer = sum(sizes[0]) + sum(sizes[1])
    assert L.mtnlg_stage_param_count(ctypes.byref(sd)) == 3 * per_layer
    assert 3 * (20480 * 7680 + 2560 * 20480 + 2 * 20480 * 10240) == 1_887_436_800   # GEMM weights alone
    off = (ctypes.c_int64 * 36)()
    assert L.mtnlg_stage_param_offsets(ctypes.byref(sd), off) == 0
    pos = 0
    for l in range(3):
        for half in (0, 1):
            for t in range(6):
                assert off[(l * 2 + half) * 6 + t] == pos
                assert pos % 8 == 0
                pos += sizes[half][t]


def test_stage_workspace_and_validation():
    L = lib()
    sd = _stage()
    n = L.mtnlg_stage_param_count(ctypes.byref(sd))
    act = align256(2048 * 20480 * 2)
    sa = align256(L.mtnlg_saved_bytes(ctypes.byref(sd.layer), _lib.ATTN))
    sm = align256(L.mtnlg_saved_bytes(ctypes.byref(sd.layer), _lib.MLP))
    lw = max(L.mtnlg_workspace_bytes(ctypes.byref(sd.layer), h) for h in (0, 1))
    want = align256(L.mtnlg_adam_workspace_bytes(n)) + act * (2 + 3 + 3) + 3 * (sa + sm) + align256(lw)
    assert L.mtnlg_stage_workspace_bytes(ctypes.byref(sd)) == want
    rc = _stage(recompute=1)
    lw = max(L.mtnlg_recompute_workspace_bytes(ctypes.byref(rc.layer), h) for h in (0, 1))
    want_rc = align256(L.mtnlg_adam_workspace_bytes(n)) + act * 8 + max(sa, sm) + align256(lw)
    assert L.mtnlg_stage_workspace_bytes(ctypes.byref(rc)) == want_rc
    dr = _stage()
    dr.dropout_p = 0.1
    assert L.mtnlg_stage_workspace_bytes(ctypes.byref(dr)) == want + act        # the masked-gradient buffer
    # batched weight gradients (the default): every micro-batch's saved tensors,
    # output gradients (dy and dU or dQKV) and LayerNorm partial rows are kept
    bt = _stage(per_mb=0)
    mb, T, h, wl, fl = 4, 2048, 20480, 16 * 160, 10240
    kept = 3 * mb * ((sa + sm) + 2 * act + T * (3 * wl + fl) * 2)
    got_bt = L.mtnlg_stage_workspace_bytes(ctypes.byref(bt))
    assert kept < got_bt < kept + want + (1 << 30), (got_bt, kept)
    assert L.mtnlg_stage_workspace_bytes(ctypes.byref(_stage(per_mb=2))) == 0
    # recompute ignores the flag
    assert L.mtnlg_stage_workspace_bytes(ctypes.byref(_stage(recompute=1, per_mb=0))) == want_rc
    # invalid descriptors
    bad = _stage()
    bad.dropout_p = 1.0
    assert L.mtnlg_stage_param_count(ctypes.byref(bad)) == -1
    bad.dropout_p = 0.9999999                     # rounds to a threshold of 65536
    assert L.mtnlg_stage_workspace_bytes(ctypes.byref(bad)) == 0
    assert L.mtnlg_stage_param_count(ctypes.byref(_stage(dtype=_lib.F32))) == -1
    assert L.mtnlg_stage_param_count(ctypes.byref(_stage(layers=0))) == -1
    assert L.mtnlg_stage_workspace_bytes(ctypes.byref(_stage(recompute=2))) == 0
    off = (ctypes.c_int64 * 36)()
    assert L.mtnlg_stage_param_offsets(ctypes.byref(_stage(dtype=_lib.F32)), off) == -3
    assert L.mtnlg_stage_param_offsets(ctypes.byref(sd), None) == -1
    cfg = _lib.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 1)
    big = 1 << 40

    def step(c=cfg, ws_bytes=big, grad=A):
        return L.mtnlg_stage_step(ctypes.byref(sd), ctypes.byref(c), A, A, A, A, grad, A, A, A, A, A, A, A,
                                  ws_bytes, None, None)
    assert step(ws_bytes=want - 1) == -5
    assert step(grad=None) == -1
    assert step(grad=ODD) == -4
    assert step(c=_lib.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 0)) == -1
