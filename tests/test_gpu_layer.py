"""GPU parity of whole layer halves and whole sliced layers against the CPU oracle.

* tiny layer, fp32, t = 2 slices run in turn: forward, backward (both halves,
  partial sums through mtnlg_reduce_partials) and one Adam step over every
  parameter, compared in full with the oracle's unsliced layer;
* GPT-style layer h 4096, t = 1, bf16: each half forward + backward in full;
* MT-NLG 1/8 shard h 20480, 16 heads x 160, bf16: each half forward + backward
  in full (the oracle runs the same slice in float64);
* run-to-run determinism of a backward;
* the backward that recomputes the forward is bit-identical to the stored one;
* the tiny layer with dropout on both halves (Philox masks) against the oracle;
* dropout on the attention probabilities (head_dim 64, 128 and 160, slices
  of rank > 0 so the global head index enters the mask, and the MT-NLG shard
  at full size): forward and backward against the oracle drawing the same
  mask, and the recomputing backward bit-identical to the stored one.
Tolerance: ||gpu - oracle||_inf / ||oracle||_inf per tensor (1e-4 fp32, 2e-2 bf16).
"""
from dataclasses import replace

import numpy as np
import pytest

from helpers import TOL, assert_close, empty, empty_bytes, rel_inf, rel_l2, round_to_f16, to_gpu, to_np
from oracle import adam as OA
from oracle.bf16 import round_to_bf16
from oracle import dropout as OD
from oracle import layer as OL
from synth.inputs import WORKLOADS, make_activation, make_half_params

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tensor_sliced_transformer_amd as tst  # noqa: E402

HALF = {"attn": tst.ATTN, "mlp": tst.MLP}


def desc_of(w, rank=0):
    return tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, w.tp, rank,
                         tst.BF16 if w.dtype == "bf16" else tst.F32, 1e-5)


def shape_of(w):
    return OL.LayerShape(batch=w.batch, seq=w.seq, hidden=w.hidden, heads=w.heads, ffn=w.ffn, tp=w.tp)


class GpuHalf:
    """Device buffers and calls of one slice of one half."""

    def __init__(self, w, half, params_np, rank=0, desc=None):
        self.w, self.half, self.dt = w, half, w.dtype
        self.desc = desc_of(w, rank) if desc is None else desc
        self.p = {k: to_gpu(v, self.dt) for k, v in params_np.items() if k != "b_out"}
        self.saved = empty_bytes(tst.saved_bytes(self.desc, HALF[half]))
        self.ws = empty_bytes(tst.workspace_bytes(self.desc, HALF[half]))
        self.g = {k: empty(v.shape, self.dt) for k, v in params_np.items()}

    def fwd(self, x):
        y = empty((self.w.tokens, self.w.hidden), self.dt)
        tst.layer_fwd(self.desc, HALF[self.half], self.p, x, y, self.saved, self.ws)
        return y

    def bwd(self, x, dy):
        dx = empty((self.w.tokens, self.w.hidden), self.dt)
        tst.layer_bwd(self.desc, HALF[self.half], self.p, x, self.saved, dy, dx, self.g, self.ws)
        return dx


def oracle_params(p):
    return {k: v.astype(np.float64) for k, v in p.items()}


def check_half(w, half, tag_x, tag_g, rank=0, attn_drop=None):
    """Forward and backward of slice `rank` of one half vs the oracle, every
    output in full. attn_drop: None, or (rate, seed, site) for dropout on the
    attention probabilities. Returns the GpuHalf and the inputs on the GPU."""
    print(f"{w.name} {half} slice {rank} attention dropout {attn_drop}", flush=True)
    pn = make_half_params(w, half, rank)
    x = make_activation(w, tag_x)
    g = make_activation(w, tag_g)
    desc = None
    if attn_drop is not None:
        desc = tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, w.tp, rank, tst.BF16, 1e-5, *attn_drop)
    gh = GpuHalf(w, half, pn, rank, desc)
    xg, gg = to_gpu(x, w.dtype), to_gpu(g, w.dtype)
    y = gh.fwd(xg)
    dx = gh.bwd(xg, gg)
    torch.cuda.synchronize()
    sh = shape_of(w)
    po = oracle_params(pn)
    fwd, bwd = (OL.attn_half_fwd, OL.attn_half_bwd) if half == "attn" else (OL.mlp_half_fwd, OL.mlp_half_bwd)

    def run_oracle(store):
        kw = {"store": store}
        if half == "attn" and store is not None:
            kw["store_qk"] = round_to_f16
        if half == "attn" and attn_drop is not None:
            kw["attn_drop"] = (*attn_drop, rank * sh.local_heads)
        part, saved = fwd(sh, x.astype(np.float64), po, **kw)
        rdx, rg, _ = bwd(sh, g.astype(np.float64), po, saved)
        return part, rdx, rg

    got = {"y_partial": to_np(y), "dx_partial": to_np(dx)}
    got.update({k: to_np(gh.g[k]) for k in ("ln_g", "ln_b", "w_in", "b_in", "w_out", "b_out")})
    part, rdx, rg = run_oracle(None)
    ref = {"y_partial": part, "dx_partial": rdx, **rg}
    errs = {k: assert_close(k, got[k], ref[k], w.dtype) for k in got}
    print("vs oracle:", {k: f"{v:.2e}" for k, v in errs.items()}, "l2(y)",
          f"{rel_l2(got['y_partial'], part):.2e}", flush=True)
    if w.dtype == "bf16":
        # diagnostic mode: the oracle also rounds the saved tensors as the
        # library stores them (LN output, V, O, U, Y in bf16; Q and K in fp16),
        # so what is left is the kernels' own error
        part, rdx, rg = run_oracle(round_to_bf16)
        ref = {"y_partial": part, "dx_partial": rdx, **rg}
        diag = {k: rel_inf(got[k], ref[k]) for k in got}
        print("vs oracle with bf16 saved tensors:", {k: f"{v:.2e}" for k, v in diag.items()}, flush=True)
        for k, e in diag.items():
            assert e <= TOL["bf16"], f"{k}: {e:.3e} against the diagnostic oracle"
    return gh, xg, gg


@pytest.mark.parametrize("half", ["attn", "mlp"])
def test_gpt_layer_h4096_halves(half):
    check_half(WORKLOADS[2], half, 1, 2)


@pytest.mark.parametrize("half", ["attn", "mlp"])
def test_mtnlg_shard_halves(half):
    check_half(WORKLOADS[3], half, 1, 2)


def test_tiny_layer_two_slices_and_adam():
    """Whole layer from t = 2 slices (fp32) against the oracle's unsliced layer, then one Adam step."""
    w = WORKLOADS[1]
    sh = shape_of(w)
    ap = [make_half_params(w, "attn", i) for i in range(w.tp)]
    mp = [make_half_params(w, "mlp", i) for i in range(w.tp)]
    x = make_activation(w, 1)
    gout = make_activation(w, 2)
    # full parameters assembled from the slices (the oracle slices them again)
    full = {k: np.zeros(s) for k, s in OL.full_param_shapes(sh).items()}
    full["ln1_g"], full["ln1_b"], full["b_o"] = ap[0]["ln_g"], ap[0]["ln_b"], ap[0]["b_out"]
    full["ln2_g"], full["ln2_b"], full["b_b"] = mp[0]["ln_g"], mp[0]["ln_b"], mp[0]["b_out"]
    wl, fl = sh.local_width, sh.local_ffn
    for i in range(w.tp):
        cols = OL.qkv_columns(sh, i)
        full["w_qkv"][:, cols] = ap[i]["w_in"]
        full["b_qkv"][cols] = ap[i]["b_in"]
        full["w_o"][i * wl:(i + 1) * wl] = ap[i]["w_out"]
        full["w_a"][:, i * fl:(i + 1) * fl] = mp[i]["w_in"]
        full["b_a"][i * fl:(i + 1) * fl] = mp[i]["b_in"]
        full["w_b"][i * fl:(i + 1) * fl] = mp[i]["w_out"]
    full = {k: np.asarray(v, dtype=np.float64) for k, v in full.items()}

    dt = w.dtype
    A = [GpuHalf(w, "attn", ap[i], i) for i in range(w.tp)]
    M = [GpuHalf(w, "mlp", mp[i], i) for i in range(w.tp)]
    xg = to_gpu(x, dt)
    bo, bb = to_gpu(ap[0]["b_out"], dt), to_gpu(mp[0]["b_out"], dt)
    x1 = empty(x.shape, dt)
    tst.reduce_partials([a.fwd(xg) for a in A], x1, residual=xg, bias=bo)
    out = empty(x.shape, dt)
    tst.reduce_partials([m.fwd(x1) for m in M], out, residual=x1, bias=bb)
    gg = to_gpu(gout, dt)
    g1 = empty(x.shape, dt)
    tst.reduce_partials([m.bwd(x1, gg) for m in M], g1, residual=gg)
    dx = empty(x.shape, dt)
    tst.reduce_partials([a.bwd(xg, g1) for a in A], dx, residual=g1)
    torch.cuda.synchronize()

    rout, st = OL.layer_fwd(sh, x.astype(np.float64), full)
    rdx, rg = OL.layer_bwd(sh, gout.astype(np.float64), full, st)
    assert_close("x1", to_np(x1), st["x1"], dt)
    assert_close("out", to_np(out), rout, dt)
    assert_close("dx", to_np(dx), rdx, dt)
    # weight gradients: slices vs the columns/rows of the unsliced gradient
    for i in range(w.tp):
        cols = OL.qkv_columns(sh, i)
        assert_close("dw_qkv", to_np(A[i].g["w_in"]), rg["w_qkv"][:, cols], dt)
        assert_close("db_qkv", to_np(A[i].g["b_in"]), rg["b_qkv"][cols], dt)
        assert_close("dw_o", to_np(A[i].g["w_out"]), rg["w_o"][i * wl:(i + 1) * wl], dt)
        assert_close("dw_a", to_np(M[i].g["w_in"]), rg["w_a"][:, i * fl:(i + 1) * fl], dt)
        assert_close("db_a", to_np(M[i].g["b_in"]), rg["b_a"][i * fl:(i + 1) * fl], dt)
        assert_close("dw_b", to_np(M[i].g["w_out"]), rg["w_b"][i * fl:(i + 1) * fl], dt)
        assert_close("db_o", to_np(A[i].g["b_out"]), rg["b_o"], dt)
        assert_close("db_b", to_np(M[i].g["b_out"]), rg["b_b"], dt)
    # replicated LayerNorm parameters: sum of the slice partials
    for key, halves, name in (("ln_g", A, "ln1_g"), ("ln_b", A, "ln1_b"), ("ln_g", M, "ln2_g"), ("ln_b", M, "ln2_b")):
        tot = empty(halves[0].g[key].shape, dt)
        tst.reduce_partials([h.g[key].view(1, -1) for h in halves], tot.view(1, -1))
        torch.cuda.synchronize()
        assert_close(name, to_np(tot), rg[name], dt)

    # one Adam step over the flat parameter vector of slice 0's attention half (fp32 grads
    # accumulated into the fp32 accumulator; lr 1e-4, betas 0.9/0.95, eps 1e-8)
    flat_p = np.concatenate([ap[0][k].ravel() for k in ("w_in", "b_in", "w_out")]).astype(np.float32)
    flat_g = torch.cat([A[0].g[k].reshape(-1) for k in ("w_in", "b_in", "w_out")]).contiguous()
    n = flat_p.size
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    tst.grad_accumulate(flat_g, acc, overwrite=True)
    mg = torch.from_numpy(flat_p.copy()).cuda()
    mm = torch.zeros(n, device="cuda")
    vv = torch.zeros(n, device="cuda")
    stats = torch.zeros(3, device="cuda")
    ws = empty_bytes(tst.adam_workspace_bytes(n))
    tst.adam_step(tst.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 1), mg, mm, vv, acc, None, stats, ws)
    torch.cuda.synchronize()
    cfg = OA.AdamConfig(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, max_grad_norm=1.0, step=1)
    ga = to_np(acc)
    rp, rm, rv, _, (norm, coef, inf) = OA.adam_step(flat_p.astype(np.float64), np.zeros(n), np.zeros(n), ga, cfg)
    assert not inf
    assert abs(to_np(stats)[0] - norm) <= 1e-5 * norm
    assert rel_inf(to_np(mg) - flat_p, rp - flat_p) < 1e-4
    assert rel_inf(to_np(mm), rm) < 1e-5 and rel_inf(to_np(vv), rv) < 1e-5


def test_backward_is_deterministic():
    w = WORKLOADS[2]
    pn = make_half_params(w, "mlp", 0)
    x = to_gpu(make_activation(w, 1), w.dtype)
    g = to_gpu(make_activation(w, 2), w.dtype)
    gh = GpuHalf(w, "mlp", pn)
    gh.fwd(x)
    dx1 = gh.bwd(x, g).clone()
    g1 = {k: v.clone() for k, v in gh.g.items()}
    dx2 = gh.bwd(x, g)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2)
    for k in g1:
        assert torch.equal(g1[k], gh.g[k]), k


@pytest.mark.parametrize("wi,half", [(1, "attn"), (1, "mlp"), (3, "attn"), (3, "mlp")])
def test_recompute_backward_matches_stored(wi, half):
    """The backward that re-runs the forward from the layer input alone gives
    bit-identical input and parameter gradients to forward + backward with the
    stored activations (the same kernels run on the same values)."""
    w = WORKLOADS[wi]
    print(f"recompute {w.name} {half}", flush=True)
    pn = make_half_params(w, half, 0)
    x = to_gpu(make_activation(w, 1), w.dtype)
    g = to_gpu(make_activation(w, 2), w.dtype)
    gh = GpuHalf(w, half, pn)
    gh.fwd(x)
    dx_ref = gh.bwd(x, g).clone()
    g_ref = {k: v.clone() for k, v in gh.g.items()}
    ws = empty_bytes(tst.recompute_workspace_bytes(gh.desc, HALF[half]))
    dx = empty((w.tokens, w.hidden), w.dtype)
    for k in gh.g:
        gh.g[k].fill_(float("nan"))
    tst.layer_bwd_recompute(gh.desc, HALF[half], gh.p, x, g, dx, gh.g, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref)
    for k in g_ref:
        assert torch.equal(gh.g[k], g_ref[k]), k


def test_tiny_layer_two_slices_with_dropout():
    """The t = 2 fp32 layer with dropout (p = 0.2) on both halves' outputs:
    forward through mtnlg_reduce_partials_dropout, backward through
    mtnlg_dropout_bwd into each half's backward, against the oracle with the
    same Philox masks (1e-4)."""
    w = WORKLOADS[1]
    sh = shape_of(w)
    p = float(np.float32(0.2))
    seed, sites = 2024, (10, 11)
    ap = [make_half_params(w, "attn", i) for i in range(w.tp)]
    mp = [make_half_params(w, "mlp", i) for i in range(w.tp)]
    x = make_activation(w, 1)
    gout = make_activation(w, 2)
    full = {k: np.zeros(s) for k, s in OL.full_param_shapes(sh).items()}
    full["ln1_g"], full["ln1_b"], full["b_o"] = ap[0]["ln_g"], ap[0]["ln_b"], ap[0]["b_out"]
    full["ln2_g"], full["ln2_b"], full["b_b"] = mp[0]["ln_g"], mp[0]["ln_b"], mp[0]["b_out"]
    wl, fl = sh.local_width, sh.local_ffn
    for i in range(w.tp):
        cols = OL.qkv_columns(sh, i)
        full["w_qkv"][:, cols] = ap[i]["w_in"]
        full["b_qkv"][cols] = ap[i]["b_in"]
        full["w_o"][i * wl:(i + 1) * wl] = ap[i]["w_out"]
        full["w_a"][:, i * fl:(i + 1) * fl] = mp[i]["w_in"]
        full["b_a"][i * fl:(i + 1) * fl] = mp[i]["b_in"]
        full["w_b"][i * fl:(i + 1) * fl] = mp[i]["w_out"]
    full = {k: np.asarray(v, dtype=np.float64) for k, v in full.items()}

    dt = w.dtype
    A = [GpuHalf(w, "attn", ap[i], i) for i in range(w.tp)]
    M = [GpuHalf(w, "mlp", mp[i], i) for i in range(w.tp)]
    xg = to_gpu(x, dt)
    bo, bb = to_gpu(ap[0]["b_out"], dt), to_gpu(mp[0]["b_out"], dt)
    x1 = empty(x.shape, dt)
    tst.reduce_partials_dropout([a.fwd(xg) for a in A], x1, p, seed, sites[0], residual=xg, bias=bo)
    out = empty(x.shape, dt)
    tst.reduce_partials_dropout([m.fwd(x1) for m in M], out, p, seed, sites[1], residual=x1, bias=bb)
    gg = to_gpu(gout, dt)
    dz = empty(x.shape, dt)
    tst.dropout_bwd(gg, dz, p, seed, sites[1])
    g1 = empty(x.shape, dt)
    tst.reduce_partials([m.bwd(x1, dz) for m in M], g1, residual=gg)
    dz1 = empty(x.shape, dt)
    tst.dropout_bwd(g1, dz1, p, seed, sites[0])
    dx = empty(x.shape, dt)
    tst.reduce_partials([a.bwd(xg, dz1) for a in A], dx, residual=g1)
    torch.cuda.synchronize()

    rout, st = OD.layer_fwd(sh, x.astype(np.float64), full, p, seed, sites)
    rdx, ga, gm = OD.layer_bwd(sh, gout.astype(np.float64), st, p, seed, sites)
    assert_close("x1", to_np(x1), st["x1"], dt)
    assert_close("out", to_np(out), rout, dt)
    assert_close("dx", to_np(dx), rdx, dt)
    for i in range(w.tp):
        for k in ("ln_g", "ln_b", "w_in", "b_in", "w_out", "b_out"):
            assert_close(f"attn{i}.{k}", to_np(A[i].g[k]), ga[i][k], dt)
            assert_close(f"mlp{i}.{k}", to_np(M[i].g[k]), gm[i][k], dt)


# Shapes for dropout on the attention probabilities: head_dim 64, 128 and 160;
# slices of rank > 0 (the mask takes the global head index); seq 384 is three
# 128-query tiles.
ATTN_DROP = [
    replace(WORKLOADS[6], index=61, name="attn-drop-d64-t2", batch=2, seq=256, hidden=256, heads=4, ffn=1024,
            tp=2, slices=(1,), extra={}),
    replace(WORKLOADS[6], index=62, name="attn-drop-d128", batch=2, seq=256, hidden=512, heads=4, ffn=1024,
            tp=1, slices=(0,), extra={}),
    replace(WORKLOADS[6], index=63, name="attn-drop-d160-t2", batch=2, seq=384, hidden=640, heads=4, ffn=1280,
            tp=2, slices=(1,), extra={}),
]


@pytest.mark.parametrize("wi", range(len(ATTN_DROP)))
def test_attention_probability_dropout(wi):
    """Forward and backward of the attention half with dropout (rate 0.1) on
    its probabilities against the oracle with the same mask; the recomputing
    backward regenerates the mask and is bit-identical to the stored one."""
    w = ATTN_DROP[wi]
    rank = w.slices[0]
    drop = (float(np.float32(0.1)), 0x5EED00 + wi, 3 + wi)
    gh, xg, gg = check_half(w, "attn", 1, 2, rank, drop)
    dx_ref = gh.bwd(xg, gg).clone()
    g_ref = {k: v.clone() for k, v in gh.g.items()}
    ws = empty_bytes(tst.recompute_workspace_bytes(gh.desc, tst.ATTN))
    dx = empty((w.tokens, w.hidden), w.dtype)
    for k in gh.g:
        gh.g[k].fill_(float("nan"))
    tst.layer_bwd_recompute(gh.desc, tst.ATTN, gh.p, xg, gg, dx, gh.g, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref)
    for k in g_ref:
        assert torch.equal(gh.g[k], g_ref[k]), k


def test_mtnlg_shard_attention_dropout():
    """The MT-NLG attention slice of rank 3 (global heads 48..63) at full size
    with dropout 0.1 on its probabilities, every output against the oracle."""
    check_half(WORKLOADS[3], "attn", 1, 2, 3, (float(np.float32(0.1)), 20220128, 5))
