"""GPU parity of one pipeline-stage step (mtnlg_stage_step) against the oracle.

Stage: 3 chained layers (h 256, 4 heads x 64, MLP 1024, 2 sequences of 128,
bf16, one slice = the whole layer), 2 micro-batches, gradient accumulation
with the norm folded into the last pass, then Adam (step 5, clipping active).
Checked:
* stage outputs and input gradients of every micro-batch, and the accumulated
  gradient tensor by tensor, against the float64 oracle (2e-2, bf16 path);
* the Adam step against the oracle applied to the GPU's own accumulator
  (delta p 1e-4, m and v 1e-5, norm 1e-6); the bf16 weights are the GPU
  master rounded to nearest even, bit for bit;
* the recompute schedule, and the accumulation overlapped on a second
  stream, give bit-identical results to the schedule that keeps the saved
  tensors with per-micro-batch gradients;
* the default schedule (weight gradients once over all micro-batches' rows)
  gives bit-identical stage outputs and input gradients, its accumulated
  gradient passes the same oracle check, and the Adam step is checked on it
  as on the other;
* all of it without dropout, with dropout (p = 0.15) on every half's
  output, and with dropout on the attention probabilities as well (rate 0.1,
  each layer and micro-batch with its own site), the masks drawn by the GPU
  and, independently, by the oracle.
Tolerance metric: ||gpu - oracle||_inf / ||oracle||_inf per tensor.
"""
import numpy as np
import pytest

from helpers import assert_bf16_copy, empty_bytes, rel_inf
from oracle import adam as OA
from oracle import layer as OL
from oracle import stage as OS
from synth.inputs import WORKLOADS, make_activation, make_half_params, randn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tensor_sliced_transformer_amd as tst  # noqa: E402

ATTN_KEYS = {"ln_g": "ln1_g", "ln_b": "ln1_b", "w_in": "w_qkv", "b_in": "b_qkv", "w_out": "w_o", "b_out": "b_o"}
MLP_KEYS = {"ln_g": "ln2_g", "ln_b": "ln2_b", "w_in": "w_a", "b_in": "b_a", "w_out": "w_b", "b_out": "b_b"}


def _setup(L=None, MB=None):
    w = WORKLOADS[6]
    L = L or w.extra["layers"]
    MB = MB or w.extra["micro_batches"]
    ld = tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, 1, 0, tst.BF16, 1e-5)
    halves = [(make_half_params(w, "attn", 0, layer=l), make_half_params(w, "mlp", 0, layer=l)) for l in range(L)]
    full = []
    for a, m in halves:
        d = {ATTN_KEYS[k]: v for k, v in a.items()}
        d.update({MLP_KEYS[k]: v for k, v in m.items()})
        full.append(d)
    xs = [make_activation(w, 10 + k) for k in range(MB)]
    gs = [make_activation(w, 50 + k) for k in range(MB)]
    return w, L, MB, ld, halves, full, xs, gs


def _run(w, L, MB, ld, halves, xs, gs, recompute, cfg, p=0.0, seed=0, aux=False, per_mb=True):
    sd = tst.make_stage_desc(ld, L, MB, recompute, p, seed, per_micro_batch_grads=per_mb)
    n = tst.stage_param_count(sd)
    offs = tst.stage_param_offsets(sd)
    flat = np.zeros(n, dtype=np.float32)
    for l, (a, m) in enumerate(halves):
        for h, p in enumerate((a, m)):
            for k, v in p.items():
                flat[offs[l][h][k]:offs[l][h][k] + v.size] = v.reshape(-1)
    m0 = randn(6001, (n,), 1e-3)
    v0 = randn(6002, (n,), 1e-3) ** 2
    dev = "cuda"
    wt = torch.from_numpy(flat).to(dev).to(torch.bfloat16)
    master = torch.from_numpy(flat).to(dev)
    mm = torch.from_numpy(m0).to(dev)
    vv = torch.from_numpy(v0).to(dev)
    grad = torch.empty(n, dtype=torch.bfloat16, device=dev)
    # batched gradients leave acc untouched: a sentinel shows it
    acc = torch.full((n,), 7.0, dtype=torch.float32, device=dev)
    x = torch.from_numpy(np.stack(xs)).to(dev).to(torch.bfloat16)
    dy = torch.from_numpy(np.stack(gs)).to(dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    stats = torch.zeros(3, dtype=torch.float32, device=dev)
    ws = empty_bytes(tst.stage_workspace_bytes(sd))
    c = tst.AdamCfg(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.max_grad_norm,
                    cfg.inv_loss_scale, cfg.step)
    aux_stream = torch.cuda.Stream() if aux else None
    tst.stage_step(sd, c, wt, master, mm, vv, grad, acc, x, dy, y, dx, stats, ws, aux_stream=aux_stream)
    torch.cuda.synchronize()
    if not per_mb:
        assert bool((acc == 7.0).all()), "batched gradients wrote acc"
    # the step's gradient: acc, or (batched) grad, which the update reads as it is
    step_grad = acc.cpu().numpy() if per_mb else grad.float().cpu().numpy()
    out = {"y": y.float().cpu().numpy(), "dx": dx.float().cpu().numpy(), "acc": step_grad,
           "master": master.cpu().numpy(), "m": mm.cpu().numpy(), "v": vv.cpu().numpy(),
           "w": wt.float().cpu().numpy(), "stats": stats.cpu().numpy()}
    return out, flat, m0, v0, offs


@pytest.mark.parametrize("p,pa", [(0.0, 0.0), (0.15, 0.0), (0.15, 0.1)])
def test_stage_step_against_oracle_and_recompute(p, pa):
    w, L, MB, ld, halves, full, xs, gs = _setup()
    p = float(np.float32(p))           # the rate as the library receives it
    pa = float(np.float32(pa))
    seed = 0xC0FFEE
    attn = (pa, 0xA77E, 7) if pa > 0.0 else None
    if attn is not None:
        ld = tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, 1, 0, tst.BF16, 1e-5, *attn)
    print(f"stage {w.name}: {L} layers, {MB} micro-batches, dropout {p}, attention dropout {pa}", flush=True)
    cfg = OA.AdamConfig(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, max_grad_norm=0.5, inv_loss_scale=1.0,
                        step=w.extra["step"])
    got, flat, m0, v0, offs = _run(w, L, MB, ld, halves, xs, gs, False, cfg, p, seed)
    again, *_ = _run(w, L, MB, ld, halves, xs, gs, True, cfg, p, seed)
    for k in got:
        assert np.array_equal(got[k], again[k]), f"recompute differs in {k}"
    # the accumulation overlapped on a second stream gives the same bits
    ovl, *_ = _run(w, L, MB, ld, halves, xs, gs, False, cfg, p, seed, aux=True)
    for k in got:
        assert np.array_equal(got[k], ovl[k]), f"second stream differs in {k}"
    # batched weight gradients: the same forward and input gradients, bit for
    # bit; the gradients and the step are checked against the oracle below
    bat, *_ = _run(w, L, MB, ld, halves, xs, gs, False, cfg, p, seed, aux=True, per_mb=False)
    for k in ("y", "dx"):
        assert np.array_equal(got[k], bat[k]), f"batched gradients change {k}"

    _against_oracle(w, L, MB, full, xs, gs, p, seed, attn, cfg, flat, m0, v0, offs, {"": got, "batched ": bat})


@pytest.mark.parametrize("L,MB,p", [(1, 1, 0.0), (2, 3, 0.15)])
def test_stage_batched_gradients_edge_shapes(L, MB, p):
    """The batched-gradient schedule at one layer and one micro-batch (the
    gradients computed right after the only backward; the top layer is also
    layer 0) and at two layers and three micro-batches with dropout: outputs
    and input gradients bit-identical to the per-micro-batch schedule, both
    against the stage and Adam oracles."""
    w, L, MB, ld, halves, full, xs, gs = _setup(L, MB)
    p = float(np.float32(p))
    seed = 0xBEE5
    print(f"stage {w.name}: {L} layers, {MB} micro-batches, dropout {p}", flush=True)
    cfg = OA.AdamConfig(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, max_grad_norm=0.5, inv_loss_scale=1.0,
                        step=w.extra["step"])
    got, flat, m0, v0, offs = _run(w, L, MB, ld, halves, xs, gs, False, cfg, p, seed)
    bat, *_ = _run(w, L, MB, ld, halves, xs, gs, False, cfg, p, seed, per_mb=False)
    for k in ("y", "dx"):
        assert np.array_equal(got[k], bat[k]), f"batched gradients change {k}"
    _against_oracle(w, L, MB, full, xs, gs, p, seed, None, cfg, flat, m0, v0, offs, {"": got, "batched ": bat})


def _against_oracle(w, L, MB, full, xs, gs, p, seed, attn, cfg, flat, m0, v0, offs, runs):
    """Every run's outputs, input gradients and accumulated gradient against the
    stage oracle (2e-2), and its Adam step against the Adam oracle applied to
    its own accumulator."""
    got = runs[""] if "" in runs else next(iter(runs.values()))
    sh = OL.LayerShape(batch=w.batch, seq=w.seq, hidden=w.hidden, heads=w.heads, ffn=w.ffn, tp=1)
    ys, dxs, flats = OS.stage_micro_batches(sh, [{k: v.astype(np.float64) for k, v in q.items()} for q in full],
                                            [x.astype(np.float64) for x in xs], [g.astype(np.float64) for g in gs],
                                            dropout=(p, seed), attn_dropout=attn)
    errs = {}
    for k in range(MB):
        errs[f"y{k}"] = rel_inf(got["y"][k], ys[k])
        errs[f"dx{k}"] = rel_inf(got["dx"][k], dxs[k])
    acc_ref = OA.accumulate(flats)
    # the oracle's flat order is the documented layout: check it tensor by tensor
    for tag, run in runs.items():
        pos = 0
        for l in range(L):
            for h, keys in enumerate((ATTN_KEYS, MLP_KEYS)):
                for k, fk in keys.items():
                    size = full[l][fk].size
                    assert offs[l][h][k] == pos, (l, h, k)
                    errs[f"{tag}acc{l}.{fk}"] = rel_inf(run["acc"][pos:pos + size], acc_ref[pos:pos + size])
                    pos += size
    worst = max(errs, key=errs.get)
    print(f"stage parity: worst {worst} {errs[worst]:.3e}", flush=True)
    for k, e in errs.items():
        assert e < 2e-2, f"{k}: {e:.3e}"

    for run in runs.values():
        rp, rm, rv, rw, (norm, coef, inf) = OA.adam_step(flat.astype(np.float64), m0.astype(np.float64),
                                                        v0.astype(np.float64), run["acc"].astype(np.float64), cfg)
        assert not inf and run["stats"][2] == 0.0
        assert coef < 1.0, "clipping should be active"
        assert abs(run["stats"][0] - norm) <= 1e-6 * norm
        assert abs(run["stats"][1] - coef) <= 1e-6
        assert rel_inf(run["master"] - flat, rp - flat) < 1e-4
        assert rel_inf(run["m"], rm) < 1e-5
        assert rel_inf(run["v"], rv) < 1e-5
        assert_bf16_copy(run["w"], run["master"], rw, rp)
