"""Every buffer the library writes stays inside its bounds, and optimizer state
can be saved and restored mid-run.

* Guard bands: each output, saved-tensor buffer and workspace is placed in
  the middle of a larger allocation whose 4 KiB before and after are filled
  with a fixed byte; after the calls every guard byte must be unchanged. Run
  for both halves of the 1/8 MT-NLG slice and of the tiny fp32 layer
  (forward, backward, backward with recompute), a pipeline-stage step, the
  optimizer entry points, the dropout kernels, GEMMs with and without split
  pieces and the attention kernels, at ragged sizes where the kernels have
  tails.
* Resume: two Adam steps equal, bit for bit, one step, a copy of the state
  to the host and back into fresh buffers, and a second step.
"""
import numpy as np
import pytest

from synth.inputs import WORKLOADS, make_activation, make_half_params

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tensor_sliced_transformer_amd as tst  # noqa: E402

PAD = 4096
FILL = 0xA5
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


class Guarded:
    """A tensor view in the middle of a guard-banded byte buffer."""

    def __init__(self, shape, dtype, nbytes=None):
        esize = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape)) if shape is not None else None
        self.nbytes = nbytes if nbytes is not None else n * esize
        self.buf = torch.full((self.nbytes + 2 * PAD,), FILL, dtype=torch.uint8, device="cuda")
        inner = self.buf[PAD:PAD + self.nbytes]
        self.t = inner if shape is None else inner.view(dtype).view(shape)

    def intact(self):
        return bool((self.buf[:PAD] == FILL).all()) and bool((self.buf[PAD + self.nbytes:] == FILL).all())


def check_all(named):
    torch.cuda.synchronize()
    bad = [k for k, g in named.items() if not g.intact()]
    assert not bad, f"written outside their bounds: {bad}"


@pytest.mark.parametrize("wi,half", [(1, "attn"), (1, "mlp"), (3, "attn"), (3, "mlp")])
def test_layer_half_writes_inside_its_buffers(wi, half):
    w = WORKLOADS[wi]
    print(f"guards {w.name} {half}", flush=True)
    hf = tst.ATTN if half == "attn" else tst.MLP
    desc = tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, w.tp, 0,
                         tst.BF16 if w.dtype == "bf16" else tst.F32, 1e-5)
    dt = TDT[w.dtype]
    pn = make_half_params(w, half, 0)
    p = {k: torch.from_numpy(v).to(dt).cuda() for k, v in pn.items() if k != "b_out"}
    x = torch.from_numpy(make_activation(w, 1)).to(dt).cuda()
    dy = torch.from_numpy(make_activation(w, 2)).to(dt).cuda()
    g = {}
    y = Guarded((w.tokens, w.hidden), dt)
    dx = Guarded((w.tokens, w.hidden), dt)
    saved = Guarded(None, torch.uint8, tst.saved_bytes(desc, hf))
    ws = Guarded(None, torch.uint8, tst.workspace_bytes(desc, hf))
    rws = Guarded(None, torch.uint8, tst.recompute_workspace_bytes(desc, hf))
    grads = {k: Guarded(v.shape, dt) for k, v in pn.items()}
    tst.layer_fwd(desc, hf, p, x, y.t, saved.t, ws.t)
    tst.layer_bwd(desc, hf, p, x, saved.t, dy, dx.t, {k: v.t for k, v in grads.items()}, ws.t)
    tst.layer_bwd_recompute(desc, hf, p, x, dy, dx.t, {k: v.t for k, v in grads.items()}, rws.t)
    g.update({"y": y, "dx": dx, "saved": saved, "ws": ws, "recompute_ws": rws})
    g.update({f"grad.{k}": v for k, v in grads.items()})
    check_all(g)


def test_stage_step_writes_inside_its_buffers():
    w = WORKLOADS[6]
    L, MB = w.extra["layers"], w.extra["micro_batches"]
    ld = tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, 1, 0, tst.BF16, 1e-5)
    sd = tst.make_stage_desc(ld, L, MB, False, 0.1, 7)
    n = tst.stage_param_count(sd)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    bufs = {"w": Guarded((n,), torch.bfloat16), "master": Guarded((n,), torch.float32),
            "m": Guarded((n,), torch.float32), "v": Guarded((n,), torch.float32),
            "grad": Guarded((n,), torch.bfloat16), "acc": Guarded((n,), torch.float32),
            "y": Guarded((MB, w.tokens, w.hidden), torch.bfloat16),
            "dx": Guarded((MB, w.tokens, w.hidden), torch.bfloat16),
            "stats": Guarded((3,), torch.float32),
            "ws": Guarded(None, torch.uint8, tst.stage_workspace_bytes(sd))}
    bufs["master"].t.copy_(torch.randn(n, device="cuda", generator=gen) * 0.02)
    bufs["w"].t.copy_(bufs["master"].t.to(torch.bfloat16))
    bufs["m"].t.zero_()
    bufs["v"].t.zero_()
    x = torch.randn((MB, w.tokens, w.hidden), device="cuda", generator=gen).to(torch.bfloat16)
    dy = torch.randn((MB, w.tokens, w.hidden), device="cuda", generator=gen).to(torch.bfloat16)
    cfg = tst.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 1)
    b = {k: v.t for k, v in bufs.items()}
    tst.stage_step(sd, cfg, b["w"], b["master"], b["m"], b["v"], b["grad"], b["acc"], x, dy, b["y"], b["dx"],
                   b["stats"], b["ws"], aux_stream=torch.cuda.Stream())
    check_all(bufs)


@pytest.mark.parametrize("n", [5, 4099, 1000003])
def test_optimizer_and_dropout_write_inside_their_buffers(n):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    g = (torch.randn(n, device="cuda", generator=gen) * 1e-3).to(torch.bfloat16)
    bufs = {"acc": Guarded((n,), torch.float32), "master": Guarded((n,), torch.float32),
            "m": Guarded((n,), torch.float32), "v": Guarded((n,), torch.float32),
            "w": Guarded((n,), torch.bfloat16), "stats": Guarded((3,), torch.float32),
            "ws": Guarded(None, torch.uint8, tst.adam_workspace_bytes(n))}
    b = {k: v.t for k, v in bufs.items()}
    b["master"].copy_(torch.randn(n, device="cuda", generator=gen) * 0.02)
    b["m"].zero_()
    b["v"].zero_()
    cfg = tst.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 1)
    tst.grad_accumulate(g, b["acc"], overwrite=True)
    tst.grad_accumulate_norm(g, b["acc"], False, 1.0, b["ws"])
    tst.adam_update(cfg, b["master"], b["m"], b["v"], b["acc"], b["w"], b["stats"], b["ws"])
    tst.adam_step(cfg, b["master"], b["m"], b["v"], b["acc"], b["w"], b["stats"], b["ws"])
    # dropout on a ragged [rows, 24] tensor (the last generator block is half used)
    rows = max(1, n // 24)
    part = torch.randn((rows, 24), device="cuda", generator=gen).to(torch.bfloat16)
    out = Guarded((rows, 24), torch.bfloat16)
    dz = Guarded((rows, 24), torch.bfloat16)
    tst.reduce_partials_dropout([part], out.t, 0.3, 5, 1, residual=part)
    tst.dropout_bwd(part, dz.t, 0.3, 5, 1)
    bufs.update({"dropout_out": out, "dropout_dz": dz})
    check_all(bufs)


def test_adam_resume_is_bit_identical():
    """Two steps in a row equal one step, the state copied to the host and into
    fresh buffers, then the second step (the state is the caller's flat buffers
    plus the step count)."""
    n = 1 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    master = torch.randn(n, device="cuda", generator=gen) * 0.02
    g1 = torch.randn(n, device="cuda", generator=gen) * 1e-3
    g2 = torch.randn(n, device="cuda", generator=gen) * 1e-3
    ws = torch.empty(tst.adam_workspace_bytes(n), dtype=torch.uint8, device="cuda")

    def step(state, grad, t):
        cfg = tst.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.01, 1.0, 1.0, t)
        stats = torch.zeros(3, device="cuda")
        tst.adam_step(cfg, state["p"], state["m"], state["v"], grad, state["w"], stats, ws)

    a = {"p": master.clone(), "m": torch.zeros(n, device="cuda"), "v": torch.zeros(n, device="cuda"),
         "w": torch.empty(n, dtype=torch.bfloat16, device="cuda")}
    step(a, g1, 1)
    step(a, g2, 2)
    b = {"p": master.clone(), "m": torch.zeros(n, device="cuda"), "v": torch.zeros(n, device="cuda"),
         "w": torch.empty(n, dtype=torch.bfloat16, device="cuda")}
    step(b, g1, 1)
    torch.cuda.synchronize()
    saved = {k: v.cpu().clone() for k, v in b.items()}
    del b
    c = {k: v.cuda() for k, v in saved.items()}
    step(c, g2, 2)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], c[k]), k


@pytest.mark.parametrize("M,N,K,ta,tb", [(2048, 2560, 20480, 0, 1), (2048, 20480, 2560, 0, 0), (200, 264, 72, 1, 0),
                                         (520, 1032, 4096, 1, 1)])
def test_gemm_and_attention_write_inside_their_buffers(M, N, K, ta, tb):
    """GEMMs with whole-problem and tail splits (fp32 partials in the workspace),
    ragged tiles, and the attention forward/backward of the slice's heads."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(14)
    a = (torch.randn((K, M) if ta else (M, K), device="cuda", generator=gen)).to(torch.bfloat16)
    b = (torch.randn((N, K) if tb else (K, N), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    c = Guarded((M, N), torch.bfloat16)
    wsb = tst.gemm_workspace_bytes(tst.BF16, M, N, K)
    ws = Guarded(None, torch.uint8, max(wsb, 16))
    tst.gemm(a, b, c.t, bool(ta), bool(tb), ws=ws.t if wsb else None)
    bufs = {"c": c, "gemm_ws": ws}
    if M == 2048:
        B, S, H, D = 1, 2048, 16, 160
        qkv32 = torch.randn((B * S, 3 * H * D), device="cuda", generator=gen) * 2.9
        # Q and K in fp16, V in bf16 (the bf16 path's storage of the attention input)
        qkv = torch.cat([qkv32[:, :2 * H * D].to(torch.float16).view(torch.bfloat16),
                         qkv32[:, 2 * H * D:].to(torch.bfloat16)], dim=1).contiguous()
        do = torch.randn((B * S, H * D), device="cuda", generator=gen).to(torch.bfloat16)
        o = Guarded((B * S, H * D), torch.bfloat16)
        lse = Guarded((H, B * S), torch.float32)
        dqkv = Guarded((B * S, 3 * H * D), torch.bfloat16)
        aws = Guarded(None, torch.uint8, max(16, tst.attention_bwd_workspace_bytes(B, S, H)))
        tst.attention_fwd(qkv, o.t, lse.t, B, S, H, D)
        tst.attention_bwd(qkv, o.t, lse.t, do, dqkv.t, aws.t, B, S, H, D)
        bufs.update({"o": o, "lse": lse, "dqkv": dqkv, "attn_ws": aws})
    check_all(bufs)
