"""GPU parity of the library's component entry points against the CPU oracle.

Each entry point of include/mtnlg.h is called through the C ABI on seeded
inputs that span several tiles and a ragged tail, and compared element by
element with the oracle (float64) on the same bf16-exact or fp32 values.
"""
import numpy as np
import pytest

from helpers import TOL, assert_bf16_copy, assert_close, empty, empty_bytes, rel_inf, to_gpu, to_np
from oracle import adam as OA
from oracle import dropout as OD
from oracle import layer as OL
from synth.inputs import qkv_bits, randn, round_f32_to_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tensor_sliced_transformer_amd as tst  # noqa: E402


def inputs(seed, shape, dtype, std=1.0, mean=0.0):
    x = randn(seed, shape, std, mean)
    return round_f32_to_bf16(x) if dtype == "bf16" else x


# ------------------------------------------------------------------ GEMM
GEMM_SHAPES = [(256, 384, 320), (136, 200, 72), (520, 264, 1032), (64, 64, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm(dtype, ta, tb, shape):
    M, N, K = shape
    print(f"gemm {dtype} ta={ta} tb={tb} {shape}", flush=True)
    a = inputs(11, (K, M) if ta else (M, K), dtype)
    b = inputs(12, (N, K) if tb else (K, N), dtype)
    bias = inputs(13, (N,), dtype)
    c = empty((M, N), dtype)
    ws = empty_bytes(tst.gemm_workspace_bytes(tst.BF16 if dtype == "bf16" else tst.F32, M, N, K))
    tst.gemm(to_gpu(a, dtype), to_gpu(b, dtype), c, bool(ta), bool(tb), bias=to_gpu(bias, dtype), ws=ws)
    torch.cuda.synchronize()
    A = a.astype(np.float64).T if ta else a.astype(np.float64)
    B = b.astype(np.float64).T if tb else b.astype(np.float64)
    assert_close("C", to_np(c), A @ B + bias.astype(np.float64)[None, :], dtype)


@pytest.mark.parametrize("M,N,K", [(2048, 2560, 1024), (2048, 10240, 2048), (4096, 4096, 512)])
def test_gemm_large_tiles_bf16(M, N, K):
    """256x256 tiles with several XCD groups; 320 tiles (2048 x 10240) exercise the K-split
    of the tiles left over after one round of 256 workgroups."""
    a = inputs(14, (M, K), "bf16")
    b = inputs(15, (K, N), "bf16")
    bias = inputs(16, (N,), "bf16")
    c = empty((M, N), "bf16")
    ws = empty_bytes(tst.gemm_workspace_bytes(tst.BF16, M, N, K))
    tst.gemm(to_gpu(a, "bf16"), to_gpu(b, "bf16"), c, bias=to_gpu(bias, "bf16"), ws=ws)
    torch.cuda.synchronize()
    assert_close("C", to_np(c), a.astype(np.float64) @ b.astype(np.float64) + bias[None, :], "bf16")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 64), (4096, 4096, 128), (4096, 4096, 200), (4000, 4104, 1032)])
def test_gemm_large_tiles_layouts_short_and_ragged_k(ta, tb, M, N, K):
    """The 256x256-tile kernel in every operand layout with one, two and a
    ragged number of 64-deep K tiles (the loop's prologue, its last tile and
    the loads it skips past the end of K), and ragged M and N (272 tiles)."""
    print(f"gemm large ta={ta} tb={tb} {M}x{N}x{K}", flush=True)
    a = inputs(17, (K, M) if ta else (M, K), "bf16")
    b = inputs(18, (N, K) if tb else (K, N), "bf16")
    bias = inputs(19, (N,), "bf16")
    c = empty((M, N), "bf16")
    ws = empty_bytes(tst.gemm_workspace_bytes(tst.BF16, M, N, K))
    tst.gemm(to_gpu(a, "bf16"), to_gpu(b, "bf16"), c, bool(ta), bool(tb), bias=to_gpu(bias, "bf16"), ws=ws)
    torch.cuda.synchronize()
    A = a.astype(np.float64).T if ta else a.astype(np.float64)
    B = b.astype(np.float64).T if tb else b.astype(np.float64)
    assert_close("C", to_np(c), A @ B + bias.astype(np.float64)[None, :], "bf16")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(4096, 8192, 64), (4104, 8200, 136)])
def test_gemm_persistent_several_items_per_workgroup(ta, tb, M, N, K):
    """The persistent 256x256-tile kernel with two or three work items per
    workgroup (512 tiles; 17 x 33 = 561 ragged tiles): each item's first K
    tiles are loaded while the previous item's epilogue runs, and every item
    starts from zeroed accumulators and its own per-lane offsets."""
    print(f"gemm persistent ta={ta} tb={tb} {M}x{N}x{K}", flush=True)
    a = inputs(27, (K, M) if ta else (M, K), "bf16")
    b = inputs(28, (N, K) if tb else (K, N), "bf16")
    bias = inputs(29, (N,), "bf16")
    c = empty((M, N), "bf16")
    ws = empty_bytes(tst.gemm_workspace_bytes(tst.BF16, M, N, K))
    tst.gemm(to_gpu(a, "bf16"), to_gpu(b, "bf16"), c, bool(ta), bool(tb), bias=to_gpu(bias, "bf16"), ws=ws)
    torch.cuda.synchronize()
    A = a.astype(np.float64).T if ta else a.astype(np.float64)
    B = b.astype(np.float64).T if tb else b.astype(np.float64)
    assert_close("C", to_np(c), A @ B + bias.astype(np.float64)[None, :], "bf16")


# ------------------------------------------------------------------ LayerNorm
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(64, 256), (37, 4096), (9, 20480), (5, 264)])
def test_layernorm(dtype, rows, cols):
    print(f"layernorm {dtype} {rows}x{cols}", flush=True)
    x = inputs(21, (rows, cols), dtype, 2.0, 0.5)
    g = inputs(22, (cols,), dtype, 0.1, 1.0)
    b = inputs(23, (cols,), dtype, 0.1)
    gy = inputs(24, (rows, cols), dtype)
    xg, gg, bg, gyg = (to_gpu(v, dtype) for v in (x, g, b, gy))
    y = empty((rows, cols), dtype)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    tst.layernorm_fwd(xg, gg, bg, 1e-5, y, mean, rstd)
    dx = empty((rows, cols), dtype)
    dgam = empty((cols,), dtype)
    dbet = empty((cols,), dtype)
    ws = empty_bytes(tst.layernorm_bwd_workspace_bytes(rows, cols))
    tst.layernorm_bwd(gyg, xg, mean, rstd, gg, dx, dgam, dbet, ws)
    torch.cuda.synchronize()
    X = x.astype(np.float64)
    ry, rmean, rrstd, xhat = OL.layernorm_fwd(X, g.astype(np.float64), b.astype(np.float64), 1e-5)
    assert_close("y", to_np(y), ry, dtype)
    assert rel_inf(to_np(mean), rmean) < 1e-5
    assert rel_inf(to_np(rstd), rrstd) < 1e-5
    rdx, rdg, rdb = OL.layernorm_bwd(gy.astype(np.float64), xhat, rrstd, g.astype(np.float64))
    assert_close("dx", to_np(dx), rdx, dtype)
    assert_close("dgamma", to_np(dgam), rdg, dtype)
    assert_close("dbeta", to_np(dbet), rdb, dtype)


# ------------------------------------------------------------------ attention
# The shortest sequence (128: the walks of one and two 64-row tiles, so the
# prologues' second tile is issued for some blocks and not for others) at an
# odd batch, and a longer walk than the ring holds at every head size.
ATTN_CASES = [("f32", 2, 128, 2, 64), ("f32", 1, 256, 2, 128), ("bf16", 2, 128, 2, 64),
              ("bf16", 1, 256, 3, 128), ("bf16", 1, 384, 2, 160), ("bf16", 2, 256, 1, 160),
              ("f32", 3, 128, 1, 64), ("bf16", 3, 128, 2, 160), ("bf16", 1, 640, 2, 128), ("bf16", 1, 640, 1, 64)]


@pytest.mark.parametrize("dtype,batch,seq,heads,d", ATTN_CASES)
def test_attention(dtype, batch, seq, heads, d):
    print(f"attention {dtype} b={batch} s={seq} h={heads} d={d}", flush=True)
    T = batch * seq
    go = inputs(32, (T, heads * d), dtype)
    if dtype == "bf16":
        # the bf16 path keeps Q and K in fp16, V in bf16
        qkv, bits = qkv_bits(randn(31, (T, 3 * heads * d)), 2 * heads * d)
        qg = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        qkv = inputs(31, (T, 3 * heads * d), dtype)
        qg = to_gpu(qkv, dtype)
    o = empty((T, heads * d), dtype)
    lse = torch.empty((heads, T), dtype=torch.float32, device="cuda")
    tst.attention_fwd(qg, o, lse, batch, seq, heads, d)
    dq = empty((T, 3 * heads * d), dtype)
    ws = empty_bytes(tst.attention_bwd_workspace_bytes(batch, seq, heads))
    tst.attention_bwd(qg, o, lse, to_gpu(go, dtype), dq, ws, batch, seq, heads, d)
    torch.cuda.synchronize()
    ro, p, rlse = OL.attention_fwd(qkv.astype(np.float64), batch, seq, heads, d)
    assert_close("o", to_np(o), ro, dtype)
    # lse [b, nh, s] -> [nh, b*s]
    rl = rlse.transpose(1, 0, 2).reshape(heads, T)
    # lse is a float32 output formed from bf16-exact scores: an error in the
    # max shift or the log base would show far above this bound
    assert np.max(np.abs(to_np(lse) - rl) / (1.0 + np.abs(rl))) < 1e-4
    # backward from the GPU's own (rounded) O: the oracle uses its P and the given dO
    rdq = OL.attention_bwd(qkv.astype(np.float64), p, go.astype(np.float64), batch, seq, heads, d)
    w = heads * d
    for name, sl in (("dq", slice(0, w)), ("dk", slice(w, 2 * w)), ("dv", slice(2 * w, 3 * w))):
        assert_close(name, to_np(dq)[:, sl], rdq[:, sl], dtype)


# ------------------------------------------------------------------ streaming kernels
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 3])
def test_reduce_partials(dtype, n):
    rows, cols = 67, 264
    parts = [inputs(40 + j, (rows, cols), dtype) for j in range(n)]
    res = inputs(50, (rows, cols), dtype)
    bias = inputs(51, (cols,), dtype)
    out = empty((rows, cols), dtype)
    tst.reduce_partials([to_gpu(p, dtype) for p in parts], out, to_gpu(res, dtype), to_gpu(bias, dtype))
    out2 = empty((rows, cols), dtype)
    tst.reduce_partials([to_gpu(p, dtype) for p in parts], out2)
    torch.cuda.synchronize()
    ref = OL.reduce_partials([p.astype(np.float64) for p in parts], res.astype(np.float64), bias.astype(np.float64))
    assert_close("out", to_np(out), ref, dtype)
    ref2 = OL.reduce_partials([p.astype(np.float64) for p in parts], np.zeros((rows, cols)), None)
    assert_close("out_nores", to_np(out2), ref2, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,p", [(3, 24, 0.1), (67, 264, 0.3), (33, 20480, 0.1), (16, 64, 0.0)])
def test_reduce_partials_dropout(dtype, rows, cols, p):
    """Dropout after the partial sum: the mask (Philox4x64-10 on the GPU,
    independently in the oracle) must match element for element -- dropped
    elements are exactly the residual -- and the kept values to the dtype's
    tolerance. 3 x 24 ends in half a generator block."""
    p = float(np.float32(p))           # the rate as the library receives it
    seed, site = 0x5EED0000DEADBEEF, 7
    parts = [inputs(140 + j, (rows, cols), dtype) for j in range(2)]
    res = inputs(150, (rows, cols), dtype)
    bias = inputs(151, (cols,), dtype)
    out = empty((rows, cols), dtype)
    tst.reduce_partials_dropout([to_gpu(q, dtype) for q in parts], out, p, seed, site, to_gpu(res, dtype),
                                to_gpu(bias, dtype))
    torch.cuda.synchronize()
    got = to_np(out)
    keep = OD.mask((rows, cols), p, seed, site)
    ref = OD.dropout_sum_fwd([q.astype(np.float64) for q in parts], res.astype(np.float64), bias.astype(np.float64),
                             p, seed, site)
    assert np.array_equal(got[~keep], res.astype(np.float64)[~keep])
    assert_close("out", got, ref, dtype)
    if p == 0.0:
        assert keep.all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,p", [(3, 24, 0.5), (129, 2056, 0.1)])
def test_dropout_bwd(dtype, rows, cols, p):
    p = float(np.float32(p))
    seed, site = 12345, 3
    g = inputs(160, (rows, cols), dtype)
    dz = empty((rows, cols), dtype)
    tst.dropout_bwd(to_gpu(g, dtype), dz, p, seed, site)
    torch.cuda.synchronize()
    got = to_np(dz)
    keep = OD.mask((rows, cols), p, seed, site)
    assert np.all(got[~keep] == 0.0)
    assert_close("dz", got, OD.dropout_bwd(g.astype(np.float64), p, seed, site), dtype)
    # a different site gives a different mask
    dz2 = empty((rows, cols), dtype)
    tst.dropout_bwd(to_gpu(g, dtype), dz2, p, seed, site + 1)
    torch.cuda.synchronize()
    assert not np.array_equal(to_np(dz2) == 0.0, got == 0.0)


@pytest.mark.parametrize("n", [8, 1000003])
def test_grad_accumulate(n):
    gs = [round_f32_to_bf16(randn(60 + k, (n,), 1e-3)) for k in range(4)]
    acc = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
    for k, g in enumerate(gs):
        tst.grad_accumulate(to_gpu(g, "bf16"), acc, overwrite=(k == 0))
    torch.cuda.synchronize()
    ref = OA.accumulate([g.astype(np.float64) for g in gs])
    assert rel_inf(to_np(acc), ref) < 1e-6


def _adam_run(n, cfg, master, m, v, acc):
    mg, mm, vv, ag = (torch.from_numpy(a.astype(np.float32)).cuda() for a in (master, m, v, acc))
    w = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    stats = torch.zeros(3, dtype=torch.float32, device="cuda")
    ws = empty_bytes(tst.adam_workspace_bytes(n))
    c = tst.AdamCfg(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.max_grad_norm,
                    cfg.inv_loss_scale, cfg.step)
    tst.adam_step(c, mg, mm, vv, ag, w, stats, ws)
    torch.cuda.synchronize()
    return to_np(mg), to_np(mm), to_np(vv), to_np(w), to_np(stats)


@pytest.mark.parametrize("n", [5, 4096, 1000003])
@pytest.mark.parametrize("max_norm", [1.0, 0.0, 1e6])
def test_adam_step(n, max_norm):
    master = randn(70, (n,), 0.02)
    m = randn(71, (n,), 1e-3)
    v = randn(72, (n,), 1e-3) ** 2
    acc = randn(73, (n,), 1e-3) * 4
    cfg = OA.AdamConfig(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, max_grad_norm=max_norm,
                        inv_loss_scale=2.0 ** -3, step=100)
    gp, gm, gv, gw, st = _adam_run(n, cfg, master, m, v, acc)
    rp, rm, rv, rw, (norm, coef, inf) = OA.adam_step(master.astype(np.float64), m.astype(np.float64),
                                                    v.astype(np.float64), acc.astype(np.float64), cfg)
    assert not inf and st[2] == 0.0
    assert abs(st[0] - norm) <= 1e-5 * norm
    assert abs(st[1] - coef) <= 1e-5
    # updates (delta p) to 1e-4 relative of the largest step, moments to 1e-5
    assert rel_inf(gp - master, rp - master) < 1e-4
    assert rel_inf(gm, rm) < 1e-5
    assert rel_inf(gv, rv) < 1e-5
    assert_bf16_copy(gw, gp, rw, rp)


@pytest.mark.parametrize("n", [0, 5, 1000003])
def test_adam_stream_reference_leaves_values(n):
    """The measurement reference moves the update's bytes and changes nothing:
    master, m and v are written back bit for bit, the bf16 copy is the
    round-to-nearest-even rounding of master."""
    master = randn(80, (n,), 0.02)
    m = randn(81, (n,), 1e-3)
    v = randn(82, (n,), 1e-3) ** 2
    g = randn(83, (n,), 1e-3)
    tm, tmm, tv, tg = (to_gpu(a, "f32") for a in (master, m, v, g))
    w = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    tst.adam_stream_reference(tm, tmm, tv, tg, w)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(tm), master.astype(np.float64))
    assert np.array_equal(to_np(tmm), m.astype(np.float64))
    assert np.array_equal(to_np(tv), v.astype(np.float64))
    assert np.array_equal(to_np(tg), g.astype(np.float64))
    assert np.array_equal(to_np(w), round_f32_to_bf16(master).astype(np.float64))


@pytest.mark.parametrize("n,mb", [(5, 1), (4096, 3), (1000003, 4)])
def test_accumulate_norm_then_update(n, mb):
    """The norm folded into the last micro-batch's accumulation, then the update
    on it: the same accumulator and step as accumulate + adam_step, checked
    against the oracle like test_adam_step."""
    master = randn(90, (n,), 0.02)
    m = randn(91, (n,), 1e-3)
    v = randn(92, (n,), 1e-3) ** 2
    gs = [round_f32_to_bf16(randn(93 + k, (n,), 1e-3)) for k in range(mb)]
    cfg = OA.AdamConfig(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, max_grad_norm=2e-4 * np.sqrt(n),
                        inv_loss_scale=2.0 ** -2, step=7)
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = empty_bytes(tst.adam_workspace_bytes(n))
    for k, g in enumerate(gs):
        if k < mb - 1:
            tst.grad_accumulate(to_gpu(g, "bf16"), acc, overwrite=(k == 0))
        else:
            tst.grad_accumulate_norm(to_gpu(g, "bf16"), acc, k == 0, cfg.inv_loss_scale, ws)
    mg, mm, vv = (torch.from_numpy(a.astype(np.float32)).cuda() for a in (master, m, v))
    w = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    stats = torch.zeros(3, dtype=torch.float32, device="cuda")
    c = tst.AdamCfg(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.max_grad_norm,
                    cfg.inv_loss_scale, cfg.step)
    tst.adam_update(c, mg, mm, vv, acc, w, stats, ws)
    torch.cuda.synchronize()
    a = to_np(acc)
    assert rel_inf(a, OA.accumulate([g.astype(np.float64) for g in gs])) < 1e-6
    rp, rm, rv, rw, (norm, coef, inf) = OA.adam_step(master.astype(np.float64), m.astype(np.float64),
                                                    v.astype(np.float64), a, cfg)
    st = to_np(stats)
    assert not inf and st[2] == 0.0
    assert abs(st[0] - norm) <= 1e-6 * norm
    assert abs(st[1] - coef) <= 1e-6
    assert rel_inf(to_np(mg) - master, rp - master) < 1e-4
    assert rel_inf(to_np(mm), rm) < 1e-5
    assert rel_inf(to_np(vv), rv) < 1e-5
    assert_bf16_copy(to_np(w), to_np(mg), rw, rp)


def test_accumulate_norm_nonfinite_skips():
    n = 4099
    master = randn(95, (n,), 0.02)
    g = round_f32_to_bf16(randn(96, (n,), 1e-3))
    g[17] = np.inf
    acc = torch.zeros(n, dtype=torch.float32, device="cuda")
    ws = empty_bytes(tst.adam_workspace_bytes(n))
    tst.grad_accumulate_norm(to_gpu(g, "bf16"), acc, False, 1.0, ws)
    mg = torch.from_numpy(master).cuda()
    mm = torch.zeros(n, device="cuda")
    vv = torch.zeros(n, device="cuda")
    stats = torch.zeros(3, device="cuda")
    tst.adam_update(tst.AdamCfg(1e-3, 0.9, 0.95, 1e-8, 1.0, 1.0, 1.0, 1), mg, mm, vv, acc, None, stats, ws)
    torch.cuda.synchronize()
    assert to_np(stats)[2] == 1.0
    assert np.array_equal(to_np(mg), master.astype(np.float64))
    assert not to_np(mm).any() and not to_np(vv).any()


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_adam_nonfinite_skips(bad):
    n = 4099
    master = randn(80, (n,), 0.02)
    m = randn(81, (n,), 1e-3)
    v = randn(82, (n,), 1e-3) ** 2
    acc = randn(83, (n,), 1e-3)
    acc[n - 2] = bad
    cfg = OA.AdamConfig(step=3)
    gp, gm, gv, gw, st = _adam_run(n, cfg, master, m, v, acc)
    assert st[2] == 1.0
    assert np.array_equal(gp, master.astype(np.float64))
    assert np.array_equal(gm, m.astype(np.float64)) and np.array_equal(gv, v.astype(np.float64))


def test_adam_constant_gradient_closed_form():
    """From zero state with constant g, each step moves p by -lr g/(|g|+eps) (Adam closed form)."""
    n = 1024
    g = np.where(np.arange(n) % 2 == 0, 3e-3, -5e-4).astype(np.float32)
    p0 = randn(84, (n,), 0.02)
    mg = torch.from_numpy(p0.copy()).cuda()
    mm = torch.zeros(n, device="cuda")
    vv = torch.zeros(n, device="cuda")
    ag = torch.from_numpy(g).cuda()
    stats = torch.zeros(3, device="cuda")
    ws = empty_bytes(tst.adam_workspace_bytes(n))
    for t in range(1, 4):
        tst.adam_step(tst.AdamCfg(1e-3, 0.9, 0.95, 1e-8, 0.0, 0.0, 1.0, t), mg, mm, vv, ag, None, stats, ws)
    torch.cuda.synchronize()
    want = p0.astype(np.float64) - 3 * 1e-3 * g / (np.abs(g) + 1e-8)
    assert rel_inf(to_np(mg) - p0, want - p0) < 1e-5
