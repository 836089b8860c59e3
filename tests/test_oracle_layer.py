"""Pins of the layer oracle to things other than itself.

* brute force: a pure-Python loop version of the whole layer on a tiny shape;
* the slicing invariant of the Megatron example in the STRONGHOLD slides
  (slides 7-8): residual + bias + sum of slice partials equals the unsliced
  layer, forward and backward, for t = 2, 4, 8;
* finite differences of L = <Out, G> for every parameter tensor and the input;
* special cases of attention, GeLU and LayerNorm with closed forms.
"""
import math

import numpy as np
import pytest

from oracle import layer as L


def rng(seed):
    return np.random.default_rng(seed)


def make_full(sh: L.LayerShape, seed=0, scale=0.3):
    r = rng(seed)
    p = {}
    for k, s in L.full_param_shapes(sh).items():
        if k in ("ln1_g", "ln2_g"):
            p[k] = 1.0 + 0.2 * r.standard_normal(s)
        else:
            p[k] = scale * r.standard_normal(s)
    return p


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

def brute_layer(sh, x, p):
    """Whole pre-LN layer with explicit Python loops (no numpy algebra)."""
    T, h, f, H = sh.tokens, sh.hidden, sh.ffn, sh.heads
    d = h // H

    def ln(rows, g, b):
        out = []
        for row in rows:
            mu = sum(row) / h
            var = sum((v - mu) ** 2 for v in row) / h
            rs = 1.0 / math.sqrt(var + sh.eps)
            out.append([g[j] * (row[j] - mu) * rs + b[j] for j in range(h)])
        return out

    def mm(a, w, bias=None):
        n = len(w[0])
        return [[sum(a[i][k] * w[k][j] for k in range(len(w))) + (bias[j] if bias is not None else 0.0)
                 for j in range(n)] for i in range(len(a))]

    xl = x.tolist()
    y1 = ln(xl, p["ln1_g"].tolist(), p["ln1_b"].tolist())
    qkv = mm(y1, p["w_qkv"].tolist(), p["b_qkv"].tolist())
    o = [[0.0] * h for _ in range(T)]
    for b in range(sh.batch):
        for n in range(H):
            for r in range(sh.seq):
                tr = b * sh.seq + r
                q = [qkv[tr][0 * h + n * d + e] for e in range(d)]
                scores = []
                for c in range(r + 1):
                    tc = b * sh.seq + c
                    k = [qkv[tc][1 * h + n * d + e] for e in range(d)]
                    scores.append(sum(q[e] * k[e] for e in range(d)) / math.sqrt(d))
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                z = sum(ex)
                for e in range(d):
                    o[tr][n * d + e] = sum(ex[c] / z * qkv[b * sh.seq + c][2 * h + n * d + e]
                                           for c in range(r + 1))
    att = mm(o, p["w_o"].tolist(), p["b_o"].tolist())
    x1 = [[xl[i][j] + att[i][j] for j in range(h)] for i in range(T)]
    y2 = ln(x1, p["ln2_g"].tolist(), p["ln2_b"].tolist())
    u = mm(y2, p["w_a"].tolist(), p["b_a"].tolist())
    a = [[0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in row] for row in u]
    z = mm(a, p["w_b"].tolist(), p["b_b"].tolist())
    return np.array([[x1[i][j] + z[i][j] for j in range(h)] for i in range(T)])


@pytest.mark.parametrize("tp", [1, 2])
def test_brute_force_forward(tp):
    sh = L.LayerShape(batch=2, seq=3, hidden=4, heads=2, ffn=6, tp=tp)
    p = make_full(sh, seed=1)
    x = rng(2).standard_normal((sh.tokens, sh.hidden))
    out, _ = L.layer_fwd(sh, x, p)
    ref = brute_layer(sh, x, p)
    assert rel(out, ref) < 1e-12


def test_rows_forward_against_brute_force():
    """The row-sampled unsliced forward equals the brute-force layer on those rows."""
    sh = L.LayerShape(batch=2, seq=3, hidden=4, heads=2, ffn=6, tp=1)
    p = make_full(sh, seed=1)
    x = rng(2).standard_normal((sh.tokens, sh.hidden))
    ref = brute_layer(sh, x, p)
    for b, rows in ((0, [2]), (1, [0, 2]), (1, [1])):
        got = L.layer_fwd_rows(sh, x[b * sh.seq:(b + 1) * sh.seq], p, rows)
        assert rel(got, ref[[b * sh.seq + r for r in rows]]) < 1e-12


@pytest.mark.parametrize("tp", [1, 8])
def test_rows_forward_against_layer(tp):
    """...and the (sliced) full oracle layer on sampled rows of every sequence."""
    sh = L.LayerShape(batch=3, seq=16, hidden=64, heads=8, ffn=128, tp=tp)
    p = make_full(sh, seed=11)
    x = rng(12).standard_normal((sh.tokens, sh.hidden))
    out, _ = L.layer_fwd(sh, x, p)
    for b in range(sh.batch):
        rows = sorted({0, sh.seq - 1, *rng(20 + b).integers(0, sh.seq, size=4).tolist()})
        got = L.layer_fwd_rows(sh, x[b * sh.seq:(b + 1) * sh.seq], p, rows)
        assert rel(got, out[[b * sh.seq + r for r in rows]]) < 1e-12


# --------------------------------------------------------------------------
# slicing invariant (forward and backward)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("tp", [2, 4, 8])
def test_slicing_invariant(tp):
    base = L.LayerShape(batch=2, seq=8, hidden=32, heads=8, ffn=64, tp=1)
    sliced = L.LayerShape(batch=2, seq=8, hidden=32, heads=8, ffn=64, tp=tp)
    p = make_full(base, seed=3)
    x = rng(4).standard_normal((base.tokens, base.hidden))
    g = rng(5).standard_normal((base.tokens, base.hidden))
    out1, st1 = L.layer_fwd(base, x, p)
    outt, stt = L.layer_fwd(sliced, x, p)
    assert rel(outt, out1) < 1e-12
    dx1, g1 = L.layer_bwd(base, g, p, st1)
    dxt, gt = L.layer_bwd(sliced, g, p, stt)
    assert rel(dxt, dx1) < 1e-12
    for k in L.FULL_KEYS:
        assert rel(gt[k], g1[k]) < 1e-12, k


def test_slices_partition_weights():
    """Every weight column/row belongs to exactly one slice (no overlap, nothing dropped)."""
    sh = L.LayerShape(batch=1, seq=2, hidden=48, heads=6, ffn=96, tp=3)
    cols = np.concatenate([L.qkv_columns(sh, i) for i in range(sh.tp)])
    assert sorted(cols.tolist()) == list(range(3 * sh.hidden))
    # q, k and v columns of a head stay together inside one slice
    for i in range(sh.tp):
        c = L.qkv_columns(sh, i)
        heads = {(cc % sh.hidden) // sh.head_dim for cc in c}
        assert heads == set(range(i * sh.local_heads, (i + 1) * sh.local_heads))


def test_row_bias_added_once():
    """Row-sliced biases enter the output once, not once per slice."""
    sh = L.LayerShape(batch=1, seq=4, hidden=16, heads=4, ffn=32, tp=4)
    p = make_full(sh, seed=6)
    x = rng(7).standard_normal((sh.tokens, sh.hidden))
    out, _ = L.layer_fwd(sh, x, p)
    p2 = dict(p)
    p2["b_b"] = p["b_b"] + 1.0
    out2, _ = L.layer_fwd(sh, x, p2)
    assert np.allclose(out2 - out, 1.0, atol=1e-12)


# --------------------------------------------------------------------------
# finite differences
# --------------------------------------------------------------------------

FD_SHAPE = L.LayerShape(batch=2, seq=5, hidden=12, heads=3, ffn=24, tp=3)


def _fd_setup():
    p = make_full(FD_SHAPE, seed=8)
    x = rng(9).standard_normal((FD_SHAPE.tokens, FD_SHAPE.hidden))
    g = rng(10).standard_normal((FD_SHAPE.tokens, FD_SHAPE.hidden))
    _, st = L.layer_fwd(FD_SHAPE, x, p)
    dx, grads = L.layer_bwd(FD_SHAPE, g, p, st)
    return p, x, g, dx, grads


@pytest.mark.parametrize("name", ("x",) + L.FULL_KEYS)
def test_finite_differences_directional(name):
    p, x, g, dx, grads = _fd_setup()
    delta = 1e-5
    u = rng(sum(map(ord, name))).standard_normal(x.shape if name == "x" else p[name].shape)

    def loss_at(s):
        if name == "x":
            return L.layer_loss(FD_SHAPE, x + s * u, p, g)
        q = dict(p)
        q[name] = p[name] + s * u
        return L.layer_loss(FD_SHAPE, x, q, g)

    fd = (loss_at(delta) - loss_at(-delta)) / (2 * delta)
    an = float(((dx if name == "x" else grads[name]) * u).sum())
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (fd, an)


@pytest.mark.parametrize("name", ("x", "w_qkv", "w_o", "w_a", "w_b", "b_qkv", "ln1_g", "ln2_b"))
def test_finite_differences_elementwise(name):
    p, x, g, dx, grads = _fd_setup()
    delta = 1e-5
    arr = x if name == "x" else p[name]
    an_all = dx if name == "x" else grads[name]
    r = rng(11)
    for _ in range(8):
        idx = tuple(int(r.integers(0, s)) for s in arr.shape)

        def loss_at(s):
            a2 = arr.copy()
            a2[idx] += s
            if name == "x":
                return L.layer_loss(FD_SHAPE, a2, p, g)
            q = dict(p)
            q[name] = a2
            return L.layer_loss(FD_SHAPE, x, q, g)

        fd = (loss_at(delta) - loss_at(-delta)) / (2 * delta)
        an = float(an_all[idx])
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-2), (name, idx, fd, an)


# --------------------------------------------------------------------------
# attention special cases
# --------------------------------------------------------------------------

def test_attention_seq1_is_v():
    nh, d = 3, 4
    qkv = rng(12).standard_normal((5, 3 * nh * d))     # batch 5 of length-1 sequences
    o, p, lse = L.attention_fwd(qkv, 5, 1, nh, d)
    assert np.array_equal(o, qkv[:, 2 * nh * d:])
    assert np.all(p == 1.0)


def test_attention_zero_query_is_prefix_mean():
    nh, d, s = 2, 4, 7
    qkv = rng(13).standard_normal((s, 3 * nh * d))
    qkv[:, :nh * d] = 0.0
    o, _, lse = L.attention_fwd(qkv, 1, s, nh, d)
    v = qkv[:, 2 * nh * d:]
    pref = np.cumsum(v, axis=0) / np.arange(1, s + 1)[:, None]
    assert np.max(np.abs(o - pref)) < 1e-14
    # all scores 0: lse = log(number of visible keys)
    assert np.max(np.abs(lse[0] - np.log(np.arange(1, s + 1))[None, :])) < 1e-14


def test_attention_causal_and_normalised():
    nh, d, s = 2, 8, 9
    qkv = rng(14).standard_normal((2 * s, 3 * nh * d))
    o, p, lse = L.attention_fwd(qkv, 2, s, nh, d)
    assert np.max(np.abs(p.sum(axis=-1) - 1.0)) < 1e-15
    assert np.all(p[..., np.triu_indices(s, 1)[0], np.triu_indices(s, 1)[1]] == 0.0)
    for r in range(s - 1):
        q2 = qkv.copy()
        q2[r + 1:s] += rng(15 + r).standard_normal((s - r - 1, qkv.shape[1]))
        o2, _, _ = L.attention_fwd(q2, 2, s, nh, d)
        assert np.array_equal(o2[:r + 1], o[:r + 1])
        assert np.array_equal(o2[s:], o[s:])      # the other sequence is untouched


def test_attention_scores_scaled_by_sqrt_d():
    """Two keys; the softmax weight of key 1 for query 1 is sigmoid((s11 - s10)/sqrt(d))."""
    nh, d, s = 1, 16, 2
    qkv = rng(16).standard_normal((s, 3 * d))
    _, p, _ = L.attention_fwd(qkv, 1, s, nh, d)
    q1 = qkv[1, :d]
    k0, k1 = qkv[0, d:2 * d], qkv[1, d:2 * d]
    want = 1.0 / (1.0 + math.exp(-(q1 @ k1 - q1 @ k0) / math.sqrt(d)))
    assert abs(p[0, 0, 1, 1] - want) < 1e-15


def test_attention_bwd_finite_differences():
    nh, d, s, b = 2, 3, 4, 2
    qkv = rng(17).standard_normal((b * s, 3 * nh * d))
    go = rng(18).standard_normal((b * s, nh * d))
    _, p, _ = L.attention_fwd(qkv, b, s, nh, d)
    dqkv = L.attention_bwd(qkv, p, go, b, s, nh, d)
    delta = 1e-6
    for idx in [(0, 0), (3, 5), (5, 7), (7, 17), (6, 11), (2, 14)]:
        qp = qkv.copy(); qp[idx] += delta
        qm = qkv.copy(); qm[idx] -= delta
        fd = ((L.attention_fwd(qp, b, s, nh, d)[0] * go).sum()
              - (L.attention_fwd(qm, b, s, nh, d)[0] * go).sum()) / (2 * delta)
        assert abs(fd - dqkv[idx]) < 1e-7 * max(1.0, abs(fd)), idx


# --------------------------------------------------------------------------
# GeLU and LayerNorm closed forms
# --------------------------------------------------------------------------

def test_gelu_identities():
    u = np.linspace(-8, 8, 1601)
    assert np.max(np.abs(L.gelu(u) - L.gelu(-u) - u)) < 1e-14
    assert L.gelu(np.array(0.0)) == 0.0
    assert abs(L.gelu_grad(np.array(0.0)) - 0.5) < 1e-16
    big = np.array([10.0, 20.0, 40.0])
    assert np.max(np.abs(L.gelu(big) - big)) < 1e-15 * 40
    # textbook value of the normal CDF: Phi(1) = 0.8413447460685429...
    assert abs(L.gelu(np.array(1.0)) - 0.8413447460685429) < 1e-15
    # Phi(-1.959963984540054) = 0.025 (two-sided 95% quantile)
    z = -1.959963984540054
    assert abs(L.gelu(np.array(z)) / z - 0.025) < 1e-14


def test_gelu_grad_matches_difference():
    u = np.linspace(-6, 6, 97)
    dl = 1e-6
    fd = (L.gelu(u + dl) - L.gelu(u - dl)) / (2 * dl)
    assert np.max(np.abs(fd - L.gelu_grad(u))) < 1e-8


def test_layernorm_moments_and_invariance():
    x = rng(19).standard_normal((6, 40)) * 3.0 + 1.5
    h = x.shape[1]
    y, mean, rstd, xhat = L.layernorm_fwd(x, np.ones(h), np.zeros(h), 1e-5)
    var = x.var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-14
    assert np.max(np.abs(y.var(axis=1) - var / (var + 1e-5))) < 1e-14
    y2, _, _, _ = L.layernorm_fwd(2.5 * x - 7.0, np.ones(h), np.zeros(h), 0.0)
    y3, _, _, _ = L.layernorm_fwd(x, np.ones(h), np.zeros(h), 0.0)
    assert np.max(np.abs(y2 - y3)) < 1e-13


def test_layernorm_bwd_finite_differences():
    r = rng(20)
    x = r.standard_normal((4, 10))
    gam = 1 + 0.3 * r.standard_normal(10)
    bet = 0.3 * r.standard_normal(10)
    gy = r.standard_normal((4, 10))
    _, _, rstd, xhat = L.layernorm_fwd(x, gam, bet, 1e-5)
    dx, dg, db = L.layernorm_bwd(gy, xhat, rstd, gam)
    delta = 1e-6

    def f(xx, gg, bb):
        return (L.layernorm_fwd(xx, gg, bb, 1e-5)[0] * gy).sum()

    for idx in [(0, 0), (1, 5), (3, 9), (2, 3)]:
        xp = x.copy(); xp[idx] += delta
        xm = x.copy(); xm[idx] -= delta
        assert abs((f(xp, gam, bet) - f(xm, gam, bet)) / (2 * delta) - dx[idx]) < 1e-8
    for j in [0, 4, 9]:
        gp = gam.copy(); gp[j] += delta
        gm = gam.copy(); gm[j] -= delta
        assert abs((f(x, gp, bet) - f(x, gm, bet)) / (2 * delta) - dg[j]) < 1e-8
        bp = bet.copy(); bp[j] += delta
        bm = bet.copy(); bm[j] -= delta
        assert abs((f(x, gam, bp) - f(x, gam, bm)) / (2 * delta) - db[j]) < 1e-8


# --------------------------------------------------------------------------
# diagnostic mode: the tensors a bf16 library keeps between its steps rounded
# --------------------------------------------------------------------------

def _diag_setup():
    sh = L.LayerShape(batch=2, seq=8, hidden=32, heads=4, ffn=64, tp=2)
    full = make_full(sh, seed=40, scale=0.3)
    x = rng(41).standard_normal((sh.tokens, sh.hidden))
    return sh, full, x


def test_diagnostic_mode_identity_store_is_the_definition():
    sh, full, x = _diag_setup()
    for fwd, sl in ((L.attn_half_fwd, L.attn_slice), (L.mlp_half_fwd, L.mlp_slice)):
        p = sl(sh, full, 1)
        a, sa = fwd(sh, x, p)
        b, sb = fwd(sh, x, p, store=lambda t: t)
        assert np.array_equal(a, b)
        for k in sa:
            assert np.array_equal(sa[k], sb[k]), k


def test_diagnostic_mode_rounds_only_the_kept_tensors():
    """With bf16 rounding, LN output, QKV, O (attention) and LN output, U, Y
    (MLP) are bf16 values; the LayerNorm statistics are not rounded; Y is the
    rounding of GeLU of the unrounded U; and the partial moves away from the
    definition by no more than a few bf16 half-ulps carried through two
    products (well below 2^-4 relative), but does move."""
    from oracle.bf16 import round_to_bf16
    sh, full, x = _diag_setup()
    for fwd, sl, kept in ((L.attn_half_fwd, L.attn_slice, ("ln_out", "qkv", "o")),
                          (L.mlp_half_fwd, L.mlp_slice, ("ln_out", "u", "y"))):
        p = sl(sh, full, 0)
        exact, se = fwd(sh, x, p)
        diag, sd = fwd(sh, x, p, store=round_to_bf16)
        for k in kept:
            assert np.array_equal(round_to_bf16(sd[k]), sd[k]), k
            assert not np.array_equal(sd[k], se[k]), k
            assert rel(sd[k], se[k]) <= 2.0 ** -8 * 4, k
        assert np.array_equal(sd["rstd"], se["rstd"]) and np.array_equal(sd["mean"], se["mean"])
        assert not np.array_equal(round_to_bf16(sd["rstd"]), sd["rstd"])
        if "u" in kept:
            u_exact = sd["ln_out"] @ p["w_in"] + p["b_in"][None, :]
            assert np.array_equal(sd["y"], round_to_bf16(L.gelu(u_exact)))
        e = rel(diag, exact)
        assert 0.0 < e < 2.0 ** -4, e
