"""Pins of the dropout oracle to things other than itself.

* Philox4x64-10 against numpy's own Philox bit generator (the same published
  generator, an independent implementation): numpy increments its 256-bit
  counter before each block, so a block at counter c is the first four raw
  outputs of a generator started at c - 1;
* the vector and the scalar (Python integer) forms agree;
* keep fraction of the mask within 5 sigma of the exact keep probability
  1 - thr/65536, for several rates; p = 0 keeps everything with scale 1;
* the forward at p = 0 equals the plain partial sum; the backward is the
  gradient of <out, g> with respect to the dropped tensor (finite differences
  are exact for this linear map, so it is checked at 1e-12);
* different sites give (statistically) independent masks.
"""
import numpy as np
import pytest

from oracle import dropout as D
from oracle import layer as OL


def _numpy_block(counter, key):
    c = [int(v) for v in counter]
    # numpy adds one (with carry over the four words) before each block
    prev, borrow = [], 1
    for w in c:
        v = w - borrow
        borrow = 1 if v < 0 else 0
        prev.append(v % (1 << 64))
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(prev, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("key", [(0, 0), (1, 2), (0xFFFFFFFFFFFFFFFF, 0x0123456789ABCDEF), (42, 7)])
def test_philox_matches_numpy(key):
    counters = [[1, 0, 0, 0], [2, 0, 0, 0], [12345, 0, 0, 0], [(1 << 63) + 3, 0, 0, 0],
                [0, 1, 0, 0], [5, 6, 7, 8], [0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 3, 0]]
    got = D.philox4x64(np.array(counters, dtype=np.uint64), key)
    for c, g in zip(counters, got):
        ref = _numpy_block(c, key)
        assert [int(v) for v in g] == ref, (c, key)
        assert D.philox4x64_scalar(c, key) == ref


def test_draw_layout_follows_blocks():
    """Element e takes bits 16*(e%4).. of word (e%16)//4 of the block at counter e//16."""
    d = D.draws16(40, 9, 3)
    for e in (0, 5, 15, 16, 31, 39):
        w = D.philox4x64_scalar([e // 16, 0, 0, 0], (9, 3))[(e % 16) // 4]
        assert int(d[e]) == (w >> (16 * (e % 4))) & 0xFFFF


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction(p):
    n = 1 << 20
    keep = D.mask((n,), p, seed=1234, site=5)
    q = 1.0 - D.threshold(p) / 65536.0
    assert abs(keep.mean() - q) <= 5.0 * np.sqrt(q * (1 - q) / n)
    assert D.keep_scale(p) == pytest.approx(1.0 / q, rel=1e-15)


def test_rate_zero_is_identity():
    r = np.random.default_rng(1)
    parts = [r.standard_normal((16, 24)) for _ in range(3)]
    res = r.standard_normal((16, 24))
    b = r.standard_normal(24)
    assert D.threshold(0.0) == 0 and D.keep_scale(0.0) == 1.0
    assert np.all(D.mask((16, 24), 0.0, 3, 4))
    np.testing.assert_allclose(D.dropout_sum_fwd(parts, res, b, 0.0, 3, 4), OL.reduce_partials(parts, res, b),
                               rtol=0, atol=1e-14)


def test_backward_is_gradient():
    r = np.random.default_rng(2)
    z = r.standard_normal((8, 32))
    g = r.standard_normal((8, 32))
    u = r.standard_normal((8, 32))
    p, seed, site = 0.3, 77, 11
    res = np.zeros_like(z)

    def loss(zz):
        return float((D.dropout_sum_fwd([zz], res, None, p, seed, site) * g).sum())

    fd = (loss(z + u) - loss(z - u)) / 2.0
    an = float((D.dropout_bwd(g, p, seed, site) * u).sum())
    assert abs(fd - an) <= 1e-12 * max(1.0, abs(an))
    dz = D.dropout_bwd(g, p, seed, site)
    keep = D.mask(g.shape, p, seed, site)
    assert np.all(dz[~keep] == 0.0)


def test_sites_independent():
    n = 1 << 18
    a = D.mask((n,), 0.5, 9, 0)
    b = D.mask((n,), 0.5, 9, 1)
    c = D.mask((n,), 0.5, 10, 0)
    q = 1.0 - D.threshold(0.5) / 65536.0
    for x, y in ((a, b), (a, c)):
        agree = float((x == y).mean())
        want = q * q + (1 - q) * (1 - q)
        assert abs(agree - want) <= 5.0 * np.sqrt(want * (1 - want) / n)


def test_layer_with_dropout_finite_differences():
    """With the masks fixed by (seed, sites), the layer is smooth: its input and
    weight gradients match central differences of L = <out, g>."""
    sh = OL.LayerShape(batch=1, seq=8, hidden=16, heads=2, ffn=32, tp=2)
    r = np.random.default_rng(5)
    full = {}
    for k, s in OL.full_param_shapes(sh).items():
        full[k] = (1.0 + 0.2 * r.standard_normal(s)) if k in ("ln1_g", "ln2_g") else 0.3 * r.standard_normal(s)
    x = r.standard_normal((sh.tokens, sh.hidden))
    g = r.standard_normal((sh.tokens, sh.hidden))
    p, seed = 0.25, 99
    _, st = D.layer_fwd(sh, x, full, p, seed)
    dx, ga, gm = D.layer_bwd(sh, g, st, p, seed)
    delta = 1e-5
    u = r.standard_normal(x.shape)
    fd = (D.layer_loss(sh, x + delta * u, full, g, p, seed) - D.layer_loss(sh, x - delta * u, full, g, p, seed)) \
        / (2 * delta)
    an = float((dx * u).sum())
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0)
    # weight of the MLP's second linear: slice i owns rows [i*f/t, (i+1)*f/t) of w_b
    uw = r.standard_normal(full["w_b"].shape)
    fl = sh.local_ffn

    def loss_w(s):
        q = dict(full)
        q["w_b"] = full["w_b"] + s * uw
        return D.layer_loss(sh, x, q, g, p, seed)

    fd = (loss_w(delta) - loss_w(-delta)) / (2 * delta)
    an = sum(float((gm[i]["w_out"] * uw[i * fl:(i + 1) * fl]).sum()) for i in range(sh.tp))
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0)
    # the attention output bias gradient is the column sum of the masked gradient
    assert np.allclose(ga[0]["b_out"], ga[1]["b_out"])
    # dropping changes the result (the masks are not all ones at p = 0.25)
    out_p, _ = D.layer_fwd(sh, x, full, p, seed)
    out_0, _ = OL.layer_fwd(sh, x, full)
    assert not np.allclose(out_p, out_0)
    out_z, _ = D.layer_fwd(sh, x, full, 0.0, seed)
    np.testing.assert_allclose(out_z, out_0, rtol=0, atol=1e-12)


# ---- dropout on the attention probabilities ----

def test_attention_keep_layout_follows_blocks():
    """Element (b, head, q, k) takes bits 16*(k%4).. of word q%4 of the block at
    counter (q//4, k//4, head, b)."""
    keep_p = 0.5
    thr = D.threshold(keep_p)
    m = D.attention_keep(2, [3, 5], 12, keep_p, seed=21, site=4)
    for (b, j, q, k) in ((0, 0, 0, 0), (1, 1, 11, 2), (0, 1, 7, 7), (1, 0, 4, 9), (0, 0, 10, 3)):
        head = [3, 5][j]
        w = D.philox4x64_scalar([q // 4, k // 4, head, b], (21, 4))[q % 4]
        assert bool(m[b, j, q, k]) == (((w >> (16 * (k % 4))) & 0xFFFF) >= thr)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_attention_keep_fraction(p):
    m = D.attention_keep(1, [0, 1, 2, 3], 256, p, seed=8, site=1)
    n = m.size
    q = 1.0 - D.threshold(p) / 65536.0
    assert abs(m.mean() - q) <= 5.0 * np.sqrt(q * (1 - q) / n)
    assert np.all(D.attention_keep(1, [0], 16, 0.0, 8, 1))
    # heads and sites draw independently: agreement at the rate of independent coins
    other = D.attention_keep(1, [4, 5, 6, 7], 256, p, seed=8, site=1)
    site2 = D.attention_keep(1, [0, 1, 2, 3], 256, p, seed=8, site=2)
    want = q * q + (1 - q) * (1 - q)
    for y in (other, site2):
        agree = float((m == y).mean())
        assert abs(agree - want) <= 5.0 * np.sqrt(want * (1 - want) / n)


def test_attention_dropout_rate_zero_and_expectation():
    """A mask of all ones at scale 1 is attention itself; over many seeds the
    dropped output averages to the undropped one (E[keep * scale] = 1)."""
    r = np.random.default_rng(3)
    b, s, nh, d = 1, 8, 1, 4
    qkv = r.standard_normal((b * s, 3 * nh * d))
    o0, p0, l0 = OL.attention_fwd(qkv, b, s, nh, d)
    ones = (np.ones((b, nh, s, s), dtype=bool), 1.0)
    o1, p1, l1 = OL.attention_fwd(qkv, b, s, nh, d, ones)
    assert np.array_equal(o0, o1) and np.array_equal(p0, p1) and np.array_equal(l0, l1)
    do = r.standard_normal((b * s, nh * d))
    assert np.array_equal(OL.attention_bwd(qkv, p0, do, b, s, nh, d), OL.attention_bwd(qkv, p0, do, b, s, nh, d, ones))
    p, n = 0.5, 4000
    acc = np.zeros_like(o0)
    for seed in range(n):
        drop = (D.attention_keep(b, [0], s, p, seed, 0), D.keep_scale(p))
        acc += OL.attention_fwd(qkv, b, s, nh, d, drop)[0]
    # each output is a sum of at most 8 terms keep*scale*p*v; the mean of n
    # independent draws is within a few standard errors of the expectation
    sd = np.sqrt(np.matmul(p0.reshape(s, s) ** 2, (qkv[:, 2 * nh * d:] ** 2)) * (D.keep_scale(p) - 1.0))
    assert np.all(np.abs(acc / n - o0) <= 6.0 * sd / np.sqrt(n) + 1e-12)


def test_layer_with_attention_dropout_finite_differences_and_slicing():
    """With the attention mask fixed by (seed, site), the layer is smooth: input
    and QKV-weight gradients match central differences of L = <out, g>; and the
    global head index makes the result independent of the slicing (t = 1 vs 2)."""
    r = np.random.default_rng(11)
    shapes = [OL.LayerShape(batch=2, seq=12, hidden=16, heads=4, ffn=32, tp=t) for t in (1, 2)]
    sh = shapes[1]
    full = {}
    for k, s in OL.full_param_shapes(sh).items():
        full[k] = (1.0 + 0.2 * r.standard_normal(s)) if k in ("ln1_g", "ln2_g") else 0.4 * r.standard_normal(s)
    x = r.standard_normal((sh.tokens, sh.hidden))
    g = r.standard_normal((sh.tokens, sh.hidden))
    drop = (0.3, 1234, 5)
    out2, st = OL.layer_fwd(sh, x, full, drop)
    out1, _ = OL.layer_fwd(shapes[0], x, full, drop)
    np.testing.assert_allclose(out1, out2, rtol=0, atol=1e-12)
    out0, _ = OL.layer_fwd(sh, x, full)
    assert not np.allclose(out0, out2)
    dx, grads = OL.layer_bwd(sh, g, full, st)
    delta = 1e-5
    u = r.standard_normal(x.shape)
    fd = (OL.layer_loss(sh, x + delta * u, full, g, drop) - OL.layer_loss(sh, x - delta * u, full, g, drop)) \
        / (2 * delta)
    an = float((dx * u).sum())
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0)
    uw = r.standard_normal(full["w_qkv"].shape)

    def loss_w(s):
        q = dict(full)
        q["w_qkv"] = full["w_qkv"] + s * uw
        return OL.layer_loss(sh, x, q, g, drop)

    fd = (loss_w(delta) - loss_w(-delta)) / (2 * delta)
    an = float((grads["w_qkv"] * uw).sum())
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0)
