"""Pins of the pipeline-stage oracle to things other than itself.

* finite differences of L = sum_k <Y_k, G_k> over a chain of layers and
  several micro-batches, along random directions in every parameter of every
  layer and in every micro-batch input: checks the chaining order, the
  reverse-order backward and that the accumulated gradient is the gradient of
  the summed loss;
* a closed form: layers whose two output projections and output biases are
  zero are the identity, so the stage returns its input and passes the
  gradient through unchanged, whatever the other parameters;
* the flat layout: each tensor sits at the offset the documented order gives.
"""
import numpy as np

from oracle import adam as OA
from oracle import layer as OL
from oracle import stage as OS

SH = OL.LayerShape(batch=1, seq=4, hidden=12, heads=3, ffn=24, tp=1)


def rng(seed):
    return np.random.default_rng(seed)


def make_layers(n, seed, scale=0.3):
    out = []
    for i in range(n):
        r = rng(seed + i)
        p = {}
        for k, s in OL.full_param_shapes(SH).items():
            p[k] = (1.0 + 0.2 * r.standard_normal(s)) if k in ("ln1_g", "ln2_g") else scale * r.standard_normal(s)
        out.append(p)
    return out


def test_stage_gradients_finite_differences():
    layers = make_layers(3, 40)
    xs = [rng(50 + k).standard_normal((SH.tokens, SH.hidden)) for k in range(2)]
    gs = [rng(60 + k).standard_normal((SH.tokens, SH.hidden)) for k in range(2)]
    _, dxs, flats = OS.stage_micro_batches(SH, layers, xs, gs)
    acc = OA.accumulate(flats)
    r = rng(70)
    up = [{k: r.standard_normal(v.shape) for k, v in p.items()} for p in layers]
    ux = [r.standard_normal(x.shape) for x in xs]
    delta = 1e-5

    def loss_at(s):
        lay = [{k: p[k] + s * u[k] for k in p} for p, u in zip(layers, up)]
        return OS.stage_loss(SH, lay, [x + s * u for x, u in zip(xs, ux)], gs)

    fd = (loss_at(delta) - loss_at(-delta)) / (2 * delta)
    an = float(acc @ OS.flatten(up)) + sum(float((dx * u).sum()) for dx, u in zip(dxs, ux))
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (fd, an)


def test_stage_parameter_gradient_per_layer():
    """Directional derivative along one layer's parameters at a time (a swapped
    layer order in the backward would fail here even if the total matched)."""
    layers = make_layers(3, 80)
    xs = [rng(90).standard_normal((SH.tokens, SH.hidden))]
    gs = [rng(91).standard_normal((SH.tokens, SH.hidden))]
    _, _, flats = OS.stage_micro_batches(SH, layers, xs, gs)
    per_layer = flats[0].size // 3
    for i in range(3):
        u = {k: rng(100 + i).standard_normal(v.shape) for k, v in layers[i].items()}
        delta = 1e-5

        def loss_at(s):
            lay = [dict(p) for p in layers]
            lay[i] = {k: layers[i][k] + s * u[k] for k in u}
            return OS.stage_loss(SH, lay, xs, gs)

        fd = (loss_at(delta) - loss_at(-delta)) / (2 * delta)
        an = float(flats[0][i * per_layer:(i + 1) * per_layer] @ OS.flatten([u]))
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (i, fd, an)


def test_stage_with_zero_output_projections_is_identity():
    layers = make_layers(3, 110)
    for p in layers:
        for k in ("w_o", "b_o", "w_b", "b_b"):
            p[k] = np.zeros_like(p[k])
    xs = [rng(120).standard_normal((SH.tokens, SH.hidden))]
    gs = [rng(121).standard_normal((SH.tokens, SH.hidden))]
    ys, dxs, _ = OS.stage_micro_batches(SH, layers, xs, gs)
    assert np.array_equal(ys[0], xs[0])
    assert np.array_equal(dxs[0], gs[0])


def test_flat_layout_follows_documented_order():
    layers = make_layers(2, 130)
    flat = OS.flatten(layers)
    h, f = SH.hidden, SH.ffn
    sizes = [h, h, h * 3 * h, 3 * h, h * h, h, h, h, h * f, f, f * h, h]
    assert flat.size == 2 * sum(sizes)
    pos = 0
    for p in layers:
        for key, n in zip([k for half in OS.FLAT_ORDER for k in half], sizes):
            assert np.array_equal(flat[pos:pos + n], p[key].reshape(-1)), key
            pos += n


def test_stage_with_dropout_finite_differences():
    """With dropout on every half (masks fixed by seed and site), the summed
    loss's gradient over 2 layers x 2 micro-batches matches central
    differences; at p = 0 the dropout path equals the plain one."""
    from oracle import dropout as OD
    layers = make_layers(2, 140)
    xs = [rng(150 + k).standard_normal((SH.tokens, SH.hidden)) for k in range(2)]
    gs = [rng(160 + k).standard_normal((SH.tokens, SH.hidden)) for k in range(2)]
    p, seed = 0.3, 77
    _, dxs, flats = OS.stage_micro_batches(SH, layers, xs, gs, dropout=(p, seed))
    acc = OA.accumulate(flats)
    r = rng(170)
    up = [{k: r.standard_normal(v.shape) for k, v in q.items()} for q in layers]
    ux = [r.standard_normal(x.shape) for x in xs]
    delta = 1e-5

    def loss_at(s):
        tot = 0.0
        for k, (x, g) in enumerate(zip(xs, gs)):
            lay = [{key: q[key] + s * u[key] for key in q} for q, u in zip(layers, up)]
            h = x + s * ux[k]
            for l, full in enumerate(lay):
                h, _ = OD.layer_fwd(SH, h, full, p, seed, ((k * 2 + l) * 2, (k * 2 + l) * 2 + 1))
            tot += float((h * g).sum())
        return tot

    fd = (loss_at(delta) - loss_at(-delta)) / (2 * delta)
    an = float(acc @ OS.flatten(up)) + sum(float((dx * u).sum()) for dx, u in zip(dxs, ux))
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (fd, an)
    # p = 0: the dropout path reduces to the plain stage
    ys0, dxs0, fl0 = OS.stage_micro_batches(SH, layers, xs[:1], gs[:1])
    y1, dx1, g1 = OS._stage_dropout(SH, layers, xs[0], gs[0], 0, 0.0, seed)
    np.testing.assert_allclose(y1, ys0[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dx1, dxs0[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(OS.flatten(g1), fl0[0], rtol=0, atol=1e-12)


def test_stage_with_attention_dropout_finite_differences():
    """Dropout on the attention probabilities of every layer (each layer and
    micro-batch keyed by its own site) together with dropout on every half's
    output: the summed loss's gradient matches central differences; each
    layer's attention mask differs from the others'; at rate 0 the stage is
    the plain one."""
    from oracle import dropout as OD
    sh = OL.LayerShape(batch=1, seq=8, hidden=12, heads=3, ffn=24, tp=1)
    layers = []
    for i in range(2):
        r = rng(180 + i)
        layers.append({k: (1.0 + 0.2 * r.standard_normal(s)) if k in ("ln1_g", "ln2_g") else 0.3 * r.standard_normal(s)
                       for k, s in OL.full_param_shapes(sh).items()})
    xs = [rng(190 + k).standard_normal((sh.tokens, sh.hidden)) for k in range(2)]
    gs = [rng(200 + k).standard_normal((sh.tokens, sh.hidden)) for k in range(2)]
    p, seed, ad = 0.2, 31, (0.25, 901, 40)
    _, dxs, flats = OS.stage_micro_batches(sh, layers, xs, gs, dropout=(p, seed), attn_dropout=ad)
    acc = OA.accumulate(flats)
    r = rng(210)
    up = [{k: r.standard_normal(v.shape) for k, v in q.items()} for q in layers]
    ux = [r.standard_normal(x.shape) for x in xs]
    delta = 1e-5

    def loss_at(s):
        tot = 0.0
        for k, (x, g) in enumerate(zip(xs, gs)):
            lay = [{key: q[key] + s * u[key] for key in q} for q, u in zip(layers, up)]
            h = x + s * ux[k]
            for l, full in enumerate(lay):
                h, _ = OD.layer_fwd(sh, h, full, p, seed, ((k * 2 + l) * 2, (k * 2 + l) * 2 + 1),
                                    (ad[0], ad[1], ad[2] + k * 2 + l))
            tot += float((h * g).sum())
        return tot

    fd = (loss_at(delta) - loss_at(-delta)) / (2 * delta)
    an = float(acc @ OS.flatten(up)) + sum(float((dx * u).sum()) for dx, u in zip(dxs, ux))
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (fd, an)
    # four layer calls, four distinct attention masks
    masks = [OD.attention_keep(1, range(3), sh.seq, ad[0], ad[1], site)
             for (_, _, site) in OS.attn_drops(2, 0, ad) + OS.attn_drops(2, 1, ad)]
    for i in range(4):
        for j in range(i):
            assert (masks[i] != masks[j]).any()
    # rate 0: the plain stage
    ys0, dxs0, fl0 = OS.stage_micro_batches(sh, layers, xs, gs)
    ys1, dxs1, fl1 = OS.stage_micro_batches(sh, layers, xs, gs, attn_dropout=(0.0, 901, 40))
    for a, b in zip(ys0 + dxs0 + fl0, ys1 + dxs1 + fl1):
        np.testing.assert_array_equal(a, b)
