"""Float64 oracle of one pipeline stage: chained layers, micro-batch gradient
accumulation and one Adam step.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
GPU library.

From the pages: the 105 layers of MT-NLG 530B are divided over a 35-way
pipeline with 8-way tensor slicing inside each node (jiqizhixin MT-NLG
article, paragraph on the 3D-parallel system), so one GPU holds three
consecutive layer slices; the batch is processed as micro-batches whose
gradients are accumulated before the optimizer step (Elamur summary page, Key
points).

Readings:

* A stage applies its layers in order; its backward runs them in reverse,
  each layer receiving the gradient of its output from the layer after it.
* Each micro-batch is independent: its forward and backward see the same
  parameters, and the step's accumulated gradient is the sum of the
  micro-batch gradients (the gradient of the sum of their losses).
* The stage's loss stand-in is L = sum_k <Y_k, G_k> with G_k the given
  gradient of micro-batch k's output (what the next stage would send).
* One slice (t = 1) is the whole layer, so the stage oracle works on full
  parameters; the optimizer step is the one in ``oracle.adam`` over all of
  the stage's parameters as one share.
* With dropout (``oracle.dropout``), each half's output of micro-batch k and
  layer l uses its own site, (k * layers + l) * 2 + half, so that no two
  dropout masks of a step coincide.
* With dropout on the attention probabilities (rate, seed, site0), layer l of
  micro-batch k keys its mask with (seed, site0 + k * layers + l).
"""
from __future__ import annotations

import numpy as np

from . import adam as OA
from . import layer as OL

# Order of a layer's tensors in a flat parameter vector: attention half, then
# MLP half, each (LayerNorm gain, LayerNorm bias, first linear weight and
# bias, second linear weight, its bias added after the slice sum).
FLAT_ORDER = (("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o"),
              ("ln2_g", "ln2_b", "w_a", "b_a", "w_b", "b_b"))


def attn_drops(n_layers: int, k: int, attn_dropout):
    """Per-layer attention-probability dropout of micro-batch k: None each, or
    (rate, seed, site0 + k * layers + l) for attn_dropout = (rate, seed, site0)."""
    if attn_dropout is None or attn_dropout[0] <= 0.0:
        return [None] * n_layers
    rate, seed, site0 = attn_dropout
    return [(rate, seed, site0 + k * n_layers + l) for l in range(n_layers)]


def stage_fwd(sh: OL.LayerShape, layers: list, x: np.ndarray, drops=None):
    """Output of the chained layers for input x, and the per-layer states.
    drops: None, or each layer's attention-probability dropout (attn_drops)."""
    states = []
    h = x
    for l, full in enumerate(layers):
        h, st = OL.layer_fwd(sh, h, full, None if drops is None else drops[l])
        states.append(st)
    return h, states


def stage_bwd(sh: OL.LayerShape, layers: list, states: list, g: np.ndarray):
    """Gradient of L = <Y, g> w.r.t. the stage input and every layer's parameters."""
    grads = [None] * len(layers)
    for i in reversed(range(len(layers))):
        g, grads[i] = OL.layer_bwd(sh, g, layers[i], states[i])
    return g, grads


def stage_loss(sh: OL.LayerShape, layers: list, xs, gs) -> float:
    """L = sum over micro-batches k of <Y_k, G_k>."""
    return float(sum((stage_fwd(sh, layers, x)[0] * g).sum() for x, g in zip(xs, gs)))


def flatten(layer_dicts: list) -> np.ndarray:
    """Concatenate per-layer tensors (parameters or gradients) in FLAT_ORDER."""
    parts = []
    for d in layer_dicts:
        for half in FLAT_ORDER:
            for k in half:
                parts.append(np.asarray(d[k], dtype=np.float64).reshape(-1))
    return np.concatenate(parts)


def _stage_dropout(sh: OL.LayerShape, layers: list, x, g, k: int, p: float, seed: int, drops=None):
    """One micro-batch through the stage with dropout on every half's output
    (``oracle.dropout``): the site of micro-batch k, layer l, half h is
    (k * layers + l) * 2 + h. One slice (t = 1), so a slice's gradients are
    the layer's. drops: None, or each layer's attention-probability dropout."""
    from . import dropout as OD
    assert sh.tp == 1
    nl = len(layers)
    sites = [((k * nl + l) * 2, (k * nl + l) * 2 + 1) for l in range(nl)]
    states, h = [], x
    for l, full in enumerate(layers):
        h, st = OD.layer_fwd(sh, h, full, p, seed, sites[l], None if drops is None else drops[l])
        states.append(st)
    y = h
    grads = [None] * nl
    names = {0: dict(zip(("ln_g", "ln_b", "w_in", "b_in", "w_out", "b_out"), FLAT_ORDER[0])),
             1: dict(zip(("ln_g", "ln_b", "w_in", "b_in", "w_out", "b_out"), FLAT_ORDER[1]))}
    for l in reversed(range(nl)):
        g, ga, gm = OD.layer_bwd(sh, g, states[l], p, seed, sites[l])
        d = {names[0][key]: v for key, v in ga[0].items()}
        d.update({names[1][key]: v for key, v in gm[0].items()})
        grads[l] = d
    return y, g, grads


def stage_micro_batches(sh: OL.LayerShape, layers: list, xs, gs, dropout=None, attn_dropout=None):
    """Forward and backward of every micro-batch. Returns (ys, dxs, per-micro-batch
    flat gradients). dropout = (p, seed) puts dropout on every half's output;
    attn_dropout = (rate, seed, site0) on the attention probabilities."""
    ys, dxs, flats = [], [], []
    for k, (x, g) in enumerate(zip(xs, gs)):
        drops = attn_drops(len(layers), k, attn_dropout)
        if dropout is not None and dropout[0] > 0.0:
            y, dx, grads = _stage_dropout(sh, layers, x, g, k, dropout[0], dropout[1], drops)
        else:
            y, states = stage_fwd(sh, layers, x, drops)
            dx, grads = stage_bwd(sh, layers, states, g)
        ys.append(y)
        dxs.append(dx)
        flats.append(flatten(grads))
    return ys, dxs, flats


def stage_step(sh: OL.LayerShape, layers: list, xs, gs, master, m, v, cfg: OA.AdamConfig):
    """The whole stage step: micro-batches, accumulation of their gradients, Adam.

    Returns (ys, dxs, acc, (master, m, v, w, stats)).
    """
    ys, dxs, flats = stage_micro_batches(sh, layers, xs, gs)
    acc = OA.accumulate(flats)
    return ys, dxs, acc, OA.adam_step(master, m, v, acc, cfg)
