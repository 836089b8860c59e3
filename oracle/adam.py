"""Float64 oracle of the mixed-precision optimizer step of one GPU's share.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
GPU library.

From the pages: mixed-precision Adam training keeps about 20 bytes per
parameter (Elamur summary page, "Key points"), and the batch is split into
micro-batches whose gradients are accumulated (same section). The Adam rule
itself is the one of Kingma & Ba (listed among the page's references).

Readings (the pages give no more):

* 20 B/param = bf16 weight 2 + bf16 gradient 2 + fp32 master 4 + m 4 + v 4 +
  fp32 gradient accumulator 4.
* Gradients of the micro-batches are summed into the accumulator
  (acc = g_1 + ... + g_k); the oracle sums in float64.
* Loss scaling: the accumulated gradient is multiplied by inv_scale before the
  norm. A non-finite value anywhere skips the step and leaves every state
  buffer unchanged (dynamic loss scaling convention).
* Global L2 clipping over the whole share: coef = max_norm / (norm + 1e-6),
  applied only when below 1; max_norm <= 0 turns clipping off.
* Adam with bias correction, eps outside the square root, decoupled weight
  decay (p <- p * (1 - lr*wd)) applied before the moment update when wd > 0.
* The bf16 weight copy is the round-to-nearest-even of the new master value.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .bf16 import round_to_bf16

CLIP_EPS = 1e-6


@dataclass(frozen=True)
class AdamConfig:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.0
    max_grad_norm: float = 1.0
    inv_loss_scale: float = 1.0
    step: int = 1          # 1-based index of the step being taken


def accumulate(grads) -> np.ndarray:
    """acc = sum of the micro-batch gradients, in float64."""
    acc = np.zeros(np.shape(grads[0]), dtype=np.float64)
    for g in grads:
        acc = acc + np.asarray(g, dtype=np.float64)
    return acc


def norm_clip(acc: np.ndarray, cfg: AdamConfig):
    """Returns (norm, clip_coef, found_inf) of the unscaled accumulated gradient."""
    gh = np.asarray(acc, dtype=np.float64) * cfg.inv_loss_scale
    found_inf = not bool(np.all(np.isfinite(gh)))
    if found_inf:
        return float("nan"), 1.0, True
    norm = float(np.sqrt(np.sum(gh * gh)))
    coef = 1.0
    if cfg.max_grad_norm > 0.0:
        c = cfg.max_grad_norm / (norm + CLIP_EPS)
        if c < 1.0:
            coef = c
    return norm, coef, False


def adam_update(master, m, v, acc, cfg: AdamConfig, coef: float, found_inf: bool):
    """One Adam step given the norm result. Returns (master, m, v, w_bf16_as_float).

    Skips (returns copies of the inputs) when found_inf is set.
    """
    master = np.asarray(master, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if found_inf:
        return master.copy(), m.copy(), v.copy(), None
    g = np.asarray(acc, dtype=np.float64) * cfg.inv_loss_scale * coef
    p = master
    if cfg.weight_decay > 0.0:
        p = p * (1.0 - cfg.lr * cfg.weight_decay)
    m2 = cfg.beta1 * m + (1.0 - cfg.beta1) * g
    v2 = cfg.beta2 * v + (1.0 - cfg.beta2) * g * g
    mhat = m2 / (1.0 - cfg.beta1 ** cfg.step)
    vhat = v2 / (1.0 - cfg.beta2 ** cfg.step)
    p2 = p - cfg.lr * mhat / (np.sqrt(vhat) + cfg.eps)
    return p2, m2, v2, round_to_bf16(p2)


def adam_step(master, m, v, acc, cfg: AdamConfig):
    """Norm + clip + update. Returns (master, m, v, w, (norm, coef, found_inf))."""
    norm, coef, found_inf = norm_clip(acc, cfg)
    p2, m2, v2, w = adam_update(master, m, v, acc, cfg, coef, found_inf)
    return p2, m2, v2, w, (norm, coef, found_inf)
