"""Float64 oracle of dropout on the outputs of the two sliced halves, with the
mask drawn from a counter-based generator.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
GPU library.

From the pages: the Megatron MLP example of the STRONGHOLD slide deck (slide
8) writes the second, row-sliced linear as Z = Dropout(Y B): dropout acts on
the output of B, i.e. after operator g has summed the slices' partials. The
pages give no rate and say nothing about the attention half.

Readings:

* Dropout is applied to the sum of the partials plus the row-sliced bias, and
  the residual is added afterwards: out = residual + mask * scale * (sum + b).
  The attention half gets the same treatment at its output projection (the
  plainest reading: both halves end in a row-sliced linear followed by g).
* The mask comes from Philox4x64-10, the counter-based generator of Salmon,
  Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
  (SC 2011), so that the backward regenerates it instead of storing it. Each
  call of the generator maps a 256-bit counter and a 128-bit key to 256
  random bits: here counter = (e // 16, 0, 0, 0) for the element with
  row-major index e of the [rows, cols] tensor, key = (seed, site), and the
  element takes the 16 bits at position e % 16 (word (e % 16) // 4, bits
  16 * (e % 4) up). `site` tells apart the dropout sites of one step (layer,
  half, micro-batch).
* The element is kept when its 16-bit value u satisfies u >= thr with
  thr = round(p * 65536); the keep probability is then exactly
  1 - thr / 65536, and kept values are scaled by 65536 / (65536 - thr) so
  that the expectation is unchanged. p = 0 keeps everything with scale 1.
* Backward: d(sum + b) = mask * scale * g, with g the gradient of out; the
  residual path passes g unchanged.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
# Philox4x64 round multipliers and key increments (Salmon et al. 2011)
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
ROUNDS = 10

_U32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.ndarray, m: int):
    """Full 128-bit product of uint64 arrays a and the constant m: (hi, lo)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.uint64(m)
    a0, a1 = a & _U32, a >> _S32
    b0, b1 = b & _U32, b >> _S32
    p00 = a0 * b0
    p01 = a0 * b1
    p10 = a1 * b0
    p11 = a1 * b1
    mid = (p00 >> _S32) + (p01 & _U32) + (p10 & _U32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = a * b  # wraps modulo 2^64
    return hi, lo


def philox4x64(counter, key):
    """Philox4x64-10 of counters [..., 4] (uint64) under key (k0, k1). Returns [..., 4] uint64."""
    x = np.array(counter, dtype=np.uint64, copy=True)
    k0, k1 = int(key[0]) & MASK64, int(key[1]) & MASK64
    with np.errstate(over="ignore"):
        for r in range(ROUNDS):
            hi0, lo0 = _mulhilo(x[..., 0], PHILOX_M0)
            hi1, lo1 = _mulhilo(x[..., 2], PHILOX_M1)
            x = np.stack([hi1 ^ x[..., 1] ^ np.uint64(k0), lo1, hi0 ^ x[..., 3] ^ np.uint64(k1), lo0], axis=-1)
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
    return x


def philox4x64_scalar(counter, key):
    """The same generator on Python integers, one block (for tiny cases)."""
    x = [int(c) & MASK64 for c in counter]
    k0, k1 = int(key[0]) & MASK64, int(key[1]) & MASK64
    for _ in range(ROUNDS):
        p0 = PHILOX_M0 * x[0]
        p1 = PHILOX_M1 * x[2]
        x = [(p1 >> 64) ^ x[1] ^ k0, p1 & MASK64, (p0 >> 64) ^ x[3] ^ k1, p0 & MASK64]
        k0 = (k0 + PHILOX_W0) & MASK64
        k1 = (k1 + PHILOX_W1) & MASK64
    return x


def threshold(p: float) -> int:
    """Integer drop threshold on a 16-bit draw (round half to even)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout rate must be in [0, 1)")
    return int(np.round(p * 65536.0))


def keep_scale(p: float) -> float:
    return 65536.0 / (65536.0 - threshold(p))


def draws16(n: int, seed: int, site: int) -> np.ndarray:
    """The 16-bit draw of each of the first n elements (uint16 array)."""
    blocks = (n + 15) // 16
    ctr = np.zeros((blocks, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(blocks, dtype=np.uint64)
    words = philox4x64(ctr, (seed, site))                          # [blocks, 4]
    shifts = np.array([0, 16, 32, 48], dtype=np.uint64)
    parts = (words[:, :, None] >> shifts[None, None, :]) & np.uint64(0xFFFF)
    return parts.reshape(-1)[:n].astype(np.uint16)


def mask(shape, p: float, seed: int, site: int) -> np.ndarray:
    """Keep mask (bool) of a row-major tensor of the given shape."""
    n = int(np.prod(shape))
    return (draws16(n, seed, site) >= threshold(p)).reshape(shape)


def attention_keep(batch: int, heads, seq: int, p: float, seed: int, site: int) -> np.ndarray:
    """Keep mask (bool [batch, len(heads), seq, seq]) of dropout on the
    attention probabilities of the given (global) heads.

    Reading: the pages name dropout only on the row-sliced output; the
    attention probabilities get their own counter-based mask, keyed so that
    one generator call serves a 4 x 4 block of (query, key) pairs. Element
    (b, head, q, k) draws from Philox4x64-10 with counter
    (q // 4, k // 4, head, b) and key (seed, site) the 16 bits at
    16 * (k % 4) of word q % 4, and is kept when that draw is >= thr (as
    ``mask``). The global head index makes the mask the same however the heads
    are split into slices.
    """
    heads = np.asarray(heads, dtype=np.uint64)
    nq = (seq + 3) // 4
    qb, kb = np.meshgrid(np.arange(nq, dtype=np.uint64), np.arange(nq, dtype=np.uint64), indexing="ij")
    thr = threshold(p)
    out = np.empty((batch, len(heads), nq * 4, nq * 4), dtype=bool)
    shifts = np.array([0, 16, 32, 48], dtype=np.uint64)
    for b in range(batch):
        for j, hg in enumerate(heads):
            ctr = np.stack([qb, kb, np.full_like(qb, hg), np.full_like(qb, b)], axis=-1)   # [nq, nq, 4]
            words = philox4x64(ctr, (seed, site))                                          # [nq, nq, 4]: word = q % 4
            d = (words[:, :, :, None] >> shifts[None, None, None, :]) & np.uint64(0xFFFF)   # [qb, kb, q%4, k%4]
            out[b, j] = (d >= thr).transpose(0, 2, 1, 3).reshape(nq * 4, nq * 4)
    return out[:, :, :seq, :seq]


def dropout_sum_fwd(partials, residual, bias, p: float, seed: int, site: int) -> np.ndarray:
    """out = residual + mask * scale * (sum of partials + bias)."""
    z = np.zeros_like(np.asarray(residual, dtype=np.float64))
    for part in partials:
        z = z + part
    if bias is not None:
        z = z + bias[None, :]
    keep = mask(z.shape, p, seed, site)
    return residual + np.where(keep, z * keep_scale(p), 0.0)


def dropout_bwd(g, p: float, seed: int, site: int) -> np.ndarray:
    """Gradient w.r.t. the dropped tensor (sum + bias) for upstream gradient g."""
    keep = mask(np.shape(g), p, seed, site)
    return np.where(keep, np.asarray(g, dtype=np.float64) * keep_scale(p), 0.0)


def layer_fwd(sh, x, full, p: float, seed: int, sites=(0, 1), attn_drop=None):
    """The sliced layer of ``oracle.layer.layer_fwd`` with dropout on the output of
    each half (after the slices' partials and the row-sliced bias are summed,
    before the residual). sites = (attention site, MLP site). attn_drop: None,
    or (rate, seed, site) for dropout on the attention probabilities as in
    ``oracle.layer.layer_fwd``. Returns (out, state)."""
    from . import layer as OL
    t = sh.tp
    ap = [OL.attn_slice(sh, full, i) for i in range(t)]
    mp = [OL.mlp_slice(sh, full, i) for i in range(t)]
    drops = [None if attn_drop is None else (*attn_drop, i * sh.local_heads) for i in range(t)]
    a_fwd = [OL.attn_half_fwd(sh, x, ap[i], attn_drop=drops[i]) for i in range(t)]
    x1 = dropout_sum_fwd([r[0] for r in a_fwd], x, full["b_o"], p, seed, sites[0])
    m_fwd = [OL.mlp_half_fwd(sh, x1, mp[i]) for i in range(t)]
    out = dropout_sum_fwd([r[0] for r in m_fwd], x1, full["b_b"], p, seed, sites[1])
    state = {"ap": ap, "mp": mp, "a_saved": [r[1] for r in a_fwd], "m_saved": [r[1] for r in m_fwd], "x1": x1}
    return out, state


def layer_bwd(sh, g, state, p: float, seed: int, sites=(0, 1)):
    """Backward of layer_fwd for L = <out, g>. Each half's slices receive the
    dropout-masked gradient; the residual paths carry g and G1 unchanged.
    Returns (dx, per-slice attention grads, per-slice MLP grads); the grads
    are those of ``oracle.layer.attn_half_bwd`` / ``mlp_half_bwd``."""
    from . import layer as OL
    t = sh.tp
    dz2 = dropout_bwd(g, p, seed, sites[1])
    m_b = [OL.mlp_half_bwd(sh, dz2, state["mp"][i], state["m_saved"][i]) for i in range(t)]
    g1 = OL.reduce_partials([r[0] for r in m_b], g, None)
    dz1 = dropout_bwd(g1, p, seed, sites[0])
    a_b = [OL.attn_half_bwd(sh, dz1, state["ap"][i], state["a_saved"][i]) for i in range(t)]
    dx = OL.reduce_partials([r[0] for r in a_b], g1, None)
    return dx, [r[1] for r in a_b], [r[1] for r in m_b]


def layer_loss(sh, x, full, g, p: float, seed: int, sites=(0, 1), attn_drop=None) -> float:
    out, _ = layer_fwd(sh, x, full, p, seed, sites, attn_drop)
    return float((out * g).sum())
