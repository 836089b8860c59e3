"""Pins of the optimizer oracle: Adam closed forms, clipping, loss scaling,
the skip on non-finite gradients, and the bf16 rounding of the weight copy."""
import numpy as np
import pytest
import torch

from oracle import adam as A
from oracle.bf16 import round_to_bf16
from synth.inputs import bf16_bits_to_f32, to_bf16_bits


def test_constant_gradient_closed_form():
    """From zero state with a constant g, mhat = g and vhat = g^2 at every step, so
    each step moves p by exactly -lr * g / (|g| + eps)."""
    g = np.array([3e-3, -2e-2, 0.5, -1.25, 1e-6])
    cfg0 = A.AdamConfig(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, max_grad_norm=0.0)
    p = np.array([0.1, -0.2, 0.3, 0.0, 1.0])
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    p0 = p.copy()
    for t in range(1, 6):
        cfg = A.AdamConfig(**{**cfg0.__dict__, "step": t})
        p, m, v, w, (norm, coef, inf) = A.adam_step(p, m, v, g, cfg)
        assert not inf and coef == 1.0
        want = p0 - t * cfg.lr * g / (np.abs(g) + cfg.eps)
        assert np.max(np.abs(p - want)) < 1e-12


def test_zero_gradient_keeps_weights():
    p = np.array([0.5, -0.25, 2.0])
    cfg = A.AdamConfig(step=3, max_grad_norm=1.0)
    p2, m2, v2, w, st = A.adam_step(p, np.zeros(3), np.zeros(3), np.zeros(3), cfg)
    assert np.array_equal(p2, p) and np.all(m2 == 0) and np.all(v2 == 0)
    assert st[0] == 0.0 and st[1] == 1.0


def test_clip_coefficient_single_entry():
    c = 7.0
    acc = np.zeros(10)
    acc[4] = -c
    cfg = A.AdamConfig(max_grad_norm=2.0)
    norm, coef, inf = A.norm_clip(acc, cfg)
    assert norm == c and not inf
    assert abs(coef - 2.0 / (c + 1e-6)) < 1e-15
    # below the threshold no clipping
    assert A.norm_clip(acc, A.AdamConfig(max_grad_norm=8.0))[1] == 1.0


def test_clip_scales_the_first_moment():
    """With m = v = 0 at step 1 and clipping coef c, m = (1-b1) c g exactly."""
    acc = np.array([3.0, 4.0])                    # norm 5
    cfg = A.AdamConfig(max_grad_norm=1.0, step=1)
    _, m, v, _, (norm, coef, _) = A.adam_step(np.zeros(2), np.zeros(2), np.zeros(2), acc, cfg)
    assert norm == 5.0
    assert np.max(np.abs(m - 0.1 * acc / (5.0 + 1e-6))) < 1e-15
    assert np.max(np.abs(v - 0.05 * (acc / (5.0 + 1e-6)) ** 2)) < 1e-15


@pytest.mark.parametrize("k", [0, 3, 10])
def test_power_of_two_unscaling_is_exact(k):
    r = np.random.default_rng(1)
    acc = r.standard_normal(64)
    scaled = acc * 2.0 ** k
    cfg = A.AdamConfig(inv_loss_scale=2.0 ** -k, max_grad_norm=0.5)
    ref = A.AdamConfig(inv_loss_scale=1.0, max_grad_norm=0.5)
    a = A.adam_step(np.ones(64), np.zeros(64), np.zeros(64), scaled, cfg)
    b = A.adam_step(np.ones(64), np.zeros(64), np.zeros(64), acc, ref)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_gradient_skips_step(bad):
    r = np.random.default_rng(2)
    p, m, v = r.standard_normal(16), r.standard_normal(16), r.random(16)
    acc = r.standard_normal(16)
    acc[7] = bad
    p2, m2, v2, w, (norm, coef, inf) = A.adam_step(p, m, v, acc, A.AdamConfig(step=9))
    assert inf and w is None
    assert np.array_equal(p2, p) and np.array_equal(m2, m) and np.array_equal(v2, v)


def test_bias_correction_second_step():
    """Two steps with g1, g2 from zero state, written out by hand."""
    b1, b2, lr, eps = 0.9, 0.95, 1e-2, 1e-8
    g1, g2 = 0.3, -0.7
    m1, v1 = (1 - b1) * g1, (1 - b2) * g1 * g1
    m2, v2 = b1 * m1 + (1 - b1) * g2, b2 * v1 + (1 - b2) * g2 * g2
    p1 = 1.0 - lr * (m1 / (1 - b1)) / (np.sqrt(v1 / (1 - b2)) + eps)
    p2 = p1 - lr * (m2 / (1 - b1 ** 2)) / (np.sqrt(v2 / (1 - b2 ** 2)) + eps)
    cfg = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, max_grad_norm=0.0)
    s1 = A.adam_step(np.array([1.0]), np.zeros(1), np.zeros(1), np.array([g1]), A.AdamConfig(step=1, **cfg))
    s2 = A.adam_step(s1[0], s1[1], s1[2], np.array([g2]), A.AdamConfig(step=2, **cfg))
    assert abs(s2[0][0] - p2) < 1e-15


def test_decoupled_weight_decay():
    cfg = A.AdamConfig(lr=0.1, weight_decay=0.5, max_grad_norm=0.0)
    p2, _, _, _, _ = A.adam_step(np.array([2.0]), np.zeros(1), np.zeros(1), np.array([0.0]), cfg)
    assert abs(p2[0] - 2.0 * (1 - 0.05)) < 1e-15


def test_accumulate_sums_microbatches():
    gs = [np.full(5, float(k)) for k in range(1, 5)]
    assert np.array_equal(A.accumulate(gs), np.full(5, 10.0))


# --------------------------------------------------------------------------
# bf16 rounding of the weight copy
# --------------------------------------------------------------------------

def test_bf16_hand_values():
    e = 2.0 ** -8
    vals = np.array([1.0, 1.0 + e, 1.0 + 3 * e, 1.0 + 1.5 * e, -(1.0 + e), 0.0, -0.0,
                     3.0e38, 3.4e38, 1e-40, np.inf, -np.inf])
    # 3.0e38 sits 225.73 spacings of 2^120 above zero in the top binade -> 226 * 2^120;
    # 1e-40 is subnormal: spacing 2^-133 (the smallest one), 1e-40 / 2^-133 = 1.089 -> 2^-133
    want = np.array([1.0, 1.0, 1.0 + 4 * e, 1.0 + 2 * e, -1.0, 0.0, -0.0,
                     226 * 2.0 ** 120, np.inf, 2.0 ** -133, np.inf, -np.inf])
    got = round_to_bf16(vals)
    assert got[0] == 1.0 and got[1] == 1.0            # tie goes to even
    assert got[2] == 1.0 + 4 * e                       # tie goes to even (up)
    assert got[3] == 1.0 + 2 * e                       # above the tie rounds up
    assert got[4] == -1.0
    assert np.signbit(got[6])
    assert got[8] == np.inf                            # beyond max finite -> inf
    assert np.isinf(got[10]) and np.isinf(got[11]) and got[11] < 0
    assert np.isnan(round_to_bf16(np.array([np.nan]))[0])
    assert got[7] == want[7]
    assert got[9] == want[9]


def test_bf16_matches_torch_and_bit_rounding():
    """Against two independent roundings: torch's float32->bfloat16 conversion and the
    input generator's bit-level one (values first made float32-exact)."""
    r = np.random.default_rng(3)
    x = (r.standard_normal(200000) * np.exp(r.uniform(-30, 30, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32(1.0) + np.arange(-512, 512, dtype=np.float32) * np.float32(2 ** -15)])
    mine = round_to_bf16(x.astype(np.float64))
    via_torch = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    via_bits = bf16_bits_to_f32(to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(mine, via_torch)
    assert np.array_equal(mine, via_bits)
