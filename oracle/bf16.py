"""The oracle's own float -> bfloat16 rounding (round to nearest, ties to even).

TEST INFRASTRUCTURE ONLY. bfloat16 keeps the top 16 bits of an IEEE binary32
value: sign, 8 exponent bits, 7 fraction bits. Rounding a binary64 value x to
bfloat16 is written here from that definition, on values rather than bits:
take the two neighbouring bfloat16 numbers around x (spaced by one unit in
the last place of an 8-bit significand at x's binade) and keep the nearer one,
the one with an even last fraction bit on a tie. NaN stays NaN; values beyond
the largest finite bfloat16 round to infinity exactly when IEEE rounding does.
"""
from __future__ import annotations

import numpy as np

# Largest finite bfloat16: (2 - 2^-7) * 2^127.
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
# Smallest positive normal is 2^-126; subnormals have spacing 2^-133.
BF16_MIN_EXP = -126
BF16_FRAC_BITS = 7


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each element of x (float64 in, float64 out)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat_in = x.reshape(-1)
    flat = out.reshape(-1)
    for start in range(0, flat_in.size, 1 << 22):
        chunk = flat_in[start:start + (1 << 22)]
        flat[start:start + chunk.size] = _round_chunk(chunk)
    return out


def _round_chunk(x: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore", over="ignore"):
        return _round_chunk_inner(x)


def _round_chunk_inner(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    finite = np.isfinite(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(finite & (ax > 0), ax, 1.0)))
    # log2 can be off by one at exact powers of two boundaries: fix by checking.
    e = np.where(2.0 ** e > ax, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= ax, e + 1, e)
    e = np.maximum(e, BF16_MIN_EXP)                  # subnormal binade shares spacing
    ulp = 2.0 ** (e - BF16_FRAC_BITS)
    q = ax / ulp                                     # exact: division by a power of two
    lo = np.floor(q)
    frac = q - lo
    up = (frac > 0.5) | ((frac == 0.5) & (np.fmod(lo, 2.0) == 1.0))
    r = (lo + up) * ulp
    r = np.where(r > BF16_MAX, np.inf, r)
    r = np.copysign(r, x)
    r = np.where(ax == 0, x, r)
    r = np.where(np.isinf(x), x, r)
    r = np.where(np.isnan(x), np.nan, r)
    return r
