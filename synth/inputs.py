"""Seeded tensors at the shapes of the MT-NLG layer-shard workloads.

Recipe (identical bytes go to the GPU and to the oracle):

* numpy ``Generator(PCG64(seed))``, ``standard_normal(dtype=float32)``, times
  the standard deviation (plus a mean where stated);
* for bfloat16 storage the float32 values are rounded to bfloat16 (nearest,
  ties to even) on their bit patterns, and the float32 copy is replaced by the
  exactly representable rounded value;
* one seed per tensor: ``seed = 1000 * workload + tensor_index``.

Distributions: activations and upstream gradients N(0, 1); linear weights and
biases N(0, 0.02); LayerNorm gamma = 1 + 0.02 N(0,1) and beta = 0.02 N(0,1) so
that their gradients are exercised. "N(0, s)" means standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["randn", "to_bf16_bits", "bf16_bits_to_f32", "round_f32_to_bf16", "qkv_bits",
           "Workload", "WORKLOADS", "half_param_shapes", "make_half_params",
           "make_activation", "make_adam_state"]


def randn(seed: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 N(mean, std) of the given shape from PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even, NaN kept quiet."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).reshape(-1)
    out = np.empty(u.size, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, u.size, step):
        c = u[s:s + step]
        nan = (c & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        r = (c >> np.uint32(16)) & np.uint32(1)       # lsb of the kept half: ties go to even
        r += np.uint32(0x7FFF)
        r += np.where(nan, np.uint32(0), c)            # NaN: no rounding carry into the exponent
        r >>= np.uint32(16)
        r = np.where(nan, (c >> np.uint32(16)) | np.uint32(0x40), r)
        out[s:s + step] = r.astype(np.uint16)
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 (returned as float32)."""
    return bf16_bits_to_f32(to_bf16_bits(x))


def qkv_bits(x: np.ndarray, qk_cols: int):
    """The 16-bit storage of an attention input [T, 3w] in the library's bf16
    path: the first qk_cols columns (Q and K) as IEEE binary16, the rest (V) as
    bfloat16, both rounded to nearest even. Returns (values as float32, uint16
    bit patterns)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    qk = x[:, :qk_cols].astype(np.float16)
    vals = np.empty_like(x)
    vals[:, :qk_cols] = qk.astype(np.float32)
    vals[:, qk_cols:] = round_f32_to_bf16(x[:, qk_cols:])
    bits = np.empty(x.shape, dtype=np.uint16)
    bits[:, :qk_cols] = qk.view(np.uint16)
    bits[:, qk_cols:] = to_bf16_bits(x[:, qk_cols:])
    return vals, bits


@dataclass(frozen=True)
class Workload:
    """One of the five measured or checked configurations."""

    index: int
    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    tp: int                 # slicing factor t
    slices: tuple           # which slice indices are run
    dtype: str              # "f32" or "bf16"
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def local_heads(self) -> int:
        return self.heads // self.tp

    @property
    def local_width(self) -> int:
        return self.local_heads * self.head_dim

    @property
    def local_ffn(self) -> int:
        return self.ffn // self.tp


WORKLOADS = {
    1: Workload(1, "tiny-layer-t2-f32", batch=2, seq=128, hidden=256, heads=4, ffn=1024,
                tp=2, slices=(0, 1), dtype="f32"),
    2: Workload(2, "gpt-h4096-tp1-bf16", batch=1, seq=2048, hidden=4096, heads=32, ffn=16384,
                tp=1, slices=(0,), dtype="bf16"),
    3: Workload(3, "mtnlg-shard-h20480-t8-bf16", batch=1, seq=2048, hidden=20480, heads=128,
                ffn=81920, tp=8, slices=(0,), dtype="bf16"),
    4: Workload(4, "adam-1.887e9", batch=0, seq=0, hidden=20480, heads=128, ffn=81920, tp=8,
                slices=(), dtype="bf16",
                extra={"n": 1_887_436_800, "micro_batches": 4, "step": 100}),
    5: Workload(5, "mtnlg-full-layer-8-slices-b4-bf16", batch=4, seq=2048, hidden=20480,
                heads=128, ffn=81920, tp=8, slices=tuple(range(8)), dtype="bf16"),
    # a pipeline stage of chained layers with micro-batch accumulation
    6: Workload(6, "stage-3-layers-tiny-bf16", batch=2, seq=128, hidden=256, heads=4, ffn=1024,
                tp=1, slices=(0,), dtype="bf16", extra={"layers": 3, "micro_batches": 2, "step": 5}),
    7: Workload(7, "mtnlg-stage-3-layers-shard-bf16", batch=1, seq=2048, hidden=20480, heads=128,
                ffn=81920, tp=8, slices=(0,), dtype="bf16", extra={"layers": 3, "micro_batches": 4, "step": 100}),
}


def half_param_shapes(w: Workload, half: str) -> dict:
    """Shapes of one slice's parameters for the "attn" or "mlp" half."""
    h = w.hidden
    if half == "attn":
        n = 3 * w.local_width
        return {"ln_g": (h,), "ln_b": (h,), "w_in": (h, n), "b_in": (n,),
                "w_out": (w.local_width, h), "b_out": (h,)}
    f = w.local_ffn
    return {"ln_g": (h,), "ln_b": (h,), "w_in": (h, f), "b_in": (f,),
            "w_out": (f, h), "b_out": (h,)}


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_f32_to_bf16(x) if dtype == "bf16" else x


def make_half_params(w: Workload, half: str, slice_index: int, layer: int = 0) -> dict:
    """float32 arrays (bf16-exact when dtype is bf16) for one slice of one half
    of layer `layer` (layers of a stage get their own seeds).

    LayerNorm parameters and the row-sliced output bias are replicated across
    slices, so their seeds do not depend on the slice index.
    """
    base = 1000 * w.index + 200 * layer + (0 if half == "attn" else 100)
    shapes = half_param_shapes(w, half)
    out = {}
    out["ln_g"] = _finish(randn(base + 1, shapes["ln_g"], 0.02, 1.0), w.dtype)
    out["ln_b"] = _finish(randn(base + 2, shapes["ln_b"], 0.02), w.dtype)
    out["b_out"] = _finish(randn(base + 3, shapes["b_out"], 0.02), w.dtype)
    s = base + 10 + 4 * slice_index
    out["w_in"] = _finish(randn(s + 0, shapes["w_in"], 0.02), w.dtype)
    out["b_in"] = _finish(randn(s + 1, shapes["b_in"], 0.02), w.dtype)
    out["w_out"] = _finish(randn(s + 2, shapes["w_out"], 0.02), w.dtype)
    return out


def make_activation(w: Workload, tag: int, cols: int | None = None, std: float = 1.0) -> np.ndarray:
    """[tokens, cols] N(0, std) activation or upstream gradient; tag picks the tensor."""
    cols = w.hidden if cols is None else cols
    return _finish(randn(1000 * w.index + 500 + tag, (w.tokens, cols), std), w.dtype)


def make_adam_state(n: int, seed_base: int = 4000, micro_batches: int = 4):
    """Adam workload of size n: master ~ N(0,0.02), m ~ N(0,1e-3), v = N(0,1e-3)^2,
    micro-batch grads ~ N(0,1e-3) stored as bf16 bits.

    Returns (master f32, m f32, v f32, [grad bf16 bits] * micro_batches).
    """
    master = randn(seed_base + 1, (n,), 0.02)
    m = randn(seed_base + 2, (n,), 1e-3)
    v = randn(seed_base + 3, (n,), 1e-3)
    v *= v
    grads = [to_bf16_bits(randn(seed_base + 10 + k, (n,), 1e-3)) for k in range(micro_batches)]
    return master, m, v, grads
