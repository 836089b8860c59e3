"""Float64 oracle of one tensor slice of a left-to-right decoder layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
GPU library.

What is computed, and from where:

* The layer is a dense left-to-right (causal) transformer block -- Elamur
  summary page of "Using DeepSpeed and Megatron to Train Megatron-Turing NLG
  530B", section "Summary"; jiqizhixin MT-NLG article, paragraph on the model
  (decoder architecture, 105 layers, hidden 20480, 128 heads).
* Tensor slicing of the MLP: A is split by columns so slice i computes
  Y_i = GeLU(X A_i) with no communication; B is split by rows so slice i
  computes Z_i = Y_i B_i and the layer output is the sum over slices.
  Operator f is identity forward / all-reduce backward, g is all-reduce
  forward / identity backward -- STRONGHOLD slide deck, slides 7-8 (Megatron
  example of intra-layer model parallelism).
* Attention is sliced the same way, by heads: the QKV projection by columns
  (whole heads per slice), the output projection by rows. The slides only say
  that individual layers are split across devices (slide 6); splitting by
  heads is the reading that keeps every slice independent up to g.

Readings where the pages are silent (each is the plainest one the rest
supports):

* Pre-LN block: X1 = X + Attn(LN1(X)), Out = X1 + MLP(LN2(X1)).
* LayerNorm: biased variance over the row, eps = 1e-5, y = gamma*xhat + beta.
* GeLU(u) = u * Phi(u) = u/2 * (1 + erf(u / sqrt 2)) (exact, not tanh).
* Every linear carries a bias. Column-sliced biases are sliced with their
  columns; the two row-sliced biases (attention output, MLP output) are added
  once, after the sum over slices, together with the residual.
* Dropout rate 0 (identity), so results are deterministic.
* Attention scale 1/sqrt(head_dim); query r sees keys c <= r of its own
  sequence; rows are ordered (sequence, position).
* QKV columns ordered (q/k/v, head, dim); slice i owns the contiguous head
  range [i*H/t, (i+1)*H/t) and keeps that order; MLP slice i owns columns
  (of A) / rows (of B) [i*f/t, (i+1)*f/t).

Layout: activations are row-major [batch*seq, width]; weights are in the
math form [in, out] so that Y = X W.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
from scipy.special import erf

SQRT2 = np.sqrt(2.0)
INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


@dataclass(frozen=True)
class LayerShape:
    """Dimensions of the full (unsliced) layer and the slicing factor t."""

    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    tp: int = 1
    eps: float = 1e-5

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
        """Width of one slice's attention output (local heads * head_dim)."""
        return self.local_heads * self.head_dim

    @property
    def local_ffn(self) -> int:
        return self.ffn // self.tp

    def check(self) -> None:
        assert self.hidden % self.heads == 0
        assert self.heads % self.tp == 0
        assert self.ffn % self.tp == 0


# --------------------------------------------------------------------------
# Elementwise and row-wise pieces
# --------------------------------------------------------------------------

def gelu(u: np.ndarray) -> np.ndarray:
    """GeLU(u) = u * Phi(u), Phi the standard normal CDF (reading: exact erf form)."""
    return 0.5 * u * (1.0 + erf(u / SQRT2))


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d/du [u Phi(u)] = Phi(u) + u phi(u)."""
    return 0.5 * (1.0 + erf(u / SQRT2)) + u * INV_SQRT_2PI * np.exp(-0.5 * u * u)


def layernorm_fwd(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float):
    """Row LayerNorm. Returns (y, mean, rstd, xhat).

    mean = average over the row, var = average of squared deviation (biased),
    rstd = 1/sqrt(var + eps), xhat = (x - mean)*rstd, y = gamma*xhat + beta.
    """
    mean = x.mean(axis=1)
    dev = x - mean[:, None]
    var = (dev * dev).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = dev * rstd[:, None]
    return gamma[None, :] * xhat + beta[None, :], mean, rstd, xhat


def layernorm_bwd(gy: np.ndarray, xhat: np.ndarray, rstd: np.ndarray, gamma: np.ndarray):
    """Backward of row LayerNorm for an upstream gradient gy.

    With gh = gy*gamma: dx = rstd * (gh - mean(gh) - xhat*mean(gh*xhat));
    dgamma = sum over rows of gy*xhat; dbeta = sum over rows of gy.
    Linear in gy, which is what lets each slice apply it to its own partial.
    """
    gh = gy * gamma[None, :]
    a = gh.mean(axis=1)
    b = (gh * xhat).mean(axis=1)
    dx = rstd[:, None] * (gh - a[:, None] - xhat * b[:, None])
    return dx, (gy * xhat).sum(axis=0), gy.sum(axis=0)


# --------------------------------------------------------------------------
# Causal attention over a block of heads
# --------------------------------------------------------------------------

def _split_qkv(qkv: np.ndarray, batch: int, seq: int, nh: int, d: int):
    """[T, 3*nh*d] with columns (q/k/v, head, dim) -> three [batch, nh, seq, d]."""
    t5 = qkv.reshape(batch, seq, 3, nh, d)
    q = t5[:, :, 0].transpose(0, 2, 1, 3)
    k = t5[:, :, 1].transpose(0, 2, 1, 3)
    v = t5[:, :, 2].transpose(0, 2, 1, 3)
    return q, k, v


def _merge_heads(o: np.ndarray) -> np.ndarray:
    """[batch, nh, seq, d] -> [batch*seq, nh*d] with columns (head, dim)."""
    b, nh, s, d = o.shape
    return o.transpose(0, 2, 1, 3).reshape(b * s, nh * d)


def causal_mask(seq: int) -> np.ndarray:
    """True where key c is visible to query r (c <= r)."""
    return np.tril(np.ones((seq, seq), dtype=bool))


def attention_fwd(qkv: np.ndarray, batch: int, seq: int, nh: int, d: int, drop=None):
    """Causal multi-head attention of nh heads of width d.

    Per sequence and head: S = Q K^T / sqrt(d); S[r, c] = -inf for c > r;
    P = softmax over each row (max subtracted); O = P V. Returns
    (O [T, nh*d], P [batch, nh, seq, seq], lse [batch, nh, seq]) where
    lse = log sum_c exp(S[r, c]) over the visible keys.

    drop: None, or (keep [batch, nh, seq, seq] bool, scale) for dropout on the
    probabilities: O = (P * keep * scale) V. P and lse stay those of the
    softmax itself (the normaliser is taken before dropout).
    """
    q, k, v = _split_qkv(qkv, batch, seq, nh, d)
    s = np.matmul(q, k.transpose(0, 1, 3, 2)) / np.sqrt(d)
    s = np.where(causal_mask(seq)[None, None], s, -np.inf)
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    z = e.sum(axis=-1, keepdims=True)
    p = e / z
    pd = p if drop is None else np.where(drop[0], p * drop[1], 0.0)
    o = np.matmul(pd, v)
    lse = (mx + np.log(z))[..., 0]
    return _merge_heads(o), p, lse


def attention_bwd(qkv: np.ndarray, p: np.ndarray, do: np.ndarray, batch: int, seq: int,
                  nh: int, d: int, drop=None) -> np.ndarray:
    """Gradient of causal attention. Returns dQKV [T, 3*nh*d] (same column order).

    dV = P~^T dO with P~ = P (or P * keep * scale under dropout); the gradient
    reaching the probabilities is dP = dO V^T (times keep * scale under
    dropout); dS = P * (dP - rowsum(dP * P)) (softmax's own backward, on P);
    dQ = dS K / sqrt(d); dK = dS^T Q / sqrt(d).
    """
    q, k, v = _split_qkv(qkv, batch, seq, nh, d)
    dob = do.reshape(batch, seq, nh, d).transpose(0, 2, 1, 3)
    pd = p if drop is None else np.where(drop[0], p * drop[1], 0.0)
    dv = np.matmul(pd.transpose(0, 1, 3, 2), dob)
    dp = np.matmul(dob, v.transpose(0, 1, 3, 2))
    if drop is not None:
        dp = np.where(drop[0], dp * drop[1], 0.0)
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    scale = 1.0 / np.sqrt(d)
    dq = np.matmul(ds, k) * scale
    dk = np.matmul(ds.transpose(0, 1, 3, 2), q) * scale
    out = np.stack([dq, dk, dv], axis=2)           # [b, nh, 3, s, d]
    return out.transpose(0, 3, 2, 1, 4).reshape(batch * seq, 3 * nh * d)


# --------------------------------------------------------------------------
# Parameters: full layer and the slices of it
# --------------------------------------------------------------------------

FULL_KEYS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
             "ln2_g", "ln2_b", "w_a", "b_a", "w_b", "b_b")


def full_param_shapes(sh: LayerShape) -> dict:
    h, f = sh.hidden, sh.ffn
    return {"ln1_g": (h,), "ln1_b": (h,), "w_qkv": (h, 3 * h), "b_qkv": (3 * h,),
            "w_o": (h, h), "b_o": (h,), "ln2_g": (h,), "ln2_b": (h,),
            "w_a": (h, f), "b_a": (f,), "w_b": (f, h), "b_b": (h,)}


def qkv_columns(sh: LayerShape, i: int) -> np.ndarray:
    """Indices of the full W_qkv columns owned by slice i, in slice order.

    Full columns are ordered (c, n, e) = c*h + n*d + e; slice i keeps heads
    n in [i*H/t, (i+1)*H/t) and the (c, n, e) order.
    """
    h, d, hl = sh.hidden, sh.head_dim, sh.local_heads
    cols = [c * h + n * d + e
            for c in range(3)
            for n in range(i * hl, (i + 1) * hl)
            for e in range(d)]
    return np.asarray(cols, dtype=np.int64)


def attn_slice(sh: LayerShape, full: dict, i: int) -> dict:
    """Slice i of the attention half: QKV columns of its heads, W_o rows of its heads."""
    cols = qkv_columns(sh, i)
    w = sh.local_width
    return {"ln_g": full["ln1_g"], "ln_b": full["ln1_b"],
            "w_in": full["w_qkv"][:, cols], "b_in": full["b_qkv"][cols],
            "w_out": full["w_o"][i * w:(i + 1) * w, :]}


def mlp_slice(sh: LayerShape, full: dict, i: int) -> dict:
    """Slice i of the MLP half: A columns and B rows [i*f/t, (i+1)*f/t)."""
    fl = sh.local_ffn
    return {"ln_g": full["ln2_g"], "ln_b": full["ln2_b"],
            "w_in": full["w_a"][:, i * fl:(i + 1) * fl], "b_in": full["b_a"][i * fl:(i + 1) * fl],
            "w_out": full["w_b"][i * fl:(i + 1) * fl, :]}


# --------------------------------------------------------------------------
# The two halves of one slice (between g all-reduces)
# --------------------------------------------------------------------------

def _keep(a: np.ndarray) -> np.ndarray:
    return a


def attn_half_fwd(sh: LayerShape, x: np.ndarray, p: dict, store=None, store_qk=None, attn_drop=None):
    """Attention half of slice i. Returns (partial, saved).

    partial = Attn_i(LN1(x)) W_o,i, without bias or residual: the operand of
    the forward all-reduce g.

    store: None for the definition itself (every intermediate in float64).
    Diagnostic mode: a rounding function (e.g. oracle.bf16.round_to_bf16)
    applied to each tensor a mixed-precision run keeps between its steps --
    LN1(x), QKV and the attention output O, the saved activations a bf16
    library hands from its forward to its backward. The rest stays float64.
    Comparing a GPU result with both modes separates the error that comes
    from storing those tensors in bf16 from the error of the kernels.
    store_qk, if given, rounds the Q and K columns of QKV instead of store
    (a library may keep them in another 16-bit format).
    attn_drop: None, or (p, seed, site, head0) for dropout on the attention
    probabilities of this slice's heads head0 .. head0 + local_heads - 1
    (global head indices; oracle.dropout.attention_keep).
    """
    rnd = store or _keep
    y, mean, rstd, xhat = layernorm_fwd(x, p["ln_g"], p["ln_b"], sh.eps)
    y = rnd(y)
    qkv = y @ p["w_in"] + p["b_in"][None, :]
    qk = 2 * sh.local_width
    qkv = np.concatenate([(store_qk or rnd)(qkv[:, :qk]), rnd(qkv[:, qk:])], axis=1)
    drop = None
    if attn_drop is not None and attn_drop[0] > 0.0:
        from oracle import dropout as OD
        rate, seed, site, head0 = attn_drop
        heads = np.arange(head0, head0 + sh.local_heads)
        drop = (OD.attention_keep(sh.batch, heads, sh.seq, rate, seed, site), OD.keep_scale(rate))
    o, prob, lse = attention_fwd(qkv, sh.batch, sh.seq, sh.local_heads, sh.head_dim, drop)
    o = rnd(o)
    partial = o @ p["w_out"]
    saved = {"ln_out": y, "mean": mean, "rstd": rstd, "xhat": xhat,
             "qkv": qkv, "o": o, "p": prob, "lse": lse, "drop": drop}
    return partial, saved


def attn_half_bwd(sh: LayerShape, g: np.ndarray, p: dict, saved: dict):
    """Backward of the attention half of slice i for upstream gradient g.

    g is the gradient of the half's output; g (identity backward) reaches
    every slice unchanged. Returns (dx_partial, grads): dx_partial is this
    slice's share of dL/dx through LN1 (f's backward all-reduce sums them; the
    residual path's g is added once by the caller). grads holds ln_g, ln_b
    (partials), w_in, b_in, w_out (this slice's) and b_out (= column sums of
    g, identical on every slice).
    """
    do = g @ p["w_out"].T
    dw_out = saved["o"].T @ g
    dqkv = attention_bwd(saved["qkv"], saved["p"], do, sh.batch, sh.seq,
                         sh.local_heads, sh.head_dim, saved.get("drop"))
    dw_in = saved["ln_out"].T @ dqkv
    db_in = dqkv.sum(axis=0)
    dln = dqkv @ p["w_in"].T
    dx, dg, dbeta = layernorm_bwd(dln, saved["xhat"], saved["rstd"], p["ln_g"])
    grads = {"ln_g": dg, "ln_b": dbeta, "w_in": dw_in, "b_in": db_in,
             "w_out": dw_out, "b_out": g.sum(axis=0)}
    inter = {"do": do, "dqkv": dqkv, "dln": dln}
    return dx, grads, inter


def mlp_half_fwd(sh: LayerShape, x1: np.ndarray, p: dict, store=None):
    """MLP half of slice i: partial = GeLU(LN2(x1) A_i + a_i) B_i (no bias, no residual).

    store: as in attn_half_fwd; the kept tensors are LN2(x1), the
    pre-activation U and Y = GeLU(U) (Y formed from the unrounded U, then
    rounded, as a bias+GeLU epilogue does).
    """
    rnd = store or _keep
    y, mean, rstd, xhat = layernorm_fwd(x1, p["ln_g"], p["ln_b"], sh.eps)
    y = rnd(y)
    u = y @ p["w_in"] + p["b_in"][None, :]
    act = rnd(gelu(u))
    u = rnd(u)
    partial = act @ p["w_out"]
    saved = {"ln_out": y, "mean": mean, "rstd": rstd, "xhat": xhat, "u": u, "y": act}
    return partial, saved


def mlp_half_bwd(sh: LayerShape, g: np.ndarray, p: dict, saved: dict):
    """Backward of the MLP half of slice i (same conventions as attn_half_bwd).

    dY = g B_i^T; dB_i = Y^T g; dU = dY * GeLU'(U); da_i = column sums of dU;
    dA_i = LN2(x1)^T dU; dLN = dU A_i^T; dx_partial = LN backward of dLN.
    """
    dy = g @ p["w_out"].T
    dw_out = saved["y"].T @ g
    du = dy * gelu_grad(saved["u"])
    dw_in = saved["ln_out"].T @ du
    db_in = du.sum(axis=0)
    dln = du @ p["w_in"].T
    dx, dg, dbeta = layernorm_bwd(dln, saved["xhat"], saved["rstd"], p["ln_g"])
    grads = {"ln_g": dg, "ln_b": dbeta, "w_in": dw_in, "b_in": db_in,
             "w_out": dw_out, "b_out": g.sum(axis=0)}
    inter = {"dy": dy, "du": du, "dln": dln}
    return dx, grads, inter


# --------------------------------------------------------------------------
# The whole layer: t slices run in turn, partials summed (what g computes)
# --------------------------------------------------------------------------

def reduce_partials(partials, residual: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """g forward (and f backward) on one device: residual + bias + sum of partials."""
    out = residual.copy()
    for part in partials:
        out = out + part
    if bias is not None:
        out = out + bias[None, :]
    return out


def layer_fwd(sh: LayerShape, x: np.ndarray, full: dict, attn_drop=None):
    """Full layer output from sh.tp slices run in turn. Returns (out, state).

    attn_drop: None, or (p, seed, site) for dropout on the attention
    probabilities (slice i's heads are global heads i*H/t .. (i+1)*H/t - 1).
    """
    sh.check()
    t = sh.tp
    ap = [attn_slice(sh, full, i) for i in range(t)]
    mp = [mlp_slice(sh, full, i) for i in range(t)]
    drops = [None if attn_drop is None else (*attn_drop, i * sh.local_heads) for i in range(t)]
    a_fwd = [attn_half_fwd(sh, x, ap[i], attn_drop=drops[i]) for i in range(t)]
    x1 = reduce_partials([r[0] for r in a_fwd], x, full["b_o"])
    m_fwd = [mlp_half_fwd(sh, x1, mp[i]) for i in range(t)]
    out = reduce_partials([r[0] for r in m_fwd], x1, full["b_b"])
    state = {"ap": ap, "mp": mp, "a_saved": [r[1] for r in a_fwd],
             "m_saved": [r[1] for r in m_fwd], "x1": x1,
             "a_part": [r[0] for r in a_fwd], "m_part": [r[0] for r in m_fwd]}
    return out, state


def layer_fwd_rows(sh: LayerShape, x_seq: np.ndarray, full: dict, rows) -> np.ndarray:
    """Output rows of the unsliced layer for some positions of ONE sequence.

    x_seq is one sequence [seq, h]; `rows` are positions in it. The same
    definition as layer_fwd with one slice (pre-LN block, causal attention of
    all heads, GeLU MLP, biases and residuals), computed only where the
    requested rows need it: keys and values for every position up to the last
    requested row, everything else for the requested rows alone. Used to check
    layers too large for the full oracle on sampled rows.
    """
    h, nh, d = sh.hidden, sh.heads, sh.head_dim
    rows = np.asarray(rows, dtype=np.int64)
    last = int(rows.max()) + 1
    x_seq = np.asarray(x_seq, dtype=np.float64)
    y, _, _, _ = layernorm_fwd(x_seq[:last], full["ln1_g"], full["ln1_b"], sh.eps)
    w_qkv = full["w_qkv"]
    b_qkv = np.asarray(full["b_qkv"], dtype=np.float64)
    k = y @ np.asarray(w_qkv[:, h:2 * h], dtype=np.float64) + b_qkv[h:2 * h]
    v = y @ np.asarray(w_qkv[:, 2 * h:], dtype=np.float64) + b_qkv[2 * h:]
    q = y[rows] @ np.asarray(w_qkv[:, :h], dtype=np.float64) + b_qkv[:h]
    k = k.reshape(last, nh, d)
    v = v.reshape(last, nh, d)
    o = np.empty((len(rows), h))
    for j, r in enumerate(rows):
        qr = q[j].reshape(nh, d)
        s = np.einsum("chd,hd->hc", k[:r + 1], qr) / np.sqrt(d)    # [heads, visible keys]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[j] = np.einsum("hc,chd->hd", p, v[:r + 1]).reshape(h)
    x1 = x_seq[rows] + o @ np.asarray(full["w_o"], dtype=np.float64) + full["b_o"]
    y2, _, _, _ = layernorm_fwd(x1, full["ln2_g"], full["ln2_b"], sh.eps)
    u = y2 @ np.asarray(full["w_a"], dtype=np.float64) + full["b_a"]
    return x1 + gelu(u) @ np.asarray(full["w_b"], dtype=np.float64) + full["b_b"]


def layer_bwd(sh: LayerShape, g: np.ndarray, full: dict, state: dict):
    """Gradients of L = <Out, g> for the full layer, assembled from t slices.

    Returns (dx, grads) with grads keyed like the full parameters: column- and
    row-sliced weights are reassembled from the slices, replicated LayerNorm
    parameters get the sum of the slice partials, and the row-sliced biases
    the (replicated) column sums.
    """
    t = sh.tp
    m_b = [mlp_half_bwd(sh, g, state["mp"][i], state["m_saved"][i]) for i in range(t)]
    g1 = reduce_partials([r[0] for r in m_b], g, None)
    a_b = [attn_half_bwd(sh, g1, state["ap"][i], state["a_saved"][i]) for i in range(t)]
    dx = reduce_partials([r[0] for r in a_b], g1, None)

    h, f = sh.hidden, sh.ffn
    grads = {k: np.zeros(s) for k, s in full_param_shapes(sh).items()}
    w = sh.local_width
    fl = sh.local_ffn
    for i in range(t):
        ga = a_b[i][1]
        gm = m_b[i][1]
        cols = qkv_columns(sh, i)
        grads["ln1_g"] += ga["ln_g"]
        grads["ln1_b"] += ga["ln_b"]
        grads["w_qkv"][:, cols] = ga["w_in"]
        grads["b_qkv"][cols] = ga["b_in"]
        grads["w_o"][i * w:(i + 1) * w, :] = ga["w_out"]
        grads["ln2_g"] += gm["ln_g"]
        grads["ln2_b"] += gm["ln_b"]
        grads["w_a"][:, i * fl:(i + 1) * fl] = gm["w_in"]
        grads["b_a"][i * fl:(i + 1) * fl] = gm["b_in"]
        grads["w_b"][i * fl:(i + 1) * fl, :] = gm["w_out"]
    grads["b_o"] = a_b[0][1]["b_out"].copy()
    grads["b_b"] = m_b[0][1]["b_out"].copy()
    assert grads["w_qkv"].shape == (h, 3 * h) and grads["w_b"].shape == (f, h)
    return dx, grads


def layer_loss(sh: LayerShape, x: np.ndarray, full: dict, g: np.ndarray, attn_drop=None) -> float:
    """L = <Out, g>: the upstream gradient g stands in for a loss (a single layer has none)."""
    out, _ = layer_fwd(sh, x, full, attn_drop)
    return float((out * g).sum())
