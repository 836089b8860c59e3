"""The pages' own arithmetic, restated so that tests can pin it to the printed numbers.

TEST INFRASTRUCTURE ONLY.

* Model: 105 layers, hidden 20480, 128 heads, 530B parameters (jiqizhixin
  MT-NLG article, model paragraph; Elamur summary, "Key points").
* ~20 bytes/param for mixed-precision Adam, > 10 TB in total (Elamur summary,
  "Key points").
* Peak activation memory 16.9 TB reduced to 8.8 GB by 1920 micro-batches
  (Elamur summary, "Key points"); sequence length 2048 is not on the pages.
* 126 / 121 / 113 TFLOP/s per GPU at 280 / 350 / 420 DGX A100 nodes (8 GPUs
  each), batch 1920, iteration 60.1 / 50.2 / 44.4 s (jiqizhixin article,
  throughput paragraph). The FLOP count per iteration used to reproduce them,
  96 B s l h^2 (1 + s/(6h)), is not on the pages (it counts the forward four
  times, i.e. with activation recomputation, and dense attention).
"""
from __future__ import annotations

LAYERS = 105
HIDDEN = 20480
HEADS = 128
BATCH = 1920
SEQ = 2048  # reading: not on the pages


def decoder_params(layers: int = LAYERS, hidden: int = HIDDEN) -> float:
    """Weights of the decoder stack: 12 l h^2 (4h^2 attention + 8h^2 MLP, biases ignored)."""
    return 12.0 * layers * hidden * hidden


def optimizer_bytes(params: float, bytes_per_param: float = 20.0) -> float:
    return params * bytes_per_param


def checkpointed_activation_bytes(layers=LAYERS, seq=SEQ, hidden=HIDDEN, elem_bytes=2) -> float:
    """Layer inputs kept for one micro-batch of one sequence: l * s * h * 2 B."""
    return float(layers) * seq * hidden * elem_bytes


def iteration_flops(batch=BATCH, seq=SEQ, layers=LAYERS, hidden=HIDDEN) -> float:
    """96 B s l h^2 (1 + s / 6h): forward counted 4x, dense attention."""
    return 96.0 * batch * seq * layers * hidden * hidden * (1.0 + seq / (6.0 * hidden))


def tflops_per_gpu(iter_seconds: float, nodes: int, gpus_per_node: int = 8) -> float:
    return iteration_flops() / (iter_seconds * nodes * gpus_per_node) / 1e12


def shard_gemm_params(hidden=HIDDEN, tp=8) -> int:
    """GEMM parameters of one 1/tp slice of a layer: QKV + out-proj + A + B."""
    h = hidden
    return h * (3 * h // tp) + (h // tp) * h + h * (4 * h // tp) + (4 * h // tp) * h


def shard_fwd_flops(tokens: int, hidden: int, heads_local: int, head_dim: int,
                    ffn_local: int, seq: int, batch: int, causal: bool = True) -> float:
    """Forward FLOPs (2 per multiply-add) of one slice: four GEMMs plus attention.

    Causal attention counts the visible pairs only: seq*(seq+1)/2 per sequence.
    """
    w = heads_local * head_dim
    gemm = 2.0 * tokens * (hidden * 3 * w + w * hidden + hidden * ffn_local + ffn_local * hidden)
    pairs = seq * (seq + 1) / 2.0 if causal else float(seq * seq)
    attn = 4.0 * batch * heads_local * head_dim * pairs
    return gemm + attn
