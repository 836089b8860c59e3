"""The oracle's page arithmetic against the numbers the pages print (tests/golden)."""
import json
import os

from oracle import pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_parameter_count_matches_530b():
    g = load()["model"]
    n = pages.decoder_params(g["layers"], g["hidden"])
    assert abs(n / 1e9 - g["params_billion"]) < 0.01 * g["params_billion"]   # 528.5 vs 530


def test_twenty_bytes_per_param_exceeds_10tb():
    g = load()
    tb = pages.optimizer_bytes(g["model"]["params_billion"] * 1e9, g["optimizer_memory"]["bytes_per_param"]) / 1e12
    assert tb > g["optimizer_memory"]["total_more_than_TB"]
    assert abs(tb - 10.6) < 0.05


def test_activation_memory():
    g = load()["activation_memory"]
    per_mb = pages.checkpointed_activation_bytes()
    assert abs(per_mb / 1e9 - g["after_GB"]) < 0.05
    assert abs(per_mb * g["micro_batches"] / 1e12 - g["before_TB"]) < 0.05


def test_throughput_rows():
    g = load()["throughput"]
    for row in g["rows"]:
        tf = pages.tflops_per_gpu(row["iter_s"], row["nodes"], g["gpus_per_node"])
        # the FLOP formula is not printed on the pages; it reproduces them to within 1%
        assert abs(tf - row["tflops_per_gpu"]) < 0.01 * row["tflops_per_gpu"], (row, tf)


def test_pipeline_share_of_one_gpu():
    """8-way slicing x 35-way pipeline: a GPU holds 3 layers' 1/8 slices ~ 530e9/280."""
    g = load()
    lay = g["parallel_layout"]
    assert lay["tensor_slicing"] * lay["pipeline"] == lay["gpus_per_replica"]
    share = 3 * pages.shard_gemm_params(g["model"]["hidden"], lay["tensor_slicing"])
    assert share == 1_887_436_800
    assert abs(share - g["model"]["params_billion"] * 1e9 / lay["gpus_per_replica"]) / share < 0.01
    assert g["model"]["layers"] // lay["pipeline"] == 3


def test_shard_flops():
    f = pages.shard_fwd_flops(tokens=2048, hidden=20480, heads_local=16, head_dim=160,
                              ffn_local=10240, seq=2048, batch=1)
    assert f == 2_598_465_699_840
    assert 3 * f == 7_795_397_099_520
