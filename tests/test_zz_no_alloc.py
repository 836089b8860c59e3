"""The Adam step that allocates nothing (mtnlg_adam_step_noalloc: its norm
partials live in the library's static per-GPU scratch) against the Adam step
with a caller workspace (mtnlg_adam_step), through the C ABI: the same kernels
on the same inputs, so master, m, v, the bf16 weights and the statistics must
be bit-identical. Two calls in a row, the second over fewer parameters (the
scratch keeps the first call's partials; the second must not read them), and
a third whose gradient holds an infinity (the step is skipped, nothing but the
statistics is written).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tensor_sliced_transformer_amd as tst  # noqa: E402


def _state(n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    master = torch.randn(n, device="cuda", generator=g).mul_(0.02)
    m = torch.randn(n, device="cuda", generator=g).mul_(1e-3)
    v = torch.randn(n, device="cuda", generator=g).mul_(1e-3).square_()
    acc = torch.randn(n, device="cuda", generator=g).mul_(2e-3)
    return master, m, v, acc


def _run(noalloc, n, seed, cfg, poison=False):
    master, m, v, acc = _state(n, seed)
    if poison:
        acc[n // 3] = float("inf")
    w = torch.full((n,), -1.0, dtype=torch.bfloat16, device="cuda")
    stats = torch.full((3,), -7.0, dtype=torch.float32, device="cuda")
    if noalloc:
        tst.adam_step_noalloc(cfg, master, m, v, acc, w, stats)
    else:
        ws = torch.empty(tst.adam_workspace_bytes(n), dtype=torch.uint8, device="cuda")
        tst.adam_step(cfg, master, m, v, acc, w, stats, ws)
    torch.cuda.synchronize()
    return {"master": master, "m": m, "v": v, "w": w, "stats": stats}


def test_adam_noalloc_matches_workspace_entry_point():
    assert tst.adam_static_scratch_bytes() == 8192 * 12
    cfg = tst.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 7)
    for n, seed, poison in ((3_000_007, 11, False), (10_007, 12, False), (65_541, 13, True)):
        print(f"adam noalloc n={n} poison={poison}", flush=True)
        ref = _run(False, n, seed, cfg, poison)
        got = _run(True, n, seed, cfg, poison)
        st = got["stats"].cpu().numpy()
        if poison:
            assert st[2] == 1.0
            fresh = _state(n, seed)
            assert torch.equal(got["master"], fresh[0]) and torch.equal(got["m"], fresh[1])
            assert torch.equal(got["v"], fresh[2])
            assert bool((got["w"] == -1.0).all())
        else:
            assert st[2] == 0.0 and 0.0 < st[1] <= 1.0, st
            assert (st[1] < 1.0) == (n > 1_000_000), st  # clipped on the large share only
        for k in ref:
            assert torch.equal(torch.nan_to_num(got[k].float(), nan=123.0),
                               torch.nan_to_num(ref[k].float(), nan=123.0)), (n, k)
