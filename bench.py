#!/usr/bin/env python3
"""Throughput of one GPU's 1/8 tensor slice of an MT-NLG decoder layer on MI355X.

One timed step = the forward and backward of the slice (hidden 20480, 16 of 128
heads x 160, MLP slice 10240, one sequence of 2048 tokens, bf16): LayerNorm,
QKV, causal attention and output projection, the local partial sum (residual +
bias), LayerNorm, MLP up + GeLU and down, the local partial sum, then the
backward of both halves including the input-gradient sums. `value` is the
algorithmic FLOP count of the step (GEMMs plus causal attention, 2 per
multiply-add, 7.795e12) divided by the step time.

Also measured in the same run:
  * the same step with activation recompute (each half's backward re-runs its
    forward from the half's input);
  * the optimizer over one GPU's share of the 530B model (1,887,436,800
    parameters): fp32 accumulation of 4 bf16 micro-batch gradients, then the
    fused unscale + global-norm clip + Adam step, as HBM GB/s;
  * one pipeline stage (3 chained layer slices, 4 micro-batches, gradient
    accumulation with the norm folded into the last pass, Adam), with and
    without activation recompute, as TFLOP/s of the model FLOPs;
  * each GEMM launch of the step alone (HIP events on the stream it runs on)
    for the roofline of the GEMM kernel;
  * the float64 CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-adam] [--no-recompute] [--no-stage] [--no-layers] [--no-components]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import statistics
import os
import sys
import time

import numpy as np

METRIC = "TFLOP/s per GPU, MT-NLG layer shard fwd+bwd bf16 (% MFMA peak); Adam GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ADAM_N = 1_887_436_800        # 3 layers x 629,145,600 slice parameters


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-adam", action="store_true")
    ap.add_argument("--adam-reps", type=int, default=5)
    ap.add_argument("--no-recompute", action="store_true")
    ap.add_argument("--no-stage", action="store_true")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the GPT-style h4096 layer and the full MT-NLG layer as 8 slices")
    ap.add_argument("--no-components", action="store_true",
                    help="skip the LayerNorm / partial-sum / attention kernels timed alone")
    ap.add_argument("--no-clock", action="store_true", help="skip the amdsmi clock and power sample")
    ap.add_argument("--stage-steps", type=int, default=3)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 512 MiB device copy (to scale HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's tensor slice on one GPU; the library has no multi-GPU "
              "path, so only --gpus 1 runs (requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch
    import tensor_sliced_transformer_amd as tst
    from synth.inputs import WORKLOADS, make_activation, make_half_params

    tst.load()  # fail loudly if the library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)    # 512 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 536870912 bytes read and written")
        del src, dst
    w = WORKLOADS[3]
    T, h, wl, fl = w.tokens, w.hidden, w.local_width, w.local_ffn
    desc = tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, w.tp, 0, tst.BF16, 1e-5)

    log("generating seeded inputs (1/8 shard, h 20480)")
    t0 = time.time()
    pa_np = make_half_params(w, "attn", 0)
    pm_np = make_half_params(w, "mlp", 0)
    x_np = make_activation(w, 1)
    g_np = make_activation(w, 2)

    def dev_bf16(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    pa = {k: dev_bf16(v) for k, v in pa_np.items()}
    pm = {k: dev_bf16(v) for k, v in pm_np.items()}
    x = dev_bf16(x_np)
    g = dev_bf16(g_np)
    log(f"inputs ready in {time.time() - t0:.1f}s")

    def zeros_like_params(p):
        return {k: torch.empty_like(v) for k, v in p.items()}

    ga, gm = zeros_like_params(pa), zeros_like_params(pm)
    sav_a = torch.empty(tst.saved_bytes(desc, tst.ATTN), dtype=torch.uint8, device=dev)
    sav_m = torch.empty(tst.saved_bytes(desc, tst.MLP), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(tst.workspace_bytes(desc, tst.ATTN), tst.workspace_bytes(desc, tst.MLP)),
                     dtype=torch.uint8, device=dev)
    part = torch.empty((T, h), dtype=torch.bfloat16, device=dev)
    x1 = torch.empty_like(part)
    out = torch.empty_like(part)
    dxp = torch.empty_like(part)
    g1 = torch.empty_like(part)
    dx = torch.empty_like(part)
    pa_call = {k: v for k, v in pa.items() if k != "b_out"}
    pm_call = {k: v for k, v in pm.items() if k != "b_out"}

    def step():
        tst.layer_fwd(desc, tst.ATTN, pa_call, x, part, sav_a, ws)
        tst.reduce_partials([part], x1, residual=x, bias=pa["b_out"])
        tst.layer_fwd(desc, tst.MLP, pm_call, x1, part, sav_m, ws)
        tst.reduce_partials([part], out, residual=x1, bias=pm["b_out"])
        tst.layer_bwd(desc, tst.MLP, pm_call, x1, sav_m, g, dxp, gm, ws)
        tst.reduce_partials([dxp], g1, residual=g)
        tst.layer_bwd(desc, tst.ATTN, pa_call, x, sav_a, g1, dxp, ga, ws)
        tst.reduce_partials([dxp], dx, residual=g1)

    flops = 3.0 * shard_fwd_flops(T, h, w.local_heads, w.head_dim, fl, w.seq, w.batch)
    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one event before every step (and one after the last): the mean over the
    # K steps is `value`; the per-step median and minimum are reported beside it
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    start, end = evs[0], evs[-1]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i].record()
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    ms_min = per_step[0]
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"fwd+bwd step {ms:.3f} ms = {tflops:.1f} TFLOP/s (median {ms_median:.3f}, min {ms_min:.3f} ms)")
    # the same step under the other counting conventions: dense attention
    # (every query against every key), and the 4x-forward count of a step that
    # recomputes the forward (the convention of the throughput figures the
    # MT-NLG news article quotes)
    fwd_dense = shard_fwd_flops(T, h, w.local_heads, w.head_dim, fl, w.seq, w.batch, causal=False)

    # ---- GPU clock and power while the step runs (not part of the timed region) ----
    clocks = None if args.no_clock else clock_sample(torch, step, ms, settle=1.0)
    if clocks and clocks["gfx_clock_mhz"]:
        peak_at_clock = PEAK_BF16_TFLOPS * clocks["gfx_clock_mhz"] / 2400.0
        clocks["mfma_peak_frac_at_clock"] = round(tflops / peak_at_clock, 4)
        log(f"under load: GPU clock {clocks['gfx_clock_mhz']:.0f} MHz, {clocks['socket_power_w']} W; "
            f"{100 * tflops / peak_at_clock:.1f}% of the peak at that clock")

    # ---- the same step with the backward recomputing each half's forward from
    # its input (only the layer inputs are kept between forward and backward) ----
    rc = None
    if not args.no_recompute:
        ws_rc = torch.empty(max(tst.recompute_workspace_bytes(desc, tst.ATTN),
                                tst.recompute_workspace_bytes(desc, tst.MLP)), dtype=torch.uint8, device=dev)

        def step_rc():
            tst.layer_fwd(desc, tst.ATTN, pa_call, x, part, sav_a, ws)
            tst.reduce_partials([part], x1, residual=x, bias=pa["b_out"])
            tst.layer_fwd(desc, tst.MLP, pm_call, x1, part, sav_m, ws)
            tst.reduce_partials([part], out, residual=x1, bias=pm["b_out"])
            tst.layer_bwd_recompute(desc, tst.MLP, pm_call, x1, g, dxp, gm, ws_rc)
            tst.reduce_partials([dxp], g1, residual=g)
            tst.layer_bwd_recompute(desc, tst.ATTN, pa_call, x, g1, dxp, ga, ws_rc)
            tst.reduce_partials([dxp], dx, residual=g1)

        for _ in range(args.warmup):
            step_rc()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            step_rc()
        end.record()
        torch.cuda.synchronize()
        ms_rc = start.elapsed_time(end) / args.steps
        # executed work: the step plus a second forward without the two output GEMMs
        hw_flops = flops + flops / 3.0 - 2.0 * T * h * (wl + fl)
        rc = {"ms_per_step": round(ms_rc, 4),
              "model_tflops": round(flops / (ms_rc * 1e-3) / 1e12, 2),
              "executed_tflops": round(hw_flops / (ms_rc * 1e-3) / 1e12, 2),
              "executed_flop_per_step": hw_flops,
              "four_x_forward_tflops": round(4.0 * fwd_dense / (ms_rc * 1e-3) / 1e12, 2),
              "four_x_forward_flop_per_step": 4.0 * fwd_dense,
              "note": "model_tflops counts the step's 3x-forward FLOPs; executed_tflops adds "
                      "the recomputed forward (output GEMMs skipped); four_x_forward_tflops uses the "
                      "4x-forward, dense-attention count of the MT-NLG throughput figures"}
        log(f"recompute step {ms_rc:.3f} ms = {rc['model_tflops']} model / {rc['executed_tflops']} "
            f"executed TFLOP/s")
        del ws_rc


    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": "mtnlg-shard-h20480-t8-bf16 fwd+bwd", "tokens": T, "hidden": h,
                   "local_heads": w.local_heads, "head_dim": w.head_dim, "local_ffn": fl, "causal": True,
                   "flop_per_step": flops},
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_median": round(ms_median, 4),
        "ms_per_step_min": round(ms_min, 4),
        "clocks": clocks,
        "dense_attention_convention": {
            "tflops": round(3.0 * fwd_dense / (ms * 1e-3) / 1e12, 2), "flop_per_step": 3.0 * fwd_dense,
            "note": "the same step time over the FLOP count with attention counted dense (every query "
                    "against every key); value counts only the causal half"},
    }
    if rc is not None:
        result["recompute"] = rc
    del pa, pm, ga, gm, sav_a, sav_m, ws
    torch.cuda.empty_cache()

    if not args.no_adam:
        result["adam"] = adam_bench(torch, tst, dev, args.adam_reps)

    if not args.no_stage:
        result["stage"] = stage_bench(torch, tst, dev, args.stage_steps, 1, flops, False)
        result["stage_recompute"] = stage_bench(torch, tst, dev, args.stage_steps, 1, flops, True)

    if not args.no_layers:
        torch.cuda.empty_cache()
        result["gpt_layer_h4096"] = layer_bench(torch, tst, dev, 2, args.steps, args.warmup)
        torch.cuda.empty_cache()
        result["full_layer_8_slices_b4"] = layer_bench(torch, tst, dev, 5, 3, 1)
        torch.cuda.empty_cache()

    if not args.no_components:
        result["components"] = component_bench(torch, tst, dev, T, h, w.local_heads, w.head_dim)

    # ---- each GEMM launch of the step alone (same shapes and operand layouts),
    # last so that a kernel trace of this script ends with these launches ----
    gemm_rows = gemm_breakdown(torch, tst, dev, T, h, wl, fl)
    g_fl = sum(r["flop"] for r in gemm_rows)
    g_ms = sum(r["ms"] for r in gemm_rows)
    gemm_tflops = g_fl / (g_ms * 1e-3) / 1e12
    log(f"GEMMs alone: {g_ms:.3f} ms of the step, {gemm_tflops:.1f} TFLOP/s")
    result["roofline"] = {
        "bound": "mfma",
        "kernel": "gemm_bf16_rs_kernel (NN, NT) and gemm_bf16_dtl64_kernel (TN), + tail_reduce_kernel (the 12 GEMM launches of one step)",
        "achieved": round(gemm_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4), "traffic": gemm_traffic_bytes(),
        "traffic_unit": "bytes per launch (average over the 12 launches)",
        "traffic_source": "profiles/gemm_traffic.json: two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE) "
                          "over the same 12 launches, scaled by a plain copy's readings; recorded with the "
                          "sha256 of gemm.hip and reported as null when the source has changed since",
        "algorithmic_bytes": sum(2 * (r["M"] * r["K"] + r["K"] * r["N"] + r["M"] * r["N"])
                                 for r in gemm_rows) / len(gemm_rows),
        "launches": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in gemm_rows]}

    if not args.no_clock:
        result["roofline"]["power_probe"] = gemm_power_probe(torch, tst, dev, T, h, fl)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pa_np, pm_np, x_np, g_np)

    print(json.dumps(result), flush=True)


def gemm_traffic_bytes():
    """HBM bytes per GEMM launch from the committed counter passes, or None when the GEMM
    source has changed since those counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(root, "profiles", "gemm_traffic.json")))
        src = open(os.path.join(root, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec["avg_bytes_per_launch"]


_SMI = []


def _smi_handle():
    """The amdsmi library and the handle of the GPU torch calls device 0 (queried
    in-process: no external program is started from a process that uses the GPU)."""
    if not _SMI:
        import amdsmi
        import torch
        try:
            h = torch.cuda._get_amdsmi_handler(0)
        except Exception:
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]
        _SMI.append((amdsmi, h))
    return _SMI[0]


def smi_sample():
    """(mean GPU core clock over the XCDs in MHz, memory clock in MHz, socket power in W)
    from the amdsmi library, or None where it is not available."""
    def num(v):
        return v if isinstance(v, (int, float)) and not isinstance(v, bool) and 0 < v < 65535 else None
    try:
        amdsmi, h = _smi_handle()
        gfx = None
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            xcd = [c for c in (num(v) for v in m.get("current_gfxclks", []) or []) if c is not None]
            gfx = sum(xcd) / len(xcd) if xcd else None
        except Exception:
            pass
        if gfx is None:
            ci = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            gfx = num(ci.get("clk", ci.get("cur_clk")))
        mi = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)
        mem = num(mi.get("clk", mi.get("cur_clk")))
        pi = amdsmi.amdsmi_get_power_info(h)
        pw = num(pi.get("current_socket_power"))
        if pw is None:
            pw = num(pi.get("average_socket_power"))
        return (gfx, mem, pw) if gfx is not None else None
    except Exception:
        return None


def clock_sample(torch, step, ms_step, seconds=1.5, settle=0.0):
    """Runs the step back to back for about `seconds` while amdsmi is polled from a
    second thread; the medians of the samples taken while the GPU is busy. With
    `settle` > 0 the step first runs that many seconds unsampled: the driver's
    clock and power readings trail the load by up to about a second, so a
    window right after a change of workload reads the previous one."""
    import threading
    samples, stop = [], threading.Event()
    if settle > 0:
        for _ in range(max(1, int(settle * 1e3 / ms_step))):
            step()

    def poll():
        while not stop.is_set():
            s = smi_sample()
            if s is None:
                return
            samples.append(s)
            stop.wait(0.02)

    n = max(1, int(seconds * 1e3 / ms_step))
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    for _ in range(n):
        step()
    th.start()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None

    def med(i):
        v = sorted(s[i] for s in samples if s[i] is not None)
        return v[len(v) // 2] if v else None
    return {"gfx_clock_mhz": med(0), "mem_clock_mhz": med(1), "socket_power_w": med(2), "samples": len(samples),
            "steps": n}


def shard_fwd_flops(tokens, hidden, heads_local, head_dim, ffn_local, seq, batch, causal=True):
    wl = heads_local * head_dim
    gemm = 2.0 * tokens * (hidden * 3 * wl + wl * hidden + hidden * ffn_local + ffn_local * hidden)
    pairs = seq * (seq + 1) / 2.0 if causal else float(seq) * seq
    attn = 4.0 * batch * heads_local * head_dim * pairs
    return gemm + attn


def layer_bench(torch, tst, dev, wi, steps, warmup):
    """A layer (or one slice of it) as a step over its slices in turn: the
    forward of every slice's attention half, their partials summed with the
    bias and residual, the same for the MLP half, then the backward of the MLP
    halves and of the attention halves, each followed by the sum of the slices'
    input-gradient partials; the slices' LayerNorm gradients are summed too.
    Weights and inputs are drawn on the GPU with the workload's distributions
    (seeded; throughput does not depend on their values)."""
    from synth.inputs import WORKLOADS, half_param_shapes
    w = WORKLOADS[wi]
    T, h = w.tokens, w.hidden
    log(f"layer workload {w.name}: {len(w.slices)} slice(s), {T} tokens")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5000 + wi)
    bf = torch.bfloat16

    def rn(shape, std, mean=0.0):
        return (torch.randn(shape, device=dev, generator=gen) * std + mean).to(bf)

    def params(half):
        return {k: rn(shp, 0.02, 1.0 if k == "ln_g" else 0.0) for k, shp in half_param_shapes(w, half).items()}

    descs = [tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, w.tp, i, tst.BF16, 1e-5) for i in w.slices]
    pa = [params("attn") for _ in w.slices]
    pm = [params("mlp") for _ in w.slices]
    for p in pa[1:]:  # LayerNorm parameters and the row-sliced bias are replicated across slices
        for k in ("ln_g", "ln_b", "b_out"):
            p[k] = pa[0][k]
    for p in pm[1:]:
        for k in ("ln_g", "ln_b", "b_out"):
            p[k] = pm[0][k]
    pa_call = [{k: v for k, v in p.items() if k != "b_out"} for p in pa]
    pm_call = [{k: v for k, v in p.items() if k != "b_out"} for p in pm]
    ga = [{k: torch.empty_like(v) for k, v in p.items()} for p in pa]
    gm = [{k: torch.empty_like(v) for k, v in p.items()} for p in pm]
    d0 = descs[0]
    sav_a = [torch.empty(tst.saved_bytes(d0, tst.ATTN), dtype=torch.uint8, device=dev) for _ in w.slices]
    sav_m = [torch.empty(tst.saved_bytes(d0, tst.MLP), dtype=torch.uint8, device=dev) for _ in w.slices]
    ws = torch.empty(max(tst.workspace_bytes(d0, tst.ATTN), tst.workspace_bytes(d0, tst.MLP)),
                     dtype=torch.uint8, device=dev)
    x, g = rn((T, h), 1.0), rn((T, h), 1.0)
    parts = [torch.empty((T, h), dtype=bf, device=dev) for _ in w.slices]
    x1, out, g1, dx = (torch.empty((T, h), dtype=bf, device=dev) for _ in range(4))
    lng = {k: torch.empty((1, h), dtype=bf, device=dev) for k in ("a_g", "a_b", "m_g", "m_b")}
    n = len(w.slices)

    def step():
        for i in range(n):
            tst.layer_fwd(descs[i], tst.ATTN, pa_call[i], x, parts[i], sav_a[i], ws)
        tst.reduce_partials(parts, x1, residual=x, bias=pa[0]["b_out"])
        for i in range(n):
            tst.layer_fwd(descs[i], tst.MLP, pm_call[i], x1, parts[i], sav_m[i], ws)
        tst.reduce_partials(parts, out, residual=x1, bias=pm[0]["b_out"])
        for i in range(n):
            tst.layer_bwd(descs[i], tst.MLP, pm_call[i], x1, sav_m[i], g, parts[i], gm[i], ws)
        tst.reduce_partials(parts, g1, residual=g)
        for i in range(n):
            tst.layer_bwd(descs[i], tst.ATTN, pa_call[i], x, sav_a[i], g1, parts[i], ga[i], ws)
        tst.reduce_partials(parts, dx, residual=g1)
        if n > 1:
            for key, gs, name in (("a_g", ga, "ln_g"), ("a_b", ga, "ln_b"), ("m_g", gm, "ln_g"), ("m_b", gm, "ln_b")):
                tst.reduce_partials([q[name].view(1, h) for q in gs], lng[key])

    flop = 3.0 * n * shard_fwd_flops(T, h, w.local_heads, w.head_dim, w.local_ffn, w.seq, w.batch)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        evs[i].record()
        step()
    evs[-1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    tf = flop / (ms * 1e-3) / 1e12
    log(f"{w.name}: {ms:.3f} ms per fwd+bwd step = {tf:.1f} TFLOP/s")
    res = {"workload": w.name, "slices": n, "tokens": T, "hidden": h, "heads": w.heads, "ffn": w.ffn,
           "steps": steps, "ms_per_step": round(ms, 4), "tflops": round(tf, 2),
           "mfma_peak_frac": round(tf / PEAK_BF16_TFLOPS, 4), "flop_per_step": flop}
    del pa, pm, pa_call, pm_call, ga, gm, sav_a, sav_m, ws, parts
    return res


def gemm_breakdown(torch, tst, dev, T, h, wl, fl, reps=10):
    """Every GEMM of the step, launched alone through mtnlg_gemm with its shape and layout."""
    # (name, M, N, K, trans_a, trans_b)
    shapes = [("qkv", T, 3 * wl, h, 0, 0), ("out_proj", T, h, wl, 0, 0), ("mlp_up", T, fl, h, 0, 0),
              ("mlp_down", T, h, fl, 0, 0), ("mlp_dY", T, fl, h, 0, 1), ("mlp_dB", fl, h, T, 1, 0),
              ("mlp_dA", h, fl, T, 1, 0), ("mlp_dX", T, h, fl, 0, 1), ("attn_dO", T, wl, h, 0, 1),
              ("attn_dWo", wl, h, T, 1, 0), ("attn_dWqkv", h, 3 * wl, T, 1, 0), ("attn_dX", T, h, 3 * wl, 0, 1)]
    # operand distributions of the step (MFMA power, and with it the clock,
    # depends on the data): the B operand is a weight, N(0, 0.02), in the
    # forward and input-gradient products; both operands are activations or
    # gradients, N(0, 1), in the weight-gradient products
    weight_b = {"qkv", "out_proj", "mlp_up", "mlp_down", "mlp_dY", "mlp_dX", "attn_dO", "attn_dX"}
    rows = []
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    for name, M, N, K, ta, tb in shapes:
        a = torch.randn((K, M) if ta else (M, K), device=dev, generator=gen).to(torch.bfloat16)
        b = torch.randn((N, K) if tb else (K, N), device=dev, generator=gen)
        b = (b * 0.02 if name in weight_b else b).to(torch.bfloat16)
        c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(tst.gemm_workspace_bytes(tst.BF16, M, N, K), 16), dtype=torch.uint8, device=dev)
        for _ in range(2):
            tst.gemm(a, b, c, bool(ta), bool(tb), ws=ws)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            tst.gemm(a, b, c, bool(ta), bool(tb), ws=ws)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        fl_ = 2.0 * M * N * K
        rows.append({"name": name, "M": M, "N": N, "K": K, "layout": f"{'T' if ta else 'N'}{'T' if tb else 'N'}",
                     "ms": ms, "tflops": fl_ / (ms * 1e-3) / 1e12, "flop": fl_})
        del a, b, c, ws
    return rows


def gemm_power_probe(torch, tst, dev, T, h, fl, reps=20):
    """One GEMM of the step (the MLP input-gradient product, NT) run back to back
    with the step's operand distributions and again with all-zero operands: the
    same instructions, schedule and memory traffic, but the zero operands draw
    less MFMA power, so the GPU holds a higher clock under its power cap. The
    TFLOP/s and the sampled clock of the two runs show how much of the distance
    to the nominal peak is the clock (power) and how much the kernel."""
    M, N, K = T, fl, h
    out = {"gemm": f"mlp_dY {M}x{N}x{K} NT"}
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    a = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
    b = (torch.randn((N, K), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(tst.gemm_workspace_bytes(tst.BF16, M, N, K), 16), dtype=torch.uint8, device=dev)
    for kind in ("step_data", "zero_operands"):
        if kind == "zero_operands":
            a.zero_()
            b.zero_()

        def run():
            tst.gemm(a, b, c, False, True, ws=ws)

        for _ in range(5):
            run()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            run()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        ck = clock_sample(torch, run, ms, seconds=1.0, settle=1.5) or {}
        row = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
               "gfx_clock_mhz": ck.get("gfx_clock_mhz"), "socket_power_w": ck.get("socket_power_w")}
        if ck.get("gfx_clock_mhz"):
            row["frac_at_clock"] = round(tf / (PEAK_BF16_TFLOPS * ck["gfx_clock_mhz"] / 2400.0), 4)
        out[kind] = row
        log(f"power probe ({kind}): {tf:.1f} TFLOP/s at {row['gfx_clock_mhz']} MHz, {row['socket_power_w']} W")
    del a, b, c, ws
    return out


def adam_bench(torch, tst, dev, reps):
    """Optimizer over 1.887e9 parameters: accumulate 4 bf16 micro-batch grads, then the step."""
    n = ADAM_N
    log(f"optimizer workload: {n} parameters")
    gen = torch.Generator(device=dev)
    gen.manual_seed(4000)
    master = torch.randn(n, device=dev, generator=gen).mul_(0.02)
    m = torch.randn(n, device=dev, generator=gen).mul_(1e-3)
    v = torch.randn(n, device=dev, generator=gen).mul_(1e-3).square_()
    grads = [torch.randn(n, device=dev, generator=gen).mul_(1e-3).to(torch.bfloat16) for _ in range(4)]
    acc = torch.empty(n, dtype=torch.float32, device=dev)
    wbf = master.to(torch.bfloat16)
    stats = torch.zeros(3, dtype=torch.float32, device=dev)
    ws = torch.empty(tst.adam_workspace_bytes(n), dtype=torch.uint8, device=dev)
    cfg = tst.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 100)

    def accumulate():
        for k, gk in enumerate(grads):
            tst.grad_accumulate(gk, acc, overwrite=(k == 0))

    def opt_step():
        tst.adam_step(cfg, master, m, v, acc, wbf, stats, ws)

    accumulate()
    opt_step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_acc = t_step = 0.0
    for _ in range(reps):
        ev[0].record()
        accumulate()
        ev[1].record()
        opt_step()
        ev[2].record()
        torch.cuda.synchronize()
        t_acc += ev[0].elapsed_time(ev[1])
        t_step += ev[1].elapsed_time(ev[2])
    t_acc /= reps
    t_step /= reps
    st = stats.cpu().tolist()

    # the norm folded into the last accumulation, then the update alone
    def accumulate_norm():
        for k, gk in enumerate(grads):
            if k + 1 < len(grads):
                tst.grad_accumulate(gk, acc, overwrite=(k == 0))
            else:
                tst.grad_accumulate_norm(gk, acc, k == 0, cfg.inv_loss_scale, ws)

    def opt_update():
        tst.adam_update(cfg, master, m, v, acc, wbf, stats, ws)

    accumulate_norm()
    opt_update()
    torch.cuda.synchronize()
    f_acc = f_upd = 0.0
    for _ in range(reps):
        ev[0].record()
        accumulate_norm()
        ev[1].record()
        opt_update()
        ev[2].record()
        torch.cuda.synchronize()
        f_acc += ev[0].elapsed_time(ev[1])
        f_upd += ev[1].elapsed_time(ev[2])
    f_acc /= reps
    f_upd /= reps
    fused = {"accumulate_with_norm_ms": round(f_acc, 3), "update_ms": round(f_upd, 3),
             "update_GBps": round(30.0 * n / (f_upd * 1e-3) / 1e9, 1),
             "total_ms": round(f_acc + f_upd, 3), "unfused_total_ms": round(t_acc + t_step, 3),
             "bytes_per_param": 66, "unfused_bytes_per_param": 70}
    log(f"norm folded into the last accumulation: {f_acc:.2f} + update {f_upd:.2f} ms "
        f"(unfused {t_acc:.2f} + {t_step:.2f} ms)")
    # the update's ceiling: the same reads and writes (30 B per parameter), the
    # same launch, no optimizer arithmetic (mtnlg_adam_stream_reference)
    tst.adam_stream_reference(master, m, v, acc, wbf)
    torch.cuda.synchronize()
    t_ref = 0.0
    for _ in range(reps):
        ev[0].record()
        tst.adam_stream_reference(master, m, v, acc, wbf)
        ev[1].record()
        torch.cuda.synchronize()
        t_ref += ev[0].elapsed_time(ev[1])
    t_ref /= reps
    ref_gbs = 30.0 * n / (t_ref * 1e-3) / 1e9
    fused["stream_reference"] = {"ms": round(t_ref, 3), "GBps": round(ref_gbs, 1),
                                 "hbm_frac": round(ref_gbs / PEAK_HBM_GBS, 4),
                                 "update_vs_reference": round(fused["update_GBps"] / ref_gbs, 4),
                                 "note": "the update's reads and writes with no arithmetic "
                                         "(mtnlg_adam_stream_reference): the ceiling of that access mix"}
    log(f"update {fused['update_GBps']:.0f} GB/s vs its stream reference {ref_gbs:.0f} GB/s "
        f"({100 * fused['update_GBps'] / ref_gbs:.1f}%)")
    acc_gbs = 36.0 * n / (t_acc * 1e-3) / 1e9
    step_gbs = 34.0 * n / (t_step * 1e-3) / 1e9
    log(f"accumulate x4 {t_acc:.2f} ms = {acc_gbs:.0f} GB/s; step {t_step:.2f} ms = {step_gbs:.0f} GB/s; "
        f"stats {st}")
    out = {"n_params": n, "micro_batches": 4,
           "step_ms": round(t_step, 3), "step_GBps": round(step_gbs, 1),
           "step_hbm_frac": round(step_gbs / PEAK_HBM_GBS, 4), "step_bytes_per_param": 34,
           "accumulate_ms": round(t_acc, 3), "accumulate_GBps": round(acc_gbs, 1),
           "accumulate_hbm_frac": round(acc_gbs / PEAK_HBM_GBS, 4), "accumulate_bytes_per_param": 36,
           "grad_norm": st[0], "clip_coef": st[1], "found_inf": st[2], "fused_norm": fused}
    del master, m, v, grads, acc, wbf, ws
    torch.cuda.empty_cache()
    # what a plain device-to-device copy reaches on the same GPU in the same run
    # (the practical streaming ceiling the optimizer kernels are compared with)
    src = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    t_copy = ev[0].elapsed_time(ev[1]) / reps
    copy_gbs = 2.0 * src.numel() * 4 / (t_copy * 1e-3) / 1e9
    out["device_copy"] = {"bytes_moved": 2 * src.numel() * 4, "ms": round(t_copy, 3), "GBps": round(copy_gbs, 1),
                          "hbm_frac": round(copy_gbs / PEAK_HBM_GBS, 4),
                          "step_vs_copy": round(step_gbs / copy_gbs, 4),
                          "accumulate_vs_copy": round(acc_gbs / copy_gbs, 4),
                          "note": "torch's copy_ of 2 GiB fp32 (read + write counted), for context only: "
                                  "it is not the memory system's ceiling (hand-written streams copy faster)"}
    log(f"plain device copy: {copy_gbs:.0f} GB/s; Adam step at {100 * step_gbs / copy_gbs:.0f}% of it, "
        f"accumulation at {100 * acc_gbs / copy_gbs:.0f}%")
    del src, dst
    torch.cuda.empty_cache()
    return out


def component_bench(torch, tst, dev, T, h, heads, head_dim, reps=20):
    """The step's bandwidth-bound kernels and the attention kernels, each launched
    alone at the slice's shapes and timed with HIP events on the stream they run
    on: achieved GB/s against their algorithmic bytes (bf16 [T, h] tensors read or
    written once, fp32 row statistics), attention in TFLOP/s (causal count)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(7000)
    bf = torch.bfloat16

    def rn(*shape, scale=1.0):
        return (torch.randn(*shape, device=dev, generator=gen) * scale).to(bf)

    def timed(fn):
        # median of per-launch event intervals: one stall of the GPU (seen once
        # at 36 ms) must not stand in for the kernel's time
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return statistics.median(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))

    x, gy, part = rn(T, h), rn(T, h), rn(T, h)
    gamma, beta, bias = rn(h, scale=0.02), rn(h, scale=0.02), rn(h, scale=0.02)
    y, dx, out = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty(T, dtype=torch.float32, device=dev)
    rstd = torch.empty_like(mean)
    dgamma, dbeta = torch.empty_like(gamma), torch.empty_like(beta)
    lws = torch.empty(max(16, tst.layernorm_bwd_workspace_bytes(T, h)), dtype=torch.uint8, device=dev)
    tb = T * h * 2
    res = {}

    def bw(name, ms, nbytes, what):
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "bytes": nbytes, "GBps": round(gbs, 1),
                     "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_counted": what}

    bw("layernorm_fwd", timed(lambda: tst.layernorm_fwd(x, gamma, beta, 1e-5, y, mean, rstd)),
       2 * tb + 8 * T, "x read, y written, mean/rstd written")
    bw("layernorm_bwd", timed(lambda: tst.layernorm_bwd(gy, x, mean, rstd, gamma, dx, dgamma, dbeta, lws)),
       3 * tb + 8 * T, "dy and x read, dx written (+ row stats; gamma/beta grads are h-sized)")
    bw("reduce_partials", timed(lambda: tst.reduce_partials([part], out, residual=x, bias=bias)),
       3 * tb, "one partial and the residual read, the sum written")
    wl = heads * head_dim
    q32 = torch.randn(T, 3 * wl, device=dev, generator=gen) * 2.9
    # the bf16 path's storage of the attention input: Q and K in fp16, V in bf16
    qkv = torch.cat([q32[:, :2 * wl].to(torch.float16).view(bf), q32[:, 2 * wl:].to(bf)], dim=1).contiguous()
    del q32
    o = torch.empty(T, wl, dtype=bf, device=dev)
    lse = torch.empty(heads, T, dtype=torch.float32, device=dev)
    do, dqkv = rn(T, wl), torch.empty_like(qkv)
    aws = torch.empty(max(16, tst.attention_bwd_workspace_bytes(1, T, heads)), dtype=torch.uint8, device=dev)
    causal = 4.0 * heads * head_dim * (T * (T + 1) / 2.0)
    ms_f = timed(lambda: tst.attention_fwd(qkv, o, lse, 1, T, heads, head_dim))
    ms_b = timed(lambda: tst.attention_bwd(qkv, o, lse, do, dqkv, aws, 1, T, heads, head_dim))
    res["attention_fwd"] = {"us": round(ms_f * 1e3, 2), "flop": causal, "tflops": round(causal / (ms_f * 1e-3) / 1e12, 1)}
    res["attention_bwd"] = {"us": round(ms_b * 1e3, 2), "flop": 2 * causal,
                            "tflops": round(2 * causal / (ms_b * 1e-3) / 1e12, 1),
                            "note": "algorithmic count (dV, dP, dQ, dK); the recomputed scores are not counted"}
    log("components alone: " + ", ".join(
        f"{k} {v['us']:.1f} us" + (f" {v['GBps']:.0f} GB/s" if "GBps" in v else f" {v['tflops']:.0f} TFLOP/s")
        for k, v in res.items()))
    del x, gy, part, y, dx, out, qkv, o, do, dqkv, lws, aws
    torch.cuda.empty_cache()
    return res


def stage_bench(torch, tst, dev, steps, warmup, layer_flops, recompute):
    """One pipeline stage on one GPU: 3 chained 1/8 layer slices, 4 micro-batches of
    2048 tokens, gradient accumulation with the norm folded in, then Adam."""
    from synth.inputs import WORKLOADS
    w = WORKLOADS[7]
    L, MB = w.extra["layers"], w.extra["micro_batches"]
    ld = tst.make_desc(w.batch, w.seq, w.hidden, w.heads, w.ffn, w.tp, 0, tst.BF16, 1e-5)
    sd = tst.make_stage_desc(ld, L, MB, recompute)
    n = tst.stage_param_count(sd)
    offs = tst.stage_param_offsets(sd)
    log(f"stage: {L} layers x {MB} micro-batches, {n} parameters, recompute {recompute}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7000)
    master = torch.randn(n, device=dev, generator=gen).mul_(0.02)
    for lay in offs:
        for half in lay:
            master[half["ln_g"]:half["ln_g"] + w.hidden].add_(1.0)
    m = torch.randn(n, device=dev, generator=gen).mul_(1e-3)
    v = torch.randn(n, device=dev, generator=gen).mul_(1e-3).square_()
    wt = master.to(torch.bfloat16)
    grad = torch.empty(n, dtype=torch.bfloat16, device=dev)
    acc = torch.empty(n, dtype=torch.float32, device=dev)
    x = torch.randn((MB, w.tokens, w.hidden), device=dev, generator=gen).to(torch.bfloat16)
    dy = torch.randn((MB, w.tokens, w.hidden), device=dev, generator=gen).to(torch.bfloat16)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    stats = torch.zeros(3, dtype=torch.float32, device=dev)
    ws = torch.empty(tst.stage_workspace_bytes(sd), dtype=torch.uint8, device=dev)
    cfg = tst.AdamCfg(1e-4, 0.9, 0.95, 1e-8, 0.0, 1.0, 1.0, 100)
    aux = torch.cuda.Stream()  # the gradient accumulation overlaps the compute on it
    for _ in range(warmup):
        tst.stage_step(sd, cfg, wt, master, m, v, grad, acc, x, dy, y, dx, stats, ws, aux_stream=aux)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        tst.stage_step(sd, cfg, wt, master, m, v, grad, acc, x, dy, y, dx, stats, ws, aux_stream=aux)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = L * MB * layer_flops
    tflops = flops / (ms * 1e-3) / 1e12
    st = stats.cpu().tolist()
    log(f"stage step {ms:.2f} ms = {tflops:.1f} TFLOP/s (model FLOPs), stats {st}")
    out = {"layers": L, "micro_batches": MB, "tokens_per_micro_batch": w.tokens, "n_params": n,
           "recompute": bool(recompute), "steps": steps, "ms_per_step": round(ms, 3), "tflops": round(tflops, 2),
           "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4), "flop_per_step": flops,
           "workspace_bytes": tst.stage_workspace_bytes(sd), "grad_norm": st[0], "clip_coef": st[1],
           "found_inf": st[2]}
    del master, m, v, wt, grad, acc, x, dy, y, dx, ws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(pa_np, pm_np, x_np, g_np, sample_tokens=2048):
    """The float64 oracle (as it stands) on the same slice and the same 2048-token sequence (the
    whole workload of one step: about 10-30 s on the host cores)."""
    from threadpoolctl import threadpool_info
    from oracle import layer as OL
    sh = OL.LayerShape(batch=1, seq=sample_tokens, hidden=20480, heads=128, ffn=81920, tp=8)
    log(f"cpu baseline: oracle fwd+bwd of the slice on {sample_tokens} tokens")
    pa = {k: v.astype(np.float64) for k, v in pa_np.items()}
    pm = {k: v.astype(np.float64) for k, v in pm_np.items()}
    x = x_np[:sample_tokens].astype(np.float64)
    g = g_np[:sample_tokens].astype(np.float64)
    reps = 2  # two passes of the step: about 10-30 s on the machine's host cores
    t0 = time.perf_counter()
    for _ in range(reps):
        pa_part, sa = OL.attn_half_fwd(sh, x, pa)
        x1 = OL.reduce_partials([pa_part], x, pa["b_out"])
        pm_part, sm = OL.mlp_half_fwd(sh, x1, pm)
        dxm, _, _ = OL.mlp_half_bwd(sh, g, pm, sm)
        g1 = OL.reduce_partials([dxm], g, None)
        OL.attn_half_bwd(sh, g1, pa, sa)
    dt = time.perf_counter() - t0
    fl = reps * 3.0 * shard_fwd_flops(sample_tokens, 20480, 16, 160, 10240, sample_tokens, 1)
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    log(f"cpu baseline {dt:.1f}s, {fl / dt / 1e12:.3f} TFLOP/s on {threads} threads")

    # the GPT-style layer (hidden 4096, 32 heads of 128, MLP 16384, 2048 tokens,
    # one slice) in full: both halves forward and backward
    from synth.inputs import WORKLOADS, make_activation, make_half_params
    w2 = WORKLOADS[2]
    sh2 = OL.LayerShape(batch=1, seq=w2.seq, hidden=w2.hidden, heads=w2.heads, ffn=w2.ffn, tp=1)
    pa2 = {k: v.astype(np.float64) for k, v in make_half_params(w2, "attn", 0).items()}
    pm2 = {k: v.astype(np.float64) for k, v in make_half_params(w2, "mlp", 0).items()}
    x2 = make_activation(w2, 1).astype(np.float64)
    g2 = make_activation(w2, 2).astype(np.float64)
    t2 = time.perf_counter()
    a_part, a_sv = OL.attn_half_fwd(sh2, x2, pa2)
    x21 = OL.reduce_partials([a_part], x2, pa2["b_out"])
    m_part, m_sv = OL.mlp_half_fwd(sh2, x21, pm2)
    dx2m, _, _ = OL.mlp_half_bwd(sh2, g2, pm2, m_sv)
    OL.attn_half_bwd(sh2, OL.reduce_partials([dx2m], g2, None), pa2, a_sv)
    dt2 = time.perf_counter() - t2
    fl2 = 3.0 * shard_fwd_flops(w2.tokens, w2.hidden, w2.heads, w2.head_dim, w2.ffn, w2.seq, 1)
    del pa2, pm2, x2, g2, a_sv, m_sv, x21, a_part, m_part, dx2m
    log(f"cpu baseline GPT-style layer: {dt2:.1f}s, {fl2 / dt2 / 1e12:.3f} TFLOP/s")

    # the full layer (8 slices' worth, 128 heads) on its sampled rows: 32 seeded
    # positions of one sequence (always its first and last), the forward of the
    # unsliced layer; keys and values of every position up to the last one
    w5 = WORKLOADS[5]
    sh5 = OL.LayerShape(batch=1, seq=w5.seq, hidden=w5.hidden, heads=w5.heads, ffn=w5.ffn, tp=1)
    r5 = np.random.Generator(np.random.PCG64(5050))
    # 5e9 parameters: a 2^22-value N(0, 0.02) pool repeated to every weight's
    # shape, float32 (the oracle's time does not depend on the values; drawing
    # them all would take longer than the oracle itself)
    pool = r5.standard_normal(1 << 22, dtype=np.float32) * np.float32(0.02)
    full5 = {k: np.resize(pool, shp) for k, shp in OL.full_param_shapes(sh5).items()}
    for k in ("ln1_g", "ln2_g"):
        full5[k] += np.float32(1.0)
    x5 = r5.standard_normal((w5.seq, w5.hidden), dtype=np.float32).astype(np.float64)
    rows5 = sorted({0, w5.seq - 1, *r5.integers(1, w5.seq - 1, size=30).tolist()})
    t5 = time.perf_counter()
    OL.layer_fwd_rows(sh5, x5, full5, rows5)
    dt5 = time.perf_counter() - t5
    h5, s5 = w5.hidden, w5.seq
    nr = len(rows5)
    # K and V of all positions, then per sampled row: Q, scores and weighted sum
    # over its visible keys (causal), output projection, MLP
    fl5 = (2.0 * s5 * h5 * 2 * h5 + 2.0 * nr * h5 * h5 + sum(4.0 * h5 * (r + 1) for r in rows5)
           + 2.0 * nr * h5 * h5 + 4.0 * nr * h5 * w5.ffn)
    del full5, x5
    log(f"cpu baseline full layer, {nr} sampled rows of one sequence: {dt5:.1f}s")

    # the oracle's optimizer step on a 2^24-element chunk of the same workload, as
    # GB/s with the step's 34 bytes per parameter (accumulator, master, m, v read;
    # master, m, v and the bf16 copy written; the norm pass)
    from oracle import adam as OA
    rng = np.random.Generator(np.random.PCG64(4040))
    nc = 1 << 24
    p0 = rng.standard_normal(nc) * 0.02
    m0 = rng.standard_normal(nc) * 1e-3
    v0 = (rng.standard_normal(nc) * 1e-3) ** 2
    a0 = rng.standard_normal(nc) * 2e-3
    t1 = time.perf_counter()
    OA.adam_step(p0, m0, v0, a0, OA.AdamConfig(step=100))
    dta = time.perf_counter() - t1
    adam_gbs = 34.0 * nc / dta / 1e9
    log(f"cpu baseline adam: {dta:.2f}s for 2^24 parameters = {adam_gbs:.2f} GB/s")
    # the tiny layer (hidden 256, 4 heads of 64, MLP 1024, 2 sequences of 128,
    # its t = 2 slices in turn), fwd+bwd through the oracle on one BLAS thread
    # and on all of them (best of 5 passes each)
    from threadpoolctl import threadpool_limits
    tsh = OL.LayerShape(batch=2, seq=128, hidden=256, heads=4, ffn=1024, tp=2)
    trng = np.random.Generator(np.random.PCG64(1001))
    tfull = {k: (1.0 if k.endswith("_g") else 0.0) + trng.standard_normal(shp) * 0.02
             for k, shp in OL.full_param_shapes(tsh).items()}
    tx, tg = trng.standard_normal((256, 256)), trng.standard_normal((256, 256))

    def tiny_pass():
        out, state = OL.layer_fwd(tsh, tx, tfull)
        OL.layer_bwd(tsh, tg, tfull, state)

    def best_of(k=5):
        best = float("inf")
        for _ in range(k):
            t2 = time.perf_counter()
            tiny_pass()
            best = min(best, time.perf_counter() - t2)
        return best

    tiny_fl = 2 * 3.0 * shard_fwd_flops(256, 256, 2, 64, 512, 128, 2)
    with threadpool_limits(limits=1):
        t_one = best_of()
    t_all = best_of()
    log(f"cpu baseline tiny layer: {t_one * 1e3:.1f} ms on one thread, {t_all * 1e3:.1f} ms on {threads}")
    return {"value": round(fl / dt / 1e12, 4), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 oracle fwd+bwd of the same 1/8 slice on the first {sample_tokens} tokens "
                      f"of the workload, {reps} passes ({fl / 1e12:.3f} TFLOP), {dt:.1f} s",
            "seconds": round(dt, 2),
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "blas": [{k: i.get(k) for k in ("internal_api", "version", "num_threads")} for i in info],
            "adam": {"value": round(adam_gbs, 3), "unit": "GB/s", "sample": "float64 oracle Adam step over one "
                     "2^24-parameter chunk of the 1.887e9-parameter share (34 B/param accounting; the whole share "
                     "would take about 113 chunks)", "seconds": round(dta, 3)},
            "gpt_layer_h4096": {"value": round(fl2 / dt2 / 1e12, 4), "unit": "TFLOP/s", "seconds": round(dt2, 2),
                                "sample": "float64 oracle fwd+bwd of the GPT-style layer (hidden 4096, 32 heads of "
                                          "128, MLP 16384, 2048 tokens, one slice) in full", "flop": fl2},
            "full_layer_sampled_rows": {"value": round(fl5 / dt5 / 1e12, 4), "unit": "TFLOP/s",
                                        "seconds": round(dt5, 2), "flop": fl5,
                                        "sample": f"float64 oracle forward of the unsliced full layer (hidden "
                                                  f"20480, 128 heads, MLP 81920; float32 weights from a repeated "
                                                  f"random pool) on {nr} sampled positions of one 2048-token "
                                                  f"sequence (keys and values of every position)"},
            "tiny_layer": {"sample": "float64 oracle fwd+bwd of the tiny layer (hidden 256, 4 heads of 64, MLP 1024, "
                           "2 x 128 tokens, 2 slices in turn; best of 5)", "flop": tiny_fl,
                           "one_core_ms": round(t_one * 1e3, 3), "all_cores_ms": round(t_all * 1e3, 3),
                           "one_core_gflops": round(tiny_fl / t_one / 1e9, 3),
                           "all_cores_gflops": round(tiny_fl / t_all / 1e9, 3)}}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
