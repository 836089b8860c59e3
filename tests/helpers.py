"""Test helpers: tolerances, error metrics and tensor conversion (no method arithmetic)."""
import numpy as np

# Tolerances on ||gpu - ref||_inf / ||ref||_inf per output tensor: 1e-4 for the fp32 path,
# 2e-2 for bf16 storage with fp32 accumulation.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_inf(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(got - ref)) / den if den > 0 else float(np.linalg.norm(got - ref))


def assert_close(name, got, ref, dtype):
    e = rel_inf(got, ref)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{name}: non-finite output"
    assert e <= TOL[dtype], f"{name}: rel_inf {e:.3e} > {TOL[dtype]} (rel_l2 {rel_l2(got, ref):.3e})"
    return e


def to_gpu(a, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def empty(shape, dtype: str):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")


def empty_bytes(n):
    import torch
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device="cuda")


def assert_bf16_copy(w_gpu, master_gpu, rw, rp):
    """The bf16 weight copy is the GPU's fp32 master rounded to nearest even, bit
    for bit; against the oracle's copy rw (of its fp64 master rp) it may differ by
    one bf16 ulp plus the GPU master's own deviation, which dominates where an
    update nearly cancels a weight (fp32 keeps the absolute error of the old
    value, far above the new value's bf16 ulp)."""
    from synth.inputs import round_f32_to_bf16
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    master_gpu = np.asarray(master_gpu, dtype=np.float64)
    assert np.array_equal(w_gpu, round_f32_to_bf16(master_gpu.astype(np.float32)).astype(np.float64))
    allow = np.abs(rw) * 2.0 ** -7 + 2.0 * np.abs(master_gpu - rp) + 1e-38
    assert np.all(np.abs(w_gpu - rw) <= allow)


def round_to_f16(a):
    """Nearest IEEE binary16 value of each element (ties to even), as float64:
    the storage of Q and K in the library's bf16 path (numpy's conversion)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)

