"""Build libmtnlg.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python -m tensor_sliced_transformer_amd.build [--jobs N]

Every call recompiles all sources (the build check must compile each time);
objects go to tensor_sliced_transformer_amd/_build/, the shared library next to
this file. Device code is built for gfx950 only, with packed-fp32 instruction
selection turned off (see EXTRA for per-file flags).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmtnlg.so")

SOURCES = ["api.cpp", "stage.cpp", "gemm.hip", "layernorm.hip", "attention.hip", "attention_bf16.hip",
           "attention_bf16_dkdv.hip", "stream.hip"]
# Per-source extra flags. The forward and dQ attention kernels keep their MFMA
# accumulators in VGPRs, so that the softmax arithmetic on them needs no copies
# between register files.
EXTRA = {"attention_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str) -> tuple[str, str]:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *lang, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out, r.stderr


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                sys.stderr.write(err)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-sanitizer build: the host-side sources (argument validation, layouts and
# launch sequences) with AddressSanitizer and UndefinedBehaviorSanitizer on the
# host pass only, linked with the ordinary device objects. The host ABI tests
# run against it on the CPU (no kernel is launched there).
HOST_SOURCES = ["api.cpp", "stage.cpp"]
SAN_LIB = os.path.join(HERE, "libmtnlg_hostsan.so")
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=undefined").split()


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload into python)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's AddressSanitizer runtime was not found")
    return path


def build_host_sanitized() -> str:
    """libmtnlg_hostsan.so: needs the device objects of build() in _build/."""
    objs = []
    for src in HOST_SOURCES:
        out = os.path.join(BUILD, os.path.splitext(src)[0] + ".hostsan.o")
        cmd = [hipcc(), "-x", "hip", *COMMON, "-O1", "-g", *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(out)
    dev = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s not in HOST_SOURCES]
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *SAN_FLAGS[:4], "-Xarch_host", "-shared-libsan",
           *objs, *dev, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--host-sanitized", action="store_true", help="also build libmtnlg_hostsan.so")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
    if a.host_sanitized:
        print(build_host_sanitized())


if __name__ == "__main__":
    main()
