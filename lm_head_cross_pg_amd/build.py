"""Build libpg_lmhead.so (the gfx950 HIP library) in place with hipcc.

    python -m lm_head_cross_pg_amd.build          # or: python lm_head_cross_pg_amd/build.py
    python -m lm_head_cross_pg_amd.build --incremental   # only sources changed since their objects

The library needs only the HIP runtime; no PyTorch headers are involved.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpg_lmhead.so")
SOURCES = ["pg_api.hip", "pg_fwd.hip", "pg_bwd.hip", "pg_gemm.hip", "pg_bpb.hip", "pg_quant.hip", "pg_window.hip"]
# Kernels that keep MFMA accumulators in VGPRs so that the hidden-row operands can live in AGPRs.
VGPR_ACC_SOURCES = {"pg_fwd.hip", "pg_bwd.hip"}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 instructions stay off: the compiler still vectorises with plain ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # check the generated machine code: a backend slip fails the build instead of running
        "-mllvm", "-verify-machineinstrs",
        "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
    ]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in (res.stderr or "").splitlines()
                    if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}\n{res.stdout}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _headers() -> list[str]:
    inc = os.path.join(ROOT, "include")
    return [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
           [os.path.join(inc, f) for f in os.listdir(inc) if f.endswith(".h")]


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source and link libpg_lmhead.so next to this file; returns its path.
    incremental: skip a source whose object is newer than it and than every header."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    newest_header = max(os.path.getmtime(h) for h in _headers())
    jobs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        path = os.path.join(CSRC, src)
        if incremental and os.path.exists(obj) and \
                os.path.getmtime(obj) > max(os.path.getmtime(path), newest_header):
            continue
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] if src in VGPR_ACC_SOURCES else []
        jobs.append(([hipcc(), *flags(), *extra, "-c", path, "-o", obj], obj))
    # one hipcc per source, in parallel: the translation units are independent
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for fut in [pool.submit(_run, cmd, verbose) for cmd, _ in jobs]:
            fut.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv[1:]))
