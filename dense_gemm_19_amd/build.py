"""Build libdg.so for gfx950 with hipcc (every source, every call).

    python -m dense_gemm_19_amd.build [-v] [--incremental]

Objects go to dense_gemm_19_amd/_build/; the library to dense_gemm_19_amd/libdg.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: no packed FP32 instructions are emitted anywhere.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
# Per-source extra flags.  The FP8 kernels promote each matrix-core block sum on
# the vector ALUs; the VGPR form of the MFMA instructions lets those sums land
# where the ALUs can use them (no copies out of accumulation registers).
EXTRA_FLAGS = {"gemm_dtl_f8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "gemm_dtl_f8s.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]

HIP_SOURCES = ["gemm_mfma.hip", "gemm_dtl_f16.hip", "gemm_dtl_bf16.hip", "gemm_dtl_f8.hip", "gemm_dtl_f8s.hip", "skinny.hip",
               "epilogue.hip", "calib.hip", "quant.hip", "noalloc.hip"]
HOST_SOURCES = ["view.cpp", "plan.cpp", "dg.cpp", "gemm_dtl.cpp"]


def _newest_header() -> float:
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    hs += [os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include"))]
    return max(os.path.getmtime(h) for h in hs)


def _compile(src: str, verbose: bool, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        t = os.path.getmtime(obj)
        if t > os.path.getmtime(os.path.join(CSRC, src)) and t > _newest_header():
            return obj
    hip = src.endswith(".hip")
    flags = HIP_FLAGS + ["-Rpass-analysis=kernel-resource-usage"] if hip else HOST_FLAGS
    cmd = [HIPCC] + flags + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = r.stderr.splitlines()
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    err = "\n".join(l for l in lines if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{err}")
    if hip:
        spills = _scratch_kernels(lines)
        if spills:
            os.remove(obj)
            raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {spills}")
    if err.strip() and verbose:
        print(err)
    return obj


def _scratch_kernels(remarks) -> list:
    """Kernels whose resource-usage remark reports scratch (spilled registers)."""
    out, name = [], None
    for l in remarks:
        if "remark: Function Name:" in l:
            name = l.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in l and name:
            n = int(l.split("ScratchSize [bytes/lane]:")[1].split("[")[0].strip())
            if n > 0:
                out.append(f"{name} ({n} bytes/lane)")
    return out


def build(verbose: bool = False, jobs: int | None = None, incremental: bool = False) -> str:
    """Compile every source (or, with incremental=True, those newer than their
    object) and link libdg.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + HOST_SOURCES
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
