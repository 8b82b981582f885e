"""Build libgdn_cpr.so in-tree with hipcc for gfx950 (cross-compiles without a GPU).

Flags that the contract depends on:
  -ffp-contract=off                  no fusion other than the explicit fmaf
  -fno-gpu-flush-denormals-to-zero   binary32 denormals kept on the GPU
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                     no packed fp32 (v_pk_*) instructions in the kernels
No -ffast-math anywhere.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn_cpr.so")

SOURCES = ["cpr_kernels.hip", "cpr_backward.hip", "cpr2.hip", "linear.hip", "api.cpp",
           "contract.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    """Compile every source into bitwise_consistent_linear_amd/libgdn_cpr.so; return its path.
    Sources compile to objects side by side (one hipcc per source), then link."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *compile_flags, "-c", "-I", INCLUDE, "-I", CSRC, "-o", obj,
               os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(compile_one, SOURCES))
    for (obj, res), src in zip(results, SOURCES):
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed to compile {src}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[obj for obj, _ in results]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to link libgdn_cpr.so")
    os.replace(tmp, LIB)
    return LIB


PROBE_LIB = os.path.join(PKG, "libgdn_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile the measurement probes (csrc/probe.hip) into libgdn_probe.so, which bench.py
    uses for the vector-issue ceiling and shader clock; the library proper does not link it."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, os.path.join(CSRC, "probe.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libgdn_probe.so")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


KERNEL_SOURCES = [s for s in SOURCES if s.endswith(".hip")]


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of every kernel source, concatenated (for instruction-mix
    checks)."""
    parts = []
    for src in KERNEL_SOURCES:
        one = out_path + "." + src + ".s"
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
               "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "--cuda-device-only", "-S", "-I", INCLUDE, "-I", CSRC, "-o", one,
               os.path.join(CSRC, src)]
        subprocess.run(cmd, check=True, capture_output=True)
        with open(one) as f:
            parts.append(f.read())
        os.remove(one)
    with open(out_path, "w") as f:
        f.write("\n".join(parts))
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
