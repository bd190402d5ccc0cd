"""Build libmxcast.so (HIP kernels + C ABI) for gfx950, in-tree.

hipcc compiles the kernels and the host API (one object per source, in
parallel) and links them into one shared library next to this file.  Flags: -ffp-contract=off (the fused pre-ops are fixed sequences of
separately rounded fp32 operations), denormals preserved, no packed-fp32
instructions.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxcast.so")
SOURCES = ["api.cpp", "mx_cast.hip", "mx_cast_any.hip", "nvfp4.hip", "nvfp4_any.hip",
           *[f"mx_cast_{kind}_{fmt}.hip" for kind in ("fmt", "grp", "rag")
             for fmt in ("e4m3", "e5m2", "e4m3_up", "e5m2_up")]]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _filtered(stderr: str) -> str:
    # the host pass does not know the packed-fp32 feature and says so; not an error
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in stderr.splitlines() if noise not in l)


def build_library(verbose: bool = False, extra=(), jobs: int = 8) -> str:
    """Compile every source to an object (in parallel, at most `jobs` at a
    time), then link them into libmxcast.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs, pending, errors = [], [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC, *compile_flags, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        pending.append((src, cmd))
    running = []
    while pending or running:
        while pending and len(running) < jobs:
            src, cmd = pending.pop(0)
            running.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.PIPE, text=True)))
        src, p = running.pop(0)
        _, err = p.communicate()
        err = _filtered(err)
        if p.returncode != 0:
            errors.append(f"{src} ({p.returncode}):\n{err}")
        elif err.strip() and verbose:
            print(err, file=sys.stderr)
    if errors:
        raise RuntimeError("hipcc failed: " + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{_filtered(r.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
