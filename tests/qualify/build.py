"""Build tests/qualify/libqualify.so: the test-only kernels that run the cast
library's per-element device routines over whole input domains.  Same
compiler and flags as the library itself (block_scaled_precision_bf16_amd/
build.py), so the routines compile to the code the library runs."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libqualify.so")


def build_qualify(verbose: bool = False) -> str:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from block_scaled_precision_bf16_amd.build import FLAGS, HIPCC, _filtered

    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, os.path.join(HERE, "qualify.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{_filtered(r.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_qualify(verbose=True))
