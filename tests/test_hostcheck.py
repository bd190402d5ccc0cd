"""Host code under AddressSanitizer, LeakSanitizer and UBSan (no GPU).

Two programs are built with gcc / g++ and run:

* tests/hostcheck/oracle_check.c links the oracle's C source and runs every
  tensor-level routine on small tensors (partial blocks, empty groups, every
  output set, format, scale rule, layout, pre-op and activation) with every
  buffer exactly as large as its layout says;
* tests/hostcheck/abi_check.cpp links the library's entry points
  (csrc/api.cpp) with recording stand-ins for the kernel launchers and drives
  every entry point through its error paths and through valid calls at the
  size limits, checking the status, that rejected calls launch nothing, and
  that accepted calls get a launch plan the kernels can run.

Either program stops at the first sanitizer finding with a non-zero status.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CHECK = os.path.join(HERE, "hostcheck")
CSRC = os.path.join(ROOT, "block_scaled_precision_bf16_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr, (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    build(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
           os.path.join(ROOT, "oracle", "mx_oracle.c"), os.path.join(CHECK, "oracle_check.c"),
           "-lm", "-o", exe])
    out = run(exe)
    assert ", 0 failed" in out


def test_entry_points_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_check")
    build(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", CHECK,
           os.path.join(CSRC, "api.cpp"), os.path.join(CHECK, "launch_record.cpp"),
           os.path.join(CHECK, "abi_check.cpp"), "-o", exe])
    out = run(exe)
    assert ", 0 failed" in out


@pytest.mark.parametrize("bug", ["heap", "overflow"])
def test_sanitizers_are_live(tmp_path, bug):
    """The same flags catch a one-element heap overrun and a signed overflow."""
    src = tmp_path / "bug.c"
    src.write_text(
        "#include <stdlib.h>\n#include <stdint.h>\n"
        "int main(int argc, char **argv) {\n"
        "  (void)argv; volatile int *p = malloc(4 * sizeof(int));\n"
        + ("  p[argc + 3] = 1;\n" if bug == "heap" else
           "  volatile int64_t v = INT64_MAX - 1 + argc; v = v * 2;\n")
        + "  free((void *)p); return 0;\n}\n")
    exe = str(tmp_path / "bug")
    build(["gcc", "-std=c11", *SAN, str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=60)
    assert r.returncode != 0
    # UBSan's object-size check or ASan reports the overrun, whichever sees it first
    want = ("heap-buffer-overflow", "insufficient space") if bug == "heap" else ("signed integer overflow",)
    assert any(w in r.stderr for w in want), r.stderr[-2000:]
