"""Device qualification of the per-element routines the cast kernels build on
(csrc/device_math.h), over their whole input domains, against the oracle.

The kernels round with gfx950 conversion instructions where those are
bit-identical to the rules the oracle implements; these tests are the
evidence.  A test-only library (tests/qualify/libqualify.so) runs each routine
on every fp32 bit pattern of its domain, in both operand positions of the
packed instructions and every byte / half position the kernels use; the
oracle's C checkers compare every result:

  bf16x2_rne   v_cvt_pk_bf16_f32           all 2^32 fp32: nearest bf16, ties
                                           to even, NaN stays NaN
  e4m3x2       +-448 clamp, v_cvt_pk_fp8_f32  all non-NaN fp32: saturating
                                           nearest E4M3
  e2m1x2       v_cvt_scalef32_pk_fp4_f32, scale 1  all non-NaN fp32: nearest
                                           E2M1, saturating at 6
  exp32_nonpos the library's exp           all 2^31 non-positive fp32 (and
                                           NaN): the oracle's exp bit for bit
  rcp_1_2      rcp + one Newton step       every float in [1, 2]: the
                                           correctly rounded 1/d
  div6_bf16    b / 6 by multiply + FMA     every finite non-negative bf16:
                                           the correctly rounded b / 6
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
QLIB = os.path.join(HERE, "qualify", "libqualify.so")
CHUNK = 1 << 28          # inputs per launch
FULL = 1 << 32


@pytest.fixture(scope="module")
def Q():
    if not os.path.exists(QLIB):
        pytest.fail(f"{QLIB} is not built (__graft_entry__.build() builds it)")
    L = ctypes.CDLL(QLIB)
    for name in ("qual_bf16_rne", "qual_e2m1", "qual_e4m3"):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                      ctypes.c_void_p]
    L.qual_exp.restype = ctypes.c_int
    L.qual_exp.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    for name in ("qual_rcp_1_2", "qual_div6"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    O.set_threads(min(16, len(os.sched_getaffinity(0))))
    return L


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def sweep(Q, name, which, out_dtype, per_input, start, stop, swaps=(0, 1)):
    """Run routine `name` on the patterns [start, stop) in chunks and check
    every result with the oracle's rule `which`."""
    out = torch.empty(int(CHUNK * per_input), dtype=out_dtype, device="cuda")
    for swap in swaps:
        for first in range(start, stop, CHUNK):
            n = min(CHUNK, stop - first)
            o = out[:int(n * per_input)]
            args = (first, n, swap, ctypes.c_void_p(o.data_ptr()), stream()) if swap is not None \
                else (first, n, ctypes.c_void_p(o.data_ptr()), stream())
            assert getattr(Q, name)(*args) == 0
            host = o.cpu().numpy()
            bad, fb = O.check_range(which, host, first)
            assert bad == 0, (f"{name} swap={swap}: {bad} inputs differ from the oracle; first "
                              f"at pattern {first + fb:#010x}")


def test_bf16_pack_rounding(Q):
    sweep(Q, "qual_bf16_rne", "bf16_round", torch.int16, 1, 0, FULL)


def test_e4m3_clamped_convert(Q):
    sweep(Q, "qual_e4m3", "e4m3", torch.uint8, 1, 0, FULL)


def test_e2m1_convert(Q):
    sweep(Q, "qual_e2m1", "e2m1", torch.uint8, 0.5, 0, FULL)


def test_exp_nonpositive(Q):
    # +0 and every pattern with the sign bit set: -0, negative subnormals and
    # normals, -Inf, and the NaNs
    sweep(Q, "qual_exp", "exp32", torch.int32, 1, 0, 2, swaps=(None,))
    sweep(Q, "qual_exp", "exp32", torch.int32, 1, 1 << 31, FULL, swaps=(None,))


def test_reciprocal_on_one_to_two(Q):
    n = (1 << 23) + 1
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    assert Q.qual_rcp_1_2(ctypes.c_void_p(out.data_ptr()), stream()) == 0
    got = out.cpu().numpy().view(np.uint32)
    d = (np.arange(n, dtype=np.uint32) + np.uint32(0x3F800000)).view(np.float32)
    want = (np.float32(1.0) / d).view(np.uint32)          # IEEE fp32 division
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (bad.size, [hex(0x3F800000 + int(i)) for i in bad[:4]])


def test_div6_on_every_bf16(Q):
    out = torch.empty(0x7F80, dtype=torch.int32, device="cuda")
    assert Q.qual_div6(ctypes.c_void_p(out.data_ptr()), stream()) == 0
    got = out.cpu().numpy().view(np.uint32)
    b = (np.arange(0x7F80, dtype=np.uint32) << 16).view(np.float32)
    want = (b / np.float32(6.0)).view(np.uint32)          # IEEE fp32 division
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (bad.size, [hex(int(i)) for i in bad[:4]])
