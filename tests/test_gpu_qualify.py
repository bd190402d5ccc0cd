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
  div_by       q / s from a prepared       every divisor mantissa at six
               reciprocal and two FMA      exponents (every subnormal divisor,
               residual steps              both sides of the 2^-90 switch, the
                                           largest tensor scales), with every
                                           dividend b / 6 of the NVFP4 scale
                                           chain: the IEEE quotient wherever
                                           it is at least 2^-10, and the same
                                           E4M3 scale code everywhere
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
    L.qual_divby.restype = ctypes.c_int
    L.qual_divby.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.qual_divby_values.restype = ctypes.c_int
    L.qual_divby_values.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] + [ctypes.c_void_p] * 2
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


# divisor exponent ranges: every subnormal divisor (the rescaled path), the
# binade above the smallest normal, the two binades around the 2^-90 switch,
# [1, 2), and the binade of the largest tensor scales (bf16 max / 2688 <
# 2^117); 2^23 divisors each
DIVISORS = [(1, (1 << 23) - 1), (1 << 23, 1 << 23), (36 << 23, 1 << 23), (37 << 23, 1 << 23),
            (127 << 23, 1 << 23), (243 << 23, 1 << 23)]


@pytest.mark.parametrize("first,n", DIVISORS, ids=[f"{f:#010x}" for f, _ in DIVISORS])
def test_division_by_tensor_scale(Q, first, n):
    counts = torch.zeros(3, dtype=torch.int64, device="cuda")
    for c0 in range(first, first + n, 1 << 21):       # launches of 2^21 divisors
        cn = min(1 << 21, first + n - c0)
        assert Q.qual_divby(c0, cn, ctypes.c_void_p(counts.data_ptr()), stream()) == 0
    bad_q, bad_code, tested = (int(v) for v in counts.cpu())
    assert tested > 1000 * n
    assert bad_q == 0 and bad_code == 0, (bad_q, bad_code, tested)


def test_division_by_tensor_scale_against_host():
    """The same routine on random (divisor, bf16 dividend) pairs across the
    whole range, compared with numpy's IEEE float32 division on the host."""
    L = ctypes.CDLL(QLIB)
    L.qual_divby_values.restype = ctypes.c_int
    L.qual_divby_values.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] + [ctypes.c_void_p] * 2
    rng = np.random.default_rng(41)
    n = 1 << 22
    s = rng.integers(1, 0x7B000000, size=n, dtype=np.uint32).view(np.float32)   # up to ~2^119
    b = (rng.integers(0, 0x7F80, size=n, dtype=np.uint32) << 16).view(np.float32)
    q = (b / np.float32(6.0)).astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        want = (q / s).astype(np.float32)
    sd, qd = torch.from_numpy(s).cuda(), torch.from_numpy(q).cuda()
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    assert L.qual_divby_values(ctypes.c_void_p(sd.data_ptr()), ctypes.c_void_p(qd.data_ptr()), n,
                               ctypes.c_void_p(out.data_ptr()), stream()) == 0
    got = out.cpu().numpy()
    # the chain's quotients: at least 2^-10 (else the scale code is 0) and at
    # most a few thousand (the block amax never exceeds the tensor amax)
    dom = (np.abs(want) >= np.float32(2.0 ** -10)) & (np.abs(want) <= np.float32(2.0 ** 20))
    assert dom.sum() > n // 16
    differ = (got.view(np.uint32) != want.view(np.uint32)) & dom
    assert not differ.any(), (s[differ][:4], q[differ][:4], got[differ][:4], want[differ][:4])
