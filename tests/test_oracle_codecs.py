"""Pins for the oracle's element and scale codecs (CPU only).

Each codec is checked against something other than the oracle itself: torch's
own bf16 / float8_e4m3fn conversions (library special cases), brute-force
nearest-value search over the format's value set, and log2.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O

E2M1_PUBLISHED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the E2M1 value set


def bf16_all():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def torch_bf16_values(bits):
    t = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16)
    return t.double().numpy()


def test_bf16_decode_all_patterns():
    bits = bf16_all()
    want = torch_bf16_values(bits)
    got = np.array([O.bf16_value(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(11)
    # every finite bf16 value, the exact midpoint above it, and its fp32 neighbours
    fin = bf16_all()
    fin = fin[(fin & 0x7F80) != 0x7F80].astype(np.uint32) << 16
    mids = fin + 0x8000
    cand = np.concatenate([fin, mids, mids + 1, mids - 1, fin + 1,
                           rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)])
    f32 = cand.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_round_array(f32.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([O.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(want)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9


def brute_nearest(a, mags):
    """Nearest of the sorted magnitude list to each a >= 0; ties to the even index."""
    mags = np.asarray(mags)
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    hit = d == best
    idx = np.argmax(hit, axis=1)                      # lowest index at min distance
    two = hit.sum(axis=1) == 2
    idx = np.where(two & (idx % 2 == 1), idx + 1, idx)
    return idx


def test_e4m3_encode_brute_force_nearest():
    rng = np.random.default_rng(12)
    mags = np.array([O.e4m3_value(c) for c in range(127)])
    mids = (mags[:-1] + mags[1:]) / 2
    a = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 600, 300_000), 2.0 ** rng.uniform(-14, 9.5, 300_000),
                        [448, 449, 463.9, 464, 465, 480, 1e6, 2.0 ** -10, 2.0 ** -11]])
    for sign in (1.0, -1.0):
        v = sign * a
        got = O.e4m3_encode_array(v)
        want = brute_nearest(a, mags).astype(np.uint8)
        if sign < 0:
            want = want | 0x80
        assert np.array_equal(got, want)


def test_e4m3_encode_exhaustive_reachable_pairs_vs_torch():
    """Every (bf16 element, scale byte) pair a block can produce: the element is
    at most the block amax, so |x| < 2^(byte-127+9).  Torch's CPU float8_e4m3fn
    conversion is round-to-nearest-even; clamping first makes it saturating."""
    bits = bf16_all()
    bits = bits[(bits & 0x7F80) != 0x7F80]
    xv = torch_bf16_values(bits)
    ebits = (bits.astype(np.int64) >> 7) & 0xFF
    total = 0
    for b in range(0, 255):
        sel = ebits <= b + 8
        v = xv[sel] * 2.0 ** (127 - b)
        got = O.e4m3_encode_array(v)
        t = torch.from_numpy(v.astype(np.float32)).clamp(-448.0, 448.0)
        want = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (b, v[bad[:5]], got[bad[:5]], want[bad[:5]])
        total += v.size
    # 256 patterns per exponent field value, fields 0..min(b+8, 254)
    assert total == sum((min(b + 8, 254) + 1) * 256 for b in range(255))


def test_e4m3_encode_signed_zero_nan_saturation():
    assert O.e4m3_encode(0.0) == 0x00
    assert O.e4m3_encode(-0.0) == 0x80
    assert O.e4m3_encode(float("nan")) == 0x7F
    assert O.e4m3_encode(1e30) == 0x7E and O.e4m3_encode(-1e30) == 0xFE
    assert O.e4m3_encode(float("inf")) == 0x7E


def test_e2m1_value_set():
    assert [O.e2m1_value(c) for c in range(8)] == E2M1_PUBLISHED
    assert [O.e2m1_value(c | 8) for c in range(8)] == [-v for v in E2M1_PUBLISHED]


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(13)
    mags = np.array(E2M1_PUBLISHED)
    mids = (mags[:-1] + mags[1:]) / 2
    near = [np.nextafter(np.float32(m), np.float32(t)) for m in mids for t in (0, 10)]
    a = np.concatenate([mags, mids, np.array(near, np.float64),
                        rng.uniform(0, 8, 2_000_000),
                        np.abs(rng.integers(0, 2**32, 2_000_000, dtype=np.uint64)
                               .astype(np.uint32).view(np.float32).astype(np.float64))])
    a = a[np.isfinite(a)]
    big = a[a > 16.0]           # far above 6 the nearest finite value is 6
    a = a[a <= 16.0]
    want = brute_nearest(a, mags).astype(np.uint8)
    assert np.array_equal(O.e2m1_encode_array(a), want)
    assert np.array_equal(O.e2m1_encode_array(-a), want | 8)
    assert big.size > 100_000 and np.all(O.e2m1_encode_array(big) == 7)
    assert O.e2m1_encode(float("inf")) == 7 and O.e2m1_encode(-float("inf")) == 15
    assert O.e2m1_encode(float("nan")) == 0
    assert O.e2m1_encode(-0.0) == 8


@pytest.fixture(scope="module")
def e2m1_sweeper(tmp_path_factory):
    """The brute-force sweep of tests/pins/e2m1_sweep.c, compiled for this run."""
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pins", "e2m1_sweep.c")
    so = str(tmp_path_factory.mktemp("pins") / "e2m1_sweep.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", src, "-o", so, "-lm"], check=True)
    L = ctypes.CDLL(so)
    L.e2m1_sweep.restype = ctypes.c_int64
    L.e2m1_sweep.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64,
                             ctypes.POINTER(ctypes.c_int64)]
    return L


def test_e2m1_encode_every_fp32(e2m1_sweeper):
    """The oracle's E2M1 encoder on all 2^32 fp32 bit patterns (NaN aside,
    pinned above) equals the brute-force nearest of the eight magnitudes."""
    enc = ctypes.cast(O.lib().orc_e2m1_encode, ctypes.c_void_p)
    fb = ctypes.c_int64()
    step = 1 << 30
    for first in range(0, 1 << 32, step):
        bad = e2m1_sweeper.e2m1_sweep(enc, first, step, ctypes.byref(fb))
        assert bad == 0, (bad, hex(first + fb.value))


def test_e2m1_sweep_catches_a_wrong_encoder(e2m1_sweeper):
    """The sweep fails an encoder with one rounding decision moved: ties
    between 2 and 3 (code 4 | 5) going up instead of to the even code."""
    fn_t = ctypes.CFUNCTYPE(ctypes.c_uint8, ctypes.c_double)

    def wrong(v):
        c = O.e2m1_encode(v)
        return (c + 1) if abs(v) == 2.5 else c
    cb = fn_t(wrong)
    fb = ctypes.c_int64()
    first = 0x40200000                         # 2.5
    bad = e2m1_sweeper.e2m1_sweep(ctypes.cast(cb, ctypes.c_void_p), first - 4, 8, ctypes.byref(fb))
    assert bad == 1 and fb.value == 4


def test_e8m0_exhaustive_over_bf16_amax():
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint32).astype(np.uint16)
    a = torch_bf16_values(bits)
    got = np.array([O.e8m0_byte(float(v)) for v in a])
    with np.errstate(divide="ignore"):
        fl = np.floor(np.log2(a))
    want = np.clip(np.where(a == 0, -np.inf, fl - 8 + 127), 0, 254).astype(np.int64)
    assert np.array_equal(got, want)
    # for normal amax the byte is the exponent field minus 8, clamped at 0
    normal = (bits >> 7) > 0
    assert np.array_equal(got[normal], np.maximum((bits[normal] >> 7).astype(np.int64) - 8, 0))
    assert got.max() == 246
    assert O.e8m0_byte(float("inf")) == 0xFF and O.e8m0_byte(float("nan")) == 0xFF
    assert O.e8m0_value(127) == 1.0 and O.e8m0_value(0) == 2.0 ** -127
