"""The GEMM-ready scale layout (MX_SCALE_TILED) fed to the instruction it is
laid out for: gfx950's block-scaled v_mfma_scale_f32_32x32x64_f8f6f4.

A test-only wave (tests/qualify/qualify.hip, mfma_consumer_kernel) loads the
cast's outputs exactly as a block-scaled GEMM would -- lane L (h = L / 32)
takes row L % 32, K values 16 h .. 16 h + 15 of each half of a 64-wide step
(the instruction's operand layout for 8-bit formats), and its scale word from
the tile layout, whose byte for the step the instruction's op_sel picks; that
byte scales K block h of the step (probed on gfx950: a lane's scale acts on
bytes 0-15 of lanes L and L ^ 32 for h = 0, on bytes 16-31 for h = 1) -- and
accumulates C = A * B over K / 64 steps:

  A [32][K]: q_row / s_row of the row-wise cast of X [32][K]
  B [K][32]: q_col / s_col of the column-wise cast of Z [K][32] (q_col is B
             transposed, blocks along K)

The inputs are n * 2^e with n in {-4 .. 4} and e drawn per 32-element block
in [-2, 2], each block holding one element of magnitude 4 * 2^e: every
element, product and partial sum is then exact in fp32, so C must equal the
float64 product of the oracle's dequantised operands bit for bit, whatever
order the hardware adds in.  The block exponents vary, so a scale taken from
the wrong block, step or lane would change C (checked on the CPU below).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_same, to_dev

pytestmark = pytest.mark.gpu

QLIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "qualify", "libqualify.so")


@pytest.fixture(scope="module")
def Q():
    L = ctypes.CDLL(QLIB)
    L.qual_mfma_consumer.restype = ctypes.c_int
    L.qual_mfma_consumer.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_int,
                                                             ctypes.c_void_p, ctypes.c_void_p]
    return L


def blocked_values(rows, cols, seed, along_cols=True):
    """n * 2^e, n in {-4..4}, e per 32-block (along cols, or along rows) in
    [-2, 2], one element of each block at +-4 * 2^e."""
    rng = np.random.default_rng(seed)
    n = rng.integers(-4, 5, size=(rows, cols)).astype(np.float64)
    if along_cols:
        e = np.repeat(rng.integers(-2, 3, size=(rows, cols // 32)), 32, axis=1)
        n[:, ::32] = np.where(rng.random((rows, cols // 32)) < 0.5, -4.0, 4.0)
    else:
        e = np.repeat(rng.integers(-2, 3, size=(rows // 32, cols)), 32, axis=0)
        n[::32, :] = np.where(rng.random((rows // 32, cols)) < 0.5, -4.0, 4.0)
    return W.bf16_bits((n * 2.0 ** e).astype(np.float32))


def dequant(q, s, fmt):
    """Elements q[R][C] times their compact scales s[R][C/32]."""
    dec = np.array([O.e5m2_value(c) if fmt else O.e4m3_value(c) for c in range(256)])
    sc = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    return dec[q] * sc


def run_consumer(Q, qa, sa, qb, sb, K, fmt):
    C = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    st = Q.qual_mfma_consumer(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(), K, fmt,
                              C.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    return C.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
def test_tiled_scales_feed_the_block_scaled_mfma(Q, fmt):
    K = 1024                                         # 16 steps: every op_sel byte, 4 tiles
    flags = mx.SCALE_TILED | (mx.ELEM_E5M2 if fmt else 0)
    x = blocked_values(32, K, seed=301)              # A, blocks along K
    z = blocked_values(K, 32, seed=302, along_cols=False)   # B, blocks along K
    ga = mx.mx_quantize(to_dev(x), axis=mx.ROWWISE | flags)
    gb = mx.mx_quantize(to_dev(z), axis=mx.COLWISE | flags)
    torch.cuda.synchronize()

    oa = O.mx_quantize(x, axis=mx.ROWWISE | (mx.ELEM_E5M2 if fmt else 0))
    ob = O.mx_quantize(z, axis=mx.COLWISE | (mx.ELEM_E5M2 if fmt else 0))
    assert_same(ga["q_row"], oa["q_row"], "A elements")
    assert_same(gb["q_col"], ob["q_col"], "B elements")
    A = dequant(oa["q_row"], oa["s_row"], fmt)       # [32][K]
    Bt = dequant(ob["q_col"], ob["s_col"], fmt)      # [32][K] = B transposed
    assert np.array_equal(A, W.bf16_to_f32(x).astype(np.float64))   # exact inputs
    want = A @ Bt.T

    # with every scale byte 127 (2^0) the product is that of the bare element
    # values: the operand layout alone
    unit = torch.full((K,), 127, dtype=torch.uint8, device="cuda")
    got_unit = run_consumer(Q, ga["q_row"], unit, gb["q_col"], unit, K, fmt)
    ones = np.full_like(oa["s_row"], 127)
    want_unit = dequant(oa["q_row"], ones, fmt) @ dequant(ob["q_col"], np.full_like(ob["s_col"], 127), fmt).T
    assert np.array_equal(got_unit, want_unit), np.argwhere(got_unit != want_unit)[:4]

    got = run_consumer(Q, ga["q_row"], ga["s_row"], gb["q_col"], gb["s_col"], K, fmt)
    assert np.array_equal(got, want), (np.argwhere(got != want)[:4], got[got != want][:4],
                                       want[got != want][:4])


def test_wrong_scale_mapping_would_show():
    """With the block exponents of these inputs, taking either operand's
    scales from the other half of a step, or from the neighbouring step,
    changes the product: the GPU comparison above is sensitive to the
    layout."""
    K = 1024
    x = blocked_values(32, K, seed=301)
    z = blocked_values(K, 32, seed=302, along_cols=False)
    oa, ob = O.mx_quantize(x, axis=mx.ROWWISE), O.mx_quantize(z, axis=mx.COLWISE)
    want = dequant(oa["q_row"], oa["s_row"], 0) @ dequant(ob["q_col"], ob["s_col"], 0).T
    s = oa["s_row"]
    halves = s.reshape(32, -1, 2)[:, :, ::-1].reshape(32, -1)          # swap the 2 blocks of a step
    steps = s.reshape(32, -1, 4)[:, :, [2, 3, 0, 1]].reshape(32, -1)   # swap neighbouring steps
    for bad in (halves, steps):
        got = dequant(oa["q_row"], bad, 0) @ dequant(ob["q_col"], ob["s_col"], 0).T
        assert not np.array_equal(got, want)
