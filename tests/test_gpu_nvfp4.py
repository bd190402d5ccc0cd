"""GPU parity of NVFP4 quantize-transpose and the tensor absmax: packed E2M1
bytes, E4M3 block scales and the fp32 global scale bit-exact against the
oracle, on shapes with ragged tiles (M a multiple of 16 but not 32 included),
the hand-worked blocks, and degenerate tensors (all zero, tiny magnitudes
that drive block scales subnormal or to zero)."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_same, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu


def run_both(x, axis=3, tensor_amax=None, two_d=False):
    xd = to_dev(x)
    if tensor_amax is None:
        amax = mx.mx_absmax_bf16(xd)
    else:
        amax = torch.tensor([tensor_amax], dtype=torch.float32, device="cuda")
    g = mx.nvfp4_quantize_transpose(xd, amax, axis=axis, two_d=two_d)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose(x, axis=axis, tensor_amax=tensor_amax, two_d=two_d)
    assert g["sg"].item() == o["sg"]
    return g, o


@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", [(16, 16), (48, 80), (128, 256), (144, 528), (400, 784)])
def test_random_shapes(M, K, axis):
    x = W.student_t_rows(M, K, seed=2000 + M + K)
    g, o = run_both(x, axis)
    mx_outputs_equal(g, o, f"nvfp4 {M}x{K} axis {axis}")


def test_absmax_matches_oracle():
    for shape, seed in (((64, 64), 1), ((1000, 24), 2), ((3, 5), 3), ((16384, 160), 4)):
        x = W.student_t_rows(*shape, seed=seed)
        a = mx.mx_absmax_bf16(to_dev(x))
        torch.cuda.synchronize()
        assert a.item() == O.absmax(x)


def test_golden_blocks():
    here = os.path.dirname(__file__)
    x = np.zeros((16, 16), np.uint16)
    for i, line in enumerate(l for l in open(os.path.join(here, "golden", "nvfp4_blocks.txt"))
                             if l.strip() and not l.startswith("#")):
        vals = [int(h, 16) for h in line.split("|")[1].split(",")]
        x[i, :len(vals)] = vals
    g, o = run_both(x, tensor_amax=2688.0)
    mx_outputs_equal(g, o, "golden")


@pytest.mark.parametrize("sigma", [0.0, 1e-20, 1e-36, 1e30])
def test_degenerate_magnitudes(sigma):
    x = W.normal(64, 96, seed=43, sigma=sigma if sigma else 1.0)
    if sigma == 0.0:
        x[:] = 0
        x[5, 5] = 0x8000
    g, o = run_both(x)
    mx_outputs_equal(g, o, f"nvfp4 sigma {sigma}")


def test_tiny_global_scale_overflowing_inverse():
    """A tensor amax below 2^-120 makes S_g so small that some block
    multipliers overflow to Inf (x*Inf saturates, 0*Inf encodes as +0)."""
    x = W.normal(32, 64, seed=44, sigma=1e-37)
    x[0, :16] = 0
    x[1, 0] = 0x8000
    g, o = run_both(x)
    mx_outputs_equal(g, o, "tiny S_g")


def test_every_row_scale_code():
    """Block magnitudes swept over 19 octaves below the tensor amax, so that
    every E4M3 block-scale code 0..126 occurs among the row blocks (checked on
    the oracle's output) and the scale chain is exercised at each of them."""
    rng = np.random.default_rng(45)
    M, K = 64, 2048
    t = np.linspace(0, 1, M * (K // 16)).reshape(M, K // 16)
    x = rng.standard_normal((M, K)).astype(np.float32) * np.repeat(2.0 ** (-19 * t), 16, axis=1)
    g, o = run_both(W.bf16_bits(x.astype(np.float32)))
    assert set(np.unique(o["s_row"]).tolist()) == set(range(127))
    mx_outputs_equal(g, o, "nvfp4 scale sweep")


# --- 2D (16 x 16 block) scaling ------------------------------------------------

@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", [(16, 16), (48, 80), (128, 256), (144, 528), (400, 784)])
def test_2d_random_shapes(M, K, axis):
    x = W.student_t_rows(M, K, seed=2100 + M + K)
    g, o = run_both(x, axis, two_d=True)
    mx_outputs_equal(g, o, f"nvfp4 2d {M}x{K} axis {axis}")


def test_2d_every_scale_code_and_tiny_global_scale():
    rng = np.random.default_rng(46)
    M, K = 256, 2048
    t = np.linspace(0, 1, (M // 16) * (K // 16)).reshape(M // 16, K // 16)
    scale = np.repeat(np.repeat(2.0 ** (-19 * t), 16, axis=0), 16, axis=1)
    x = W.bf16_bits((rng.standard_normal((M, K)) * scale).astype(np.float32))
    g, o = run_both(x, two_d=True)
    assert set(np.unique(o["s_row"]).tolist()) == set(range(127))
    mx_outputs_equal(g, o, "nvfp4 2d scale sweep")
    x = W.normal(32, 64, seed=47, sigma=1e-37)
    x[0:16, 0:16] = 0
    x[1, 20] = 0x8000
    g, o = run_both(x, two_d=True)
    mx_outputs_equal(g, o, "nvfp4 2d tiny S_g")


def _nan_or_inf_equal(a, b):
    return (np.isnan(a) and np.isnan(b)) or a == b


@pytest.mark.parametrize("bits", [0x7FC0, 0xFFC1, 0x7F80, 0xFF80])
@pytest.mark.parametrize("two_d", [False, True])
@pytest.mark.parametrize("M,K", [(48, 80), (144, 528), (1040, 272)])
def test_nonfinite_tensor(bits, two_d, M, K):
    """A tensor holding a NaN or an Inf: the device absmax is NaN / Inf, and
    the cast writes 0x7F scale bytes and zero codes over every (ragged) tile,
    as the oracle does; S_g stays NaN / Inf."""
    x = W.student_t_rows(M, K, seed=2100 + M)
    x[M // 2 + 1, K - 3] = bits
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16(xd)
    torch.cuda.synchronize()
    A = amax.item()
    assert _nan_or_inf_equal(A, O.absmax(x)) and not np.isfinite(A)
    g = mx.nvfp4_quantize_transpose(xd, amax, two_d=two_d)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose(x, two_d=two_d)
    assert _nan_or_inf_equal(g["sg"].item(), o["sg"])
    mx_outputs_equal(g, o, f"nvfp4 non-finite {bits:#06x} {M}x{K} 2d={two_d}")


@pytest.mark.parametrize("two_d", [False, True])
def test_nonfinite_group(two_d):
    """One group of a grouped cast holds a NaN: that group's outputs are the
    non-finite fill, the others are cast as usual."""
    rows = [144, 16, 0, 400, 32]
    x = W.student_t_rows(sum(rows), 272, seed=2200)
    x[144 + 3, 100] = 0x7FC0
    x[160 + 399, 0] = 0xFF80            # an Inf in the fourth group
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16_grouped(xd, rows)
    g = mx.nvfp4_quantize_transpose_grouped(xd, rows, amax, two_d=two_d)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose_grouped(x, rows, two_d=two_d)
    got_sg = g["sg"].cpu().numpy()
    assert np.isnan(got_sg[1]) and np.isinf(got_sg[3]) and got_sg[2] == 1.0
    assert all(_nan_or_inf_equal(a, b) for a, b in zip(got_sg, o["sg"]))
    mx_outputs_equal(g, o, f"grouped nvfp4 non-finite 2d={two_d}")
