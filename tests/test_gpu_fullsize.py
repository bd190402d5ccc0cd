"""The five workloads at full size, in the launch configuration the benchmark
times, compared with the oracle on every output element (the oracle runs
these sizes in seconds with OpenMP over rows / columns).

  16384^2 log-uniform rows: dim1 only, and dim0 + dim1 in one pass
  8192^2 N(0, 2): GELU + dbias, and dGELU(x) * grad + dbias
  8192 x 8192 [gate | linear]: SwiGLU and GeGLU, both directions
  16384^2 Student-t with 1% of rows x100: NVFP4 quantize-transpose
and the backward casts at the same sizes as their forward ones:
  8192^2 N(0, 2) with grad N(0, 1): dSiLU(x) * grad + dbias
  grad 8192 x 4096 with [gate | linear] 8192 x 8192: dSwiGLU and dGeGLU
and the grouped workloads: eight experts' rows (1104, 3008, 1072, 6560, 1632,
608, 2256, 144) of 16384 x 7168 N(0, 1) tokens cast as MXFP8 and as NVFP4,
and of a 16384 x 4096 [gate | linear] input through grouped SwiGLU.
"""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def loguniform16k():
    return W.make("c2_dim1_16384")


def test_c2_dim1_16384(loguniform16k):
    x = loguniform16k
    g = mx.mx_quantize(to_dev(x), axis=mx.COLWISE)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, axis=mx.COLWISE)
    mx_outputs_equal(g, o, "C2 dim1")


def test_metric_dim0_dim1_16384(loguniform16k):
    x = loguniform16k
    g = mx.mx_quantize(to_dev(x), axis=mx.ROWWISE | mx.COLWISE)
    torch.cuda.synchronize()
    o = O.mx_quantize(x)
    mx_outputs_equal(g, o, "dim0+dim1 16384")


@pytest.mark.parametrize("pre", [mx.FUSE_GELU, mx.FUSE_DGELU])
def test_c3_fused_dbias_8192(pre):
    x, grad = W.make("c3_gelu_dbias_8192")
    f = pre | mx.FUSE_DBIAS
    g = mx.mx_quantize(to_dev(x), to_dev(grad), fusion=f)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, fusion=f, want_y=True)
    mx_outputs_equal(g, o, f"C3 pre-op {pre}")
    ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
    assert_dbias_close(g["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_c4_gated_8192(act):
    x = W.make("c4_gated_8192")
    g = mx.mx_quantize_gated(to_dev(x), act)
    torch.cuda.synchronize()
    o = O.mx_quantize_gated(x, act)
    mx_outputs_equal(g, o, f"C4 act {act}")


@pytest.mark.parametrize("two_d", [False, True])
def test_c5_nvfp4_16384(two_d):
    x = W.make("c5_nvfp4_16384")
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16(xd)
    g = mx.nvfp4_quantize_transpose(xd, amax, two_d=two_d)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose(x, two_d=two_d)
    assert g["sg"].item() == o["sg"]
    mx_outputs_equal(g, o, f"C5 nvfp4 two_d={two_d}")


def test_dsilu_dbias_8192():
    x, grad = W.make("f1_dsilu_dbias_8192")
    f = mx.FUSE_DSILU | mx.FUSE_DBIAS
    g = mx.mx_quantize(to_dev(x), to_dev(grad), fusion=f)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, fusion=f, want_y=True)
    mx_outputs_equal(g, o, "dSiLU + dbias")
    ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
    assert_dbias_close(g["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_gated_backward_8192(act):
    grad, x = W.make("f1_dgated_8192")
    g = mx.mx_quantize_dgated(to_dev(grad), to_dev(x), act)
    torch.cuda.synchronize()
    o = O.mx_quantize_dgated(grad, x, act)
    mx_outputs_equal(g, o, f"gated backward act {act}")


def test_c1_special_256x512():
    x = W.special_256x512()
    g = mx.mx_quantize(to_dev(x))
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize(x), "C1")


@pytest.mark.parametrize("M,K", [(1 << 23, 32), (32, 1 << 23), ((1 << 23) - 16, 40),
                                 # ragged row counts: the tiled kernel's variant for
                                 # transposed rows at any byte
                                 ((1 << 23) - 1, 8), (17, 1 << 23)])
@pytest.mark.parametrize("layout", [0, mx.SCALE_TILED], ids=["compact", "tiled"])
def test_mxfp8_maximum_dimensions(M, K, layout):
    """The largest row count (2^23 rows of 32 or 40 columns: the most
    sub-tiles along M, and a transposed output with rows of 2^23 bytes) and
    the largest row length (32 rows of 2^23 columns: in-tile load offsets up
    to 31 * 2^24).  Offsets up to 127 * 2^24, just below 2^31, are reached by
    the 128-row casts of test_gpu_limits.py."""
    x = W.loguniform_rows(M, K, seed=90)
    g = mx.mx_quantize(to_dev(x), axis=3 | layout)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, axis=3 | layout)
    mx_outputs_equal(g, o, f"max dims {M}x{K} {layout}")


@pytest.mark.parametrize("M,K", [(1 << 23, 16), (16, 1 << 23), ((1 << 23) - 1, 16), (17, 1 << 23)])
def test_nvfp4_maximum_dimensions(M, K):
    x = W.student_t_rows(M, K, seed=91)
    xd = to_dev(x)
    g = mx.nvfp4_quantize_transpose(xd, mx.mx_absmax_bf16(xd))
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose(x)
    mx_outputs_equal(g, o, f"nvfp4 max dims {M}x{K}")


@pytest.fixture(scope="module")
def moe_rows():
    return W.moe_group_rows(16384, groups=8, seed=8)


def test_grouped_mxfp8_8x_16384x7168(moe_rows):
    x = W.make("f4_grouped_moe")
    g = mx.mx_quantize_grouped(to_dev(x), moe_rows)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize_grouped(x, moe_rows), "grouped mxfp8 8 experts")


@pytest.mark.parametrize("two_d", [False, True])
def test_grouped_nvfp4_8x_16384x7168(moe_rows, two_d):
    x = W.make("f4_grouped_moe")
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16_grouped(xd, moe_rows)
    g = mx.nvfp4_quantize_transpose_grouped(xd, moe_rows, amax, two_d=two_d)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose_grouped(x, moe_rows, two_d=two_d)
    mx_outputs_equal(g, o, f"grouped nvfp4 8 experts two_d={two_d}")
    assert np.array_equal(g["sg"].cpu().numpy(), o["sg"])


def test_grouped_swiglu_8x_16384x4096(moe_rows):
    x = W.make("f4_grouped_moe", 16384, 4096)
    g = mx.mx_quantize_gated_grouped(to_dev(x), moe_rows, mx.GATED_SWIGLU)
    torch.cuda.synchronize()
    o = O.mx_quantize_gated_grouped(x, moe_rows, mx.GATED_SWIGLU)
    mx_outputs_equal(g, o, "grouped swiglu 8 experts")
