"""The model shapes of the TransformerEngine results tables ("Full
per-workload numbers": 2048 x 12288, 4096 x 4096, 4096 x 14336, 8192 x 8192,
16384 x 5120, 8192 x 28672) as extra full-size parity shapes: the MXFP8 cast
in both directions, the GELU + dbias cast, the SwiGLU cast of the shape as a
[gate | linear] input, and NVFP4 1D, every output element compared with the
oracle (dbias within the tolerance of the fused tests).  N(0, 1) inputs, one
seed per shape."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(2048, 12288), (4096, 4096), (4096, 14336), (8192, 8192), (16384, 5120), (8192, 28672)]


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


def inputs(M, K):
    return W.normal(M, K, seed=3000 + M // 1024 + K // 1024)


@pytest.mark.parametrize("M,K", SHAPES, ids=[f"{m}x{k}" for m, k in SHAPES])
def test_mxfp8_both_directions(M, K):
    x = inputs(M, K)
    g = mx.mx_quantize(to_dev(x))
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize(x), f"mxfp8 {M}x{K}")


@pytest.mark.parametrize("M,K", SHAPES, ids=[f"{m}x{k}" for m, k in SHAPES])
def test_gelu_dbias(M, K):
    x = inputs(M, K)
    f = mx.FUSE_GELU | mx.FUSE_DBIAS
    g = mx.mx_quantize(to_dev(x), fusion=f)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, fusion=f, want_y=True)
    mx_outputs_equal(g, o, f"gelu+dbias {M}x{K}")
    ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
    assert_dbias_close(g["dbias"], o["dbias"], ycols, f"gelu+dbias {M}x{K}")


@pytest.mark.parametrize("M,K", SHAPES, ids=[f"{m}x{k}" for m, k in SHAPES])
def test_swiglu(M, K):
    x = inputs(M, K)                       # [gate | linear], N = K / 2
    g = mx.mx_quantize_gated(to_dev(x), mx.GATED_SWIGLU)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize_gated(x, mx.GATED_SWIGLU), f"swiglu {M}x{K}")


@pytest.mark.parametrize("M,K", SHAPES, ids=[f"{m}x{k}" for m, k in SHAPES])
def test_nvfp4(M, K):
    x = inputs(M, K)
    g = mx.nvfp4_quantize_transpose(to_dev(x))
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose(x)
    assert g["sg"].item() == o["sg"]
    mx_outputs_equal(g, o, f"nvfp4 {M}x{K}")
