"""GPU parity of the GEMM-ready (MFMA tile) scale layout, MX_SCALE_TILED,
against the oracle byte for byte: scale tensors in the tile layout (padding
included), element tensors unchanged.

Shapes cover partial last block tiles (K/32 and M/32 not multiples of 8),
walks of odd length at the tensor's end, tensors of one sub-tile row (where the
walk length is raised to two), every kernel family and the format flags, and
the 16384^2 workload at full size.
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

T = mx.SCALE_TILED


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", [(32, 32), (64, 96), (128, 256), (160, 800), (288, 544),
                                 (416, 1056), (1024, 4096), (8192, 256)])
def test_plain_tiled(M, K, axis):
    x = W.loguniform_rows(M, K, seed=3000 + M + K)
    g = mx.mx_quantize(to_dev(x), axis=axis | T)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, axis=axis | T)
    mx_outputs_equal(g, o, f"tiled {M}x{K} axis {axis}")
    if axis & 1:
        assert g["s_row"].numel() == O.tiled_scale_bytes(M, K // 32)


def test_tiled_equals_compact_rearranged():
    x = W.loguniform_rows(416, 1056, seed=31)
    c = mx.mx_quantize(to_dev(x), axis=3)
    t = mx.mx_quantize(to_dev(x), axis=3 | T)
    torch.cuda.synchronize()
    assert torch.equal(c["q_row"], t["q_row"]) and torch.equal(c["q_col"], t["q_col"])
    assert np.array_equal(t["s_row"].cpu().numpy(), O.scale_tiles(c["s_row"].cpu().numpy()))
    assert np.array_equal(t["s_col"].cpu().numpy(), O.scale_tiles(c["s_col"].cpu().numpy()))


@pytest.mark.parametrize("mode", [0, mx.ELEM_E5M2 | mx.SCALE_ROUND_UP])
@pytest.mark.parametrize("fusion", [mx.FUSE_GELU | mx.FUSE_DBIAS, mx.FUSE_DSILU, mx.FUSE_DBIAS])
def test_fused_tiled(fusion, mode):
    M, K = 288, 544
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    g = mx.mx_quantize(to_dev(x), to_dev(grad), axis=3 | T | mode, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=3 | T | mode, fusion=fusion, want_y=True)
    mx_outputs_equal(g, o, f"tiled fusion {fusion} mode {mode}")
    if fusion & mx.FUSE_DBIAS:
        ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
        assert_dbias_close(g["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_gated_tiled(act):
    x = W.make("c4_gated_8192", 160, 576)
    g = mx.mx_quantize_gated(to_dev(x), act, axis=3 | T)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize_gated(x, act, axis=3 | T), f"tiled gated {act}")
    grad, xb = W.make("f1_dgated_8192", 96, 160)
    g = mx.mx_quantize_dgated(to_dev(grad), to_dev(xb), act, axis=3 | T)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize_dgated(grad, xb, act, axis=3 | T), f"tiled dgated {act}")


def test_dim0_dim1_16384_tiled():
    x = W.make("c2_dim1_16384")
    g = mx.mx_quantize(to_dev(x), axis=3 | T)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize(x, axis=3 | T), "16384 tiled")


def test_deep_walks_with_odd_tail_tiled():
    """131 sub-tile rows at K = 8192 give walks of 8 sub-tiles and a last walk
    of 3: its final column-scale tile is half real blocks, half zero padding."""
    x = W.loguniform_rows(16768, 8192, seed=32)
    g = mx.mx_quantize(to_dev(x), axis=3 | T)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize(x, axis=3 | T), "16768x8192 tiled")
