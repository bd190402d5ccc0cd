"""GPU parity of the MXFP8 casts whose row length is a multiple of 8 but whose
row count (or a group's) is not a multiple of 16: the tiled kernel takes them,
and the variant of its transposed flush for transposed rows that start at any
byte writes q_col (each sub-tile's 8 aligned 16-byte pieces per row, the
previous sub-tile's last bytes carried in LDS).  MoE stacks with ragged expert
sizes are the common case.  Compared with the oracle byte for byte in canary-
filled buffers with guard bands: plain casts in both output sets and every
format and scale layout, the pre-ops with dbias, the gated casts and their
backward, grouped stacks (one launch over groups of any size, empty ones
included), the allocation-free cast, and a 16383 x 16384 tensor."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev
from test_gpu_any_shape import FLAG_IDS, FLAGS, Guarded

pytestmark = pytest.mark.gpu

# M not a multiple of 16, K a multiple of 8: single sub-tiles, walks of many
# sub-tiles (the carry across them), several walks per strip, partial strips
SHAPES = [(1, 8), (17, 8), (40, 64), (129, 256), (255, 264), (1000, 520), (4097, 256),
          (33, 7168), (2049, 1032)]


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("flags", FLAGS, ids=FLAG_IDS)
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", SHAPES)
def test_ragged_plain(M, K, axis, flags):
    x = W.loguniform_rows(M, K, seed=9100 + 3 * M + K)
    g = Guarded(M, K, axis | flags)
    r = mx.mx_quantize(to_dev(x), axis=axis | flags, out=g.out)
    torch.cuda.synchronize()
    what = f"{M}x{K} axis {axis} flags {flags}"
    mx_outputs_equal(r, O.mx_quantize(x, axis=axis | flags), what)
    g.guards_intact(what)


@pytest.mark.parametrize("fusion", [mx.FUSE_GELU | mx.FUSE_DBIAS, mx.FUSE_DGELU | mx.FUSE_DBIAS,
                                    mx.FUSE_DSILU, mx.FUSE_DBIAS, mx.FUSE_GELU])
@pytest.mark.parametrize("M,K", [(401, 1048), (33, 8), (1, 264), (1313, 256)])
def test_ragged_fused(M, K, fusion):
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    mode = mx.SCALE_TILED if fusion & 1 else 0
    g = Guarded(M, K, 3 | mode)
    r = mx.mx_quantize(to_dev(x), to_dev(grad), axis=3 | mode, fusion=fusion, out=g.out)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=3 | mode, fusion=fusion, want_y=True)
    mx_outputs_equal(r, o, f"{M}x{K} fusion {fusion}")
    g.guards_intact(f"{M}x{K} fusion {fusion}")
    if fusion & mx.FUSE_DBIAS:
        ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
        assert_dbias_close(r["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
@pytest.mark.parametrize("M,N", [(1, 8), (47, 40), (401, 264), (129, 8), (777, 1024)])
def test_ragged_gated(M, N, act):
    x = W.make("c4_gated_8192", M, 2 * N)
    g = Guarded(M, N, 3)
    r = mx.mx_quantize_gated(to_dev(x), act, axis=3, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_gated(x, act, axis=3), f"gated {M}x{N}")
    g.guards_intact(f"gated {M}x{N}")
    grad, xb = W.make("f1_dgated_8192", M, N)
    axis = 2 | mx.SCALE_TILED
    g = Guarded(M, 2 * N, axis)
    r = mx.mx_quantize_dgated(to_dev(grad), to_dev(xb), act, axis=axis, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_dgated(grad, xb, act, axis=axis), f"dgated {M}x{N}")
    g.guards_intact(f"dgated {M}x{N}")


# stacks with ragged groups (empty ones too) and the MoE shape with expert
# sizes drawn without rounding
GROUPS = [([1101, 0, 17, 640, 3], 520), ([5, 1, 0, 2], 8), ([4099, 0, 3001, 17, 9000], 264),
          (W.moe_group_rows(16384, 8, seed=8, step=1), 7168)]


@pytest.mark.parametrize("flags", FLAGS, ids=FLAG_IDS)
@pytest.mark.parametrize("axis", [2, 3])
@pytest.mark.parametrize("rows,K", GROUPS, ids=["mixed", "tiny", "large", "moe"])
def test_ragged_grouped(rows, K, axis, flags):
    M = sum(rows)
    x = W.loguniform_rows(M, K, seed=9200 + M + K)
    g = Guarded(M, K, axis | flags, grouped_rows=rows)
    r = mx.mx_quantize_grouped(to_dev(x), rows, axis=axis | flags, out=g.out)
    torch.cuda.synchronize()
    what = f"grouped {rows} K={K} axis {axis} flags {flags}"
    mx_outputs_equal(r, O.mx_quantize_grouped(x, rows, axis=axis | flags), what)
    g.guards_intact(what)


def test_ragged_grouped_row_only():
    """Row-wise alone: the plain grouped kernel, whatever the group sizes."""
    rows, K = [301, 0, 47, 900, 5], 264
    M = sum(rows)
    x = W.loguniform_rows(M, K, seed=9300)
    g = Guarded(M, K, 1, grouped_rows=rows)
    r = mx.mx_quantize_grouped(to_dev(x), rows, axis=1, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_grouped(x, rows, axis=1), "grouped row-wise")
    g.guards_intact("grouped row-wise")


def test_ragged_grouped_fused_dbias():
    rows, K = [301, 0, 47, 900], 528
    M = sum(rows)
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    fusion = mx.FUSE_DSILU | mx.FUSE_DBIAS
    r = mx.mx_quantize_grouped(to_dev(x), rows, grad=to_dev(grad), fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize_grouped(x, rows, grad=grad, fusion=fusion)
    mx_outputs_equal(r, o, "grouped dSiLU + dbias")
    r0 = 0
    for gi, m in enumerate(rows):
        if m == 0:
            assert torch.all(r["dbias"][gi] == 0)
            continue
        y = O.mx_quantize(np.ascontiguousarray(x[r0:r0 + m]),
                          grad=np.ascontiguousarray(grad[r0:r0 + m]), fusion=fusion,
                          want_y=True)["y"]
        ycols = np.abs(W.bf16_to_f32(y).astype(np.float64)).sum(axis=0)
        assert_dbias_close(r["dbias"][gi], o["dbias"][gi], ycols, f"group {gi}")
        r0 += m


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_ragged_grouped_gated(act):
    rows, N = [33, 0, 100, 7, 250], 264
    M = sum(rows)
    x = W.make("c4_gated_8192", M, 2 * N)
    r = mx.mx_quantize_gated_grouped(to_dev(x), rows, act, axis=3 | mx.SCALE_TILED)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_gated_grouped(x, rows, act, axis=3 | mx.SCALE_TILED),
                     f"grouped gated {act}")
    grad, xb = W.make("f1_dgated_8192", M, N)
    r = mx.mx_quantize_gated_grouped(to_dev(xb), rows, act, grad=to_dev(grad), axis=3)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_gated_grouped(xb, rows, act, axis=3, grad=grad),
                     f"grouped dgated {act}")


def test_ragged_noalloc_with_dbias():
    M, K = 333, 1000
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    fusion = mx.FUSE_GELU | mx.FUSE_DBIAS
    g = Guarded(M, K, 3)
    out = dict(g.out, dbias=torch.empty(K, dtype=torch.float32, device="cuda"))
    r = mx.mx_quantize_noalloc(to_dev(x), out, axis=3, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=3, fusion=fusion, want_y=True)
    mx_outputs_equal(r, o, "noalloc ragged")
    g.guards_intact("noalloc ragged")
    ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
    assert_dbias_close(r["dbias"], o["dbias"], ycols)


def test_ragged_metric_sized():
    """16383 x 16384: the metric tensor less one row, both outputs."""
    M, K = 16383, 16384
    x = W.loguniform_rows(M, K, seed=93)
    g = Guarded(M, K, 3)
    r = mx.mx_quantize(to_dev(x), axis=3, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize(x, axis=3), "16383x16384")
    g.guards_intact("16383x16384")
