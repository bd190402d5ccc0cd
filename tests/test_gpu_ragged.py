"""GPU parity of the casts whose row length is a multiple of 8 (MXFP8) or 16
(NVFP4) but whose row count (or a group's) is not a multiple of 16: the tiled
kernels take them, and the variant of their transposed flush for transposed
rows that start at any byte writes q_col (whole 128-byte lines from two staged
tiles, bytes at a walk's ends one by one).  MoE stacks with unrounded expert
sizes are the common case.  Compared with the oracle byte for byte in canary-
filled buffers with guard bands.  MXFP8: plain casts in every output set,
format and scale layout, the pre-ops with dbias, the gated casts and their
backward, grouped stacks (one launch over groups of any size, empty ones
included), the allocation-free cast and a 16383 x 16384 tensor.  NVFP4: 1D
and 2D blocks, single and grouped, non-finite and tiny-scale tensors, and
16383 x 16384."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev
from test_gpu_any_shape import FLAG_IDS, FLAGS, Guarded, nv_both, nv_guarded

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


# --- NVFP4: K a multiple of 16, rows (or a group's) not ---------------------

NV_SHAPES = [(1, 16), (17, 32), (40, 64), (129, 256), (255, 272), (1000, 528), (4097, 256),
             (33, 7168), (2049, 1040)]


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", NV_SHAPES)
def test_ragged_nvfp4(M, K, axis, two_d):
    x = W.student_t_rows(M, K, seed=9400 + 3 * M + K)
    r, o, g = nv_both(x, axis, two_d)
    what = f"nvfp4 {M}x{K} axis {axis} 2d={two_d}"
    assert r["sg"].item() == o["sg"], what
    mx_outputs_equal(r, o, what)
    g.guards_intact(what)


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
def test_ragged_nvfp4_nonfinite_and_tiny_scale(two_d):
    x = W.student_t_rows(131, 80, seed=9500)
    x[70, 76] = 0x7FC0                       # NaN: 0x7F scales, zero codes
    r, o, g = nv_both(x, 3, two_d)
    assert np.isnan(r["sg"].item()) and np.isnan(o["sg"])
    mx_outputs_equal(r, o, "nvfp4 ragged non-finite")
    g.guards_intact("nvfp4 ragged non-finite")
    x = W.normal(33, 64, seed=9501, sigma=1e-37)   # multipliers that overflow to Inf
    x[0, :16] = 0
    x[1, 0] = 0x8000
    r, o, g = nv_both(x, 3, two_d)
    assert r["sg"].item() == o["sg"]
    mx_outputs_equal(r, o, "nvfp4 ragged tiny S_g")
    g.guards_intact("nvfp4 ragged tiny S_g")


NV_GROUPS = [([1101, 0, 17, 640, 3], 528), ([5, 1, 0, 2], 16), ([4099, 0, 3001, 17, 9000], 272),
             (W.moe_group_rows(16384, 8, seed=8, step=1), 7168)]


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
@pytest.mark.parametrize("axis", [2, 3])
@pytest.mark.parametrize("rows,K", NV_GROUPS, ids=["mixed", "tiny", "large", "moe"])
def test_ragged_nvfp4_grouped(rows, K, axis, two_d):
    M = sum(rows)
    x = W.student_t_rows(M, K, seed=9600 + M + K)
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16_grouped(xd, rows)
    qcol = K * sum(-(-m // 2) for m in rows)
    scol = K * sum(-(-m // 16) for m in rows)
    g = nv_guarded(M, K, axis, len(rows), qcol, scol)
    r = mx.nvfp4_quantize_transpose_grouped(xd, rows, amax, axis=axis, two_d=two_d, out=g.out)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose_grouped(x, rows, axis=axis, two_d=two_d)
    what = f"grouped nvfp4 {rows} K={K} axis {axis} 2d={two_d}"
    assert np.array_equal(r["sg"].cpu().numpy(), o["sg"]), what
    mx_outputs_equal(r, o, what)
    g.guards_intact(what)


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
def test_ragged_nvfp4_large(two_d):
    """16383 x 16384: the NVFP4 metric-sized tensor less one row."""
    x = W.student_t_rows(16383, 16384, seed=9700)
    r, o, g = nv_both(x, 3, two_d)
    assert r["sg"].item() == o["sg"]
    mx_outputs_equal(r, o, f"nvfp4 16383x16384 2d={two_d}")
    g.guards_intact("nvfp4 16383x16384")
