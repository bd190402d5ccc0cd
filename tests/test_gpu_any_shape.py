"""GPU parity of the casts at shapes the tiled kernels do not take -- row
counts that are not multiples of 16 and row lengths that are not multiples of
8 (MXFP8) or 16 (NVFP4), down to a single element -- which go to the
any-shape kernels.  Compared with the oracle byte for byte (both directions;
MXFP8 with compact and tiled scales and every format variant, for the plain
cast, the pre-ops with dbias, the gated casts and their backward, the
grouped casts, the fused values and the allocation-free cast; NVFP4 1D and
2D, single and grouped, with non-finite and tiny-scale tensors).  Outputs are
preallocated and filled with a canary between guard bands, so a byte the
kernel fails to write (tile-layout padding included) or writes past its
tensor is seen."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu

CANARY, GUARD = 0xA5, 512

SHAPES = [(1, 1), (1, 40), (40, 1), (3, 7), (17, 9), (40, 64), (48, 36), (100, 129), (129, 300),
          (65, 1000), (1000, 65), (191, 257), (255, 12), (12, 255), (2049, 1030)]
FLAGS = [0, mx.SCALE_TILED, mx.ELEM_E5M2 | mx.SCALE_ROUND_UP, mx.ELEM_E5M2 | mx.SCALE_TILED]
FLAG_IDS = ["e4m3", "tiled", "e5m2-up", "e5m2-tiled"]


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


def scale_shape(rows, cols, axis):
    if axis & mx.SCALE_TILED:
        return (mx.mx_scale_size(rows, cols, axis),)
    return (rows, -(-cols // 32))


class Guarded:
    """The outputs of an M x K cast in canary-filled buffers with guard bands."""

    def __init__(self, M, K, axis, grouped_rows=None):
        shapes = {}
        if axis & mx.ROWWISE:
            shapes["q_row"] = (M, K)
            shapes["s_row"] = (self.grouped_scale(K, grouped_rows, axis, 0),) if grouped_rows \
                else scale_shape(M, K, axis)
        if axis & mx.COLWISE:
            shapes["q_col"] = (K * M,) if grouped_rows else (K, M)
            shapes["s_col"] = (self.grouped_scale(K, grouped_rows, axis, 1),) if grouped_rows \
                else scale_shape(K, M, axis)
        self.bufs, self.out = {}, {}
        for name, shape in shapes.items():
            n = int(np.prod(shape))
            b = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
            self.bufs[name] = b
            self.out[name] = b[GUARD:GUARD + n].view(shape)

    @staticmethod
    def grouped_scale(K, rows, axis, colwise):
        return mx.mx_grouped_scale_size(K, rows, axis, colwise)

    def guards_intact(self, what):
        for name, b in self.bufs.items():
            assert torch.all(b[:GUARD] == CANARY) and torch.all(b[-GUARD:] == CANARY), (what, name)


@pytest.mark.parametrize("flags", FLAGS, ids=FLAG_IDS)
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", SHAPES)
def test_any_plain(M, K, axis, flags):
    x = W.loguniform_rows(M, K, seed=7000 + 3 * M + K)
    g = Guarded(M, K, axis | flags)
    r = mx.mx_quantize(to_dev(x), axis=axis | flags, out=g.out)
    torch.cuda.synchronize()
    what = f"{M}x{K} axis {axis} flags {flags}"
    mx_outputs_equal(r, O.mx_quantize(x, axis=axis | flags), what)
    g.guards_intact(what)


@pytest.mark.parametrize("fusion", [mx.FUSE_GELU | mx.FUSE_DBIAS, mx.FUSE_DGELU | mx.FUSE_DBIAS,
                                    mx.FUSE_DSILU, mx.FUSE_DBIAS, mx.FUSE_DSILU | mx.FUSE_DBIAS])
@pytest.mark.parametrize("M,K", [(401, 1049), (33, 7), (1, 300)])
def test_any_fused(M, K, fusion):
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    mode = mx.ELEM_E5M2 if fusion & 1 else 0
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
@pytest.mark.parametrize("M,N", [(1, 1), (47, 41), (113, 70), (401, 263), (16, 20), (64, 33)])
def test_any_gated(M, N, act):
    x = W.make("c4_gated_8192", M, 2 * N)
    g = Guarded(M, N, 3)
    r = mx.mx_quantize_gated(to_dev(x), act, axis=3, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_gated(x, act, axis=3), f"gated {M}x{N}")
    g.guards_intact(f"gated {M}x{N}")
    grad, xb = W.make("f1_dgated_8192", M, N)
    axis = 3 | mx.SCALE_TILED
    g = Guarded(M, 2 * N, axis)
    r = mx.mx_quantize_dgated(to_dev(grad), to_dev(xb), act, axis=axis, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_dgated(grad, xb, act, axis=axis), f"dgated {M}x{N}")
    g.guards_intact(f"dgated {M}x{N}")


@pytest.mark.parametrize("op", [mx.FUSE_GELU, mx.FUSE_DGELU, mx.FUSE_DSILU,
                                mx.OP_GATED | mx.GATED_SWIGLU, mx.OP_DGATED | mx.GATED_GEGLU])
def test_any_fused_values(op):
    M, N = 47, 41
    if op & mx.OP_DGATED:
        grad, x = W.make("f1_dgated_8192", M, N)
        y = mx.mx_fused_values(to_dev(x), to_dev(grad), op=op)
        want = O.mx_quantize_dgated(grad, x, op & 3, axis=1, want_y=True)["y"]
    elif op & mx.OP_GATED:
        x = W.make("c4_gated_8192", M, 2 * N)
        y = mx.mx_fused_values(to_dev(x), op=op)
        want = O.mx_quantize_gated(x, op & 3, axis=1, want_y=True)["y"]
    else:
        x, grad = W.make("c3_gelu_dbias_8192", M, N)
        y = mx.mx_fused_values(to_dev(x), to_dev(grad), op=op)
        want = O.mx_quantize(x, grad=grad, fusion=op, axis=1, want_y=True)["y"]
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want)


GROUPS = [([1101, 0, 17, 640, 3], 517), ([5, 1, 0, 2], 3), ([4099, 0, 3001, 17, 9000], 4100)]


@pytest.mark.parametrize("flags", [0, mx.SCALE_TILED], ids=["compact", "tiled"])
@pytest.mark.parametrize("rows,K", GROUPS)
def test_any_grouped(rows, K, flags):
    M = sum(rows)
    x = W.loguniform_rows(M, K, seed=8000 + M + K)
    g = Guarded(M, K, 3 | flags, grouped_rows=rows)
    r = mx.mx_quantize_grouped(to_dev(x), rows, axis=3 | flags, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize_grouped(x, rows, axis=3 | flags), f"grouped {rows} K={K}")
    g.guards_intact(f"grouped {rows} K={K}")


def test_any_grouped_fused_dbias():
    rows, K = [301, 0, 47, 900], 523
    M = sum(rows)
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    fusion = mx.FUSE_DGELU | mx.FUSE_DBIAS
    r = mx.mx_quantize_grouped(to_dev(x), rows, grad=to_dev(grad), fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize_grouped(x, rows, grad=grad, fusion=fusion)
    mx_outputs_equal(r, o, "grouped dGELU + dbias")
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
def test_any_grouped_gated(act):
    rows, N = [33, 0, 100, 7], 45
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


def test_any_noalloc_with_dbias():
    M, K = 333, 1001
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    fusion = mx.FUSE_GELU | mx.FUSE_DBIAS
    g = Guarded(M, K, 3)
    out = dict(g.out, dbias=torch.empty(K, dtype=torch.float32, device="cuda"))
    r = mx.mx_quantize_noalloc(to_dev(x), out, axis=3, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=3, fusion=fusion, want_y=True)
    mx_outputs_equal(r, o, "noalloc any-shape")
    g.guards_intact("noalloc any-shape")
    ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
    assert_dbias_close(r["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("flags", [0, mx.SCALE_TILED, mx.ELEM_E5M2 | mx.SCALE_ROUND_UP],
                         ids=["e4m3", "tiled", "e5m2-up"])
def test_any_large_multi_step_walks(flags):
    """8191 x 8193: walks of 8 steps of 64 rows, the last one partial, in 65
    strips whose last holds a single column."""
    M, K = 8191, 8193
    x = W.loguniform_rows(M, K, seed=91)
    g = Guarded(M, K, 3 | flags)
    r = mx.mx_quantize(to_dev(x), axis=3 | flags, out=g.out)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize(x, axis=3 | flags), f"8191x8193 flags {flags}")
    g.guards_intact(f"8191x8193 flags {flags}")


def test_any_large_gelu_dbias():
    M, K = 8191, 8193
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    fusion = mx.FUSE_GELU | mx.FUSE_DBIAS
    r = mx.mx_quantize(to_dev(x), axis=3, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, axis=3, fusion=fusion, want_y=True)
    mx_outputs_equal(r, o, "8191x8193 GELU + dbias")
    ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
    assert_dbias_close(r["dbias"], o["dbias"], ycols)


def test_any_metric_sized():
    """16383 x 16383, the metric tensor less one row and one column."""
    M = K = 16383
    x = W.loguniform_rows(M, K, seed=92)
    r = mx.mx_quantize(to_dev(x), axis=3)
    torch.cuda.synchronize()
    mx_outputs_equal(r, O.mx_quantize(x, axis=3), "16383^2")


# --- NVFP4 of any shape ---------------------------------------------------------

def nv_guarded(M, K, axis, n_sg=1, qcol=None, scol=None):
    """NVFP4 outputs ([rows][ceil(cols/2)] codes, [rows][ceil(cols/16)] scales)
    in canary-filled buffers with guard bands."""
    shapes = {}
    if axis & mx.ROWWISE:
        shapes["q_row"] = (M, -(-K // 2))
        shapes["s_row"] = (M, -(-K // 16))
    if axis & mx.COLWISE:
        shapes["q_col"] = (qcol,) if qcol is not None else (K, -(-M // 2))
        shapes["s_col"] = (scol,) if scol is not None else (K, -(-M // 16))
    g = Guarded.__new__(Guarded)
    g.bufs, g.out = {}, {}
    for name, shape in shapes.items():
        n = int(np.prod(shape))
        b = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        g.bufs[name] = b
        g.out[name] = b[GUARD:GUARD + n].view(shape)
    g.out["sg"] = torch.empty(n_sg, dtype=torch.float32, device="cuda")
    return g


def nv_both(x, axis=3, two_d=False):
    M, K = x.shape
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16(xd)
    g = nv_guarded(M, K, axis)
    r = mx.nvfp4_quantize_transpose(xd, amax, axis=axis, two_d=two_d, out=g.out)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose(x, axis=axis, two_d=two_d)
    return r, o, g


NV_SHAPES = [(1, 1), (1, 40), (40, 1), (3, 7), (17, 9), (16, 24), (24, 16), (48, 36), (100, 129),
             (129, 300), (65, 1000), (1000, 65), (191, 257), (2049, 1030)]


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", NV_SHAPES)
def test_nv_any(M, K, axis, two_d):
    x = W.student_t_rows(M, K, seed=9000 + 3 * M + K)
    r, o, g = nv_both(x, axis, two_d)
    what = f"nvfp4 {M}x{K} axis {axis} 2d={two_d}"
    assert r["sg"].item() == o["sg"], what
    mx_outputs_equal(r, o, what)
    g.guards_intact(what)


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
def test_nv_any_nonfinite_and_tiny_scale(two_d):
    x = W.student_t_rows(131, 77, seed=9100)
    x[70, 76] = 0x7FC0                       # NaN: 0x7F scales, zero codes
    r, o, g = nv_both(x, 3, two_d)
    assert np.isnan(r["sg"].item()) and np.isnan(o["sg"])
    mx_outputs_equal(r, o, "nvfp4 any non-finite")
    g.guards_intact("nvfp4 any non-finite")
    x = W.normal(33, 71, seed=9101, sigma=1e-37)   # multipliers that overflow to Inf
    x[0, :16] = 0
    x[1, 0] = 0x8000
    r, o, g = nv_both(x, 3, two_d)
    assert r["sg"].item() == o["sg"]
    mx_outputs_equal(r, o, "nvfp4 any tiny S_g")


def test_nv_any_every_scale_code():
    rng = np.random.default_rng(9102)
    M, K = 63, 2047
    nb = -(-K // 16)
    t = np.linspace(0, 1, M * nb).reshape(M, nb)
    x = rng.standard_normal((M, nb * 16)).astype(np.float32) * np.repeat(2.0 ** (-19 * t), 16, axis=1)
    x = W.bf16_bits(np.ascontiguousarray(x[:, :K]).astype(np.float32))
    r, o, g = nv_both(x)
    assert set(np.unique(o["s_row"]).tolist()) == set(range(127))
    mx_outputs_equal(r, o, "nvfp4 any scale sweep")


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
@pytest.mark.parametrize("rows,K", [([1101, 0, 17, 640, 3], 517), ([5, 1, 0, 2], 3),
                                    ([4099, 0, 3001, 17, 9000], 4100), ([48, 16, 0, 32], 40)])
def test_nv_any_grouped(rows, K, two_d):
    M = sum(rows)
    x = W.student_t_rows(M, K, seed=9200 + M + K)
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16_grouped(xd, rows)
    torch.cuda.synchronize()
    r0 = 0
    for gi, m in enumerate(rows):     # the grouped absmax over ragged groups
        want = O.absmax(np.ascontiguousarray(x[r0:r0 + m])) if m else 0.0
        assert amax[gi].item() == want, (gi, m)
        r0 += m
    qcol = K * sum(-(-m // 2) for m in rows)
    scol = K * sum(-(-m // 16) for m in rows)
    g = nv_guarded(M, K, 3, len(rows), qcol, scol)
    r = mx.nvfp4_quantize_transpose_grouped(xd, rows, amax, two_d=two_d, out=g.out)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose_grouped(x, rows, two_d=two_d)
    assert np.array_equal(r["sg"].cpu().numpy(), o["sg"])
    mx_outputs_equal(r, o, f"grouped nvfp4 {rows} K={K} 2d={two_d}")
    g.guards_intact(f"grouped nvfp4 {rows} K={K}")


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
def test_nv_any_large(two_d):
    x = W.student_t_rows(8191, 8193, seed=9300)
    r, o, g = nv_both(x, 3, two_d)
    assert r["sg"].item() == o["sg"]
    mx_outputs_equal(r, o, f"nvfp4 8191x8193 2d={two_d}")
    g.guards_intact("nvfp4 8191x8193")
