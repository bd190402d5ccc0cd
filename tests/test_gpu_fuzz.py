"""Seeded random combinations of the casts' options, each compared with the
oracle byte for byte (dbias within its tolerance): shapes with partial edges,
output selection, element format, scale rule and layout, pre-op and dbias for
the MXFP8 cast; the gated casts and their backward; NVFP4 1D and 2D; grouped
casts with random expert sizes; the same at any shape (sizes from 1 up, not
multiples of 16 or 8); and at row counts that are not multiples of 16 with
aligned rows (the tiled kernels' ragged variants, up to several sub-tiles per
walk).  The cases are drawn from fixed seeds, so the set
is the same on every run; each case's parameters are in its test id."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu

FORMATS = [0, mx.ELEM_E5M2, mx.SCALE_ROUND_UP, mx.ELEM_E5M2 | mx.SCALE_ROUND_UP]
FUSIONS = [mx.FUSE_NONE, mx.FUSE_GELU, mx.FUSE_DGELU, mx.FUSE_DSILU]


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


def planted(x, rng):
    """Random tensor with a few degenerate blocks planted: zeros, -0, a lone
    large value and a row of subnormals."""
    x = x.copy()
    M, K = x.shape
    r, c = rng.integers(0, M), rng.integers(0, K)
    x[r, :] = 0
    x[rng.integers(0, M), rng.integers(0, K)] = 0x8000
    x[rng.integers(0, M), c] = 0x7F00                 # ~1.7e38
    x[rng.integers(0, M), :] &= 0x807F                # bf16 subnormals
    return x


def mx_cases(n=160, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, K = 16 * int(rng.integers(1, 35)), 8 * int(rng.integers(1, 131))
        axis = int(rng.integers(1, 4))
        flags = FORMATS[int(rng.integers(0, 4))] | (mx.SCALE_TILED if rng.random() < 0.3 else 0)
        fusion = FUSIONS[int(rng.integers(0, 4))] | (mx.FUSE_DBIAS if rng.random() < 0.4 else 0)
        out.append(pytest.param(i, M, K, axis, flags, fusion,
                                id=f"{i}-{M}x{K}-a{axis}-f{flags}-u{fusion}"))
    return out


@pytest.mark.parametrize("i,M,K,axis,flags,fusion", mx_cases())
def test_mx_quantize_fuzz(i, M, K, axis, flags, fusion):
    rng = np.random.default_rng(7000 + i)
    x = planted(W.loguniform_rows(M, K, seed=7000 + i) if i % 2 else
                W.normal(M, K, seed=7000 + i, sigma=2.0), rng)
    grad = W.normal(M, K, seed=8000 + i) if (fusion & 0xF) in (mx.FUSE_DGELU, mx.FUSE_DSILU) else None
    g = mx.mx_quantize(to_dev(x), None if grad is None else to_dev(grad), axis=axis | flags,
                       fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=axis | flags, fusion=fusion, want_y=True)
    mx_outputs_equal(g, o, f"case {i}")
    if fusion & mx.FUSE_DBIAS:
        ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
        assert_dbias_close(g["dbias"], o["dbias"], ycols, f"case {i} dbias")


def gated_cases(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N = 16 * int(rng.integers(1, 25)), 8 * int(rng.integers(1, 65))
        act = [mx.GATED_SWIGLU, mx.GATED_GEGLU][int(rng.integers(0, 2))]
        axis = int(rng.integers(1, 4))
        flags = FORMATS[int(rng.integers(0, 4))] | (mx.SCALE_TILED if rng.random() < 0.3 else 0)
        bwd = bool(rng.random() < 0.5)
        out.append(pytest.param(i, M, N, act, axis, flags, bwd,
                                id=f"{i}-{M}x{N}-act{act}-a{axis}-f{flags}-{'bwd' if bwd else 'fwd'}"))
    return out


@pytest.mark.parametrize("i,M,N,act,axis,flags,bwd", gated_cases())
def test_gated_fuzz(i, M, N, act, axis, flags, bwd):
    x = W.normal(M, 2 * N, seed=9000 + i, sigma=1.5)
    if bwd:
        grad = W.normal(M, N, seed=9500 + i)
        g = mx.mx_quantize_dgated(to_dev(grad), to_dev(x), act, axis=axis | flags)
        torch.cuda.synchronize()
        o = O.mx_quantize_dgated(grad, x, act, axis=axis | flags)
    else:
        g = mx.mx_quantize_gated(to_dev(x), act, axis=axis | flags)
        torch.cuda.synchronize()
        o = O.mx_quantize_gated(x, act, axis=axis | flags)
    mx_outputs_equal(g, o, f"gated case {i}")


def nvfp4_cases(n=40, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, K = 16 * int(rng.integers(1, 35)), 16 * int(rng.integers(1, 65))
        axis = int(rng.integers(1, 4))
        two_d = bool(rng.random() < 0.5)
        out.append(pytest.param(i, M, K, axis, two_d, id=f"{i}-{M}x{K}-a{axis}-{'2d' if two_d else '1d'}"))
    return out


@pytest.mark.parametrize("i,M,K,axis,two_d", nvfp4_cases())
def test_nvfp4_fuzz(i, M, K, axis, two_d):
    x = W.student_t_rows(M, K, seed=9900 + i)
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16(xd)
    g = mx.nvfp4_quantize_transpose(xd, amax, axis=axis, two_d=two_d)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose(x, axis=axis, two_d=two_d)
    assert g["sg"].item() == o["sg"]
    mx_outputs_equal(g, o, f"nvfp4 case {i}")


def grouped_cases(n=24, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.integers(1, 9))
        rows = [16 * int(v) for v in rng.integers(0, 40, G)]
        if sum(rows) == 0:
            rows[0] = 16
        K = 8 * int(rng.integers(1, 131)) if i % 2 else 16 * int(rng.integers(1, 65))
        axis = int(rng.integers(1, 4))
        flags = FORMATS[int(rng.integers(0, 4))] | (mx.SCALE_TILED if rng.random() < 0.3 else 0)
        nv = i % 2 == 0
        out.append(pytest.param(i, rows, K, axis, flags, nv,
                                id=f"{i}-{'nvfp4' if nv else 'mxfp8'}-G{G}-K{K}-a{axis}-f{flags}"))
    return out


@pytest.mark.parametrize("i,rows,K,axis,flags,nv", grouped_cases())
def test_grouped_fuzz(i, rows, K, axis, flags, nv):
    x = W.normal(sum(rows), K, seed=9950 + i, sigma=3.0)
    xd = to_dev(x)
    if nv:
        amax = mx.mx_absmax_bf16_grouped(xd, rows)
        two_d = i % 4 == 0
        g = mx.nvfp4_quantize_transpose_grouped(xd, rows, amax, axis=axis, two_d=two_d)
        torch.cuda.synchronize()
        o = O.nvfp4_quantize_transpose_grouped(x, rows, axis=axis, two_d=two_d)
    else:
        g = mx.mx_quantize_grouped(xd, rows, axis=axis | flags)
        torch.cuda.synchronize()
        o = O.mx_quantize_grouped(x, rows, axis=axis | flags)
    mx_outputs_equal(g, o, f"grouped case {i}")


# --- any shape: sizes that need not be multiples of 16 or 8 ---------------------

def any_cases(n=80, seed=20261206):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, K = int(rng.integers(1, 600)), int(rng.integers(1, 1200))
        axis = int(rng.integers(1, 4))
        flags = FORMATS[int(rng.integers(0, 4))] | (mx.SCALE_TILED if rng.random() < 0.3 else 0)
        fusion = FUSIONS[int(rng.integers(0, 4))] | (mx.FUSE_DBIAS if rng.random() < 0.4 else 0)
        out.append(pytest.param(i, M, K, axis, flags, fusion,
                                id=f"any{i}-{M}x{K}-a{axis}-f{flags}-u{fusion}"))
    return out


@pytest.mark.parametrize("i,M,K,axis,flags,fusion", any_cases())
def test_any_shape_fuzz(i, M, K, axis, flags, fusion):
    test_mx_quantize_fuzz(1000 + i, M, K, axis, flags, fusion)


def any_nvfp4_cases(n=40, seed=20261207):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, K = int(rng.integers(1, 600)), int(rng.integers(1, 1200))
        axis = int(rng.integers(1, 4))
        two_d = bool(rng.random() < 0.5)
        out.append(pytest.param(i, M, K, axis, two_d,
                                id=f"any{i}-{M}x{K}-a{axis}-{'2d' if two_d else '1d'}"))
    return out


@pytest.mark.parametrize("i,M,K,axis,two_d", any_nvfp4_cases())
def test_any_shape_nvfp4_fuzz(i, M, K, axis, two_d):
    test_nvfp4_fuzz(1000 + i, M, K, axis, two_d)


def any_grouped_cases(n=20, seed=20261208):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.integers(1, 9))
        rows = [int(v) for v in rng.integers(0, 400, G)]
        if sum(rows) == 0:
            rows[0] = 1
        K = int(rng.integers(1, 1100))
        axis = int(rng.integers(1, 4))
        flags = FORMATS[int(rng.integers(0, 4))] | (mx.SCALE_TILED if rng.random() < 0.3 else 0)
        nv = i % 2 == 0
        out.append(pytest.param(i, rows, K, axis, flags, nv,
                                id=f"any{i}-{'nvfp4' if nv else 'mxfp8'}-G{G}-K{K}-a{axis}-f{flags}"))
    return out


@pytest.mark.parametrize("i,rows,K,axis,flags,nv", any_grouped_cases())
def test_any_shape_grouped_fuzz(i, rows, K, axis, flags, nv):
    test_grouped_fuzz(1000 + i, rows, K, axis, flags, nv)


# --- ragged row counts: row lengths multiples of 8 (MXFP8) or 16 (NVFP4), row
# counts (or a group's) not multiples of 16 -- the tiled kernels with
# transposed rows at any byte; sizes up to several sub-tiles per walk

def ragged_cases(n=80, seed=20261209):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 3000))
        M += 1 if M % 16 == 0 else 0
        K = 8 * int(rng.integers(1, 200))
        axis = int(rng.integers(1, 4))
        flags = FORMATS[int(rng.integers(0, 4))] | (mx.SCALE_TILED if rng.random() < 0.3 else 0)
        fusion = FUSIONS[int(rng.integers(0, 4))] | (mx.FUSE_DBIAS if rng.random() < 0.4 else 0)
        out.append(pytest.param(i, M, K, axis, flags, fusion,
                                id=f"rag{i}-{M}x{K}-a{axis}-f{flags}-u{fusion}"))
    return out


@pytest.mark.parametrize("i,M,K,axis,flags,fusion", ragged_cases())
def test_ragged_fuzz(i, M, K, axis, flags, fusion):
    test_mx_quantize_fuzz(2000 + i, M, K, axis, flags, fusion)


def ragged_nvfp4_cases(n=40, seed=20261210):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 3000))
        M += 1 if M % 16 == 0 else 0
        K = 16 * int(rng.integers(1, 100))
        axis = int(rng.integers(1, 4))
        two_d = bool(rng.random() < 0.5)
        out.append(pytest.param(i, M, K, axis, two_d,
                                id=f"rag{i}-{M}x{K}-a{axis}-{'2d' if two_d else '1d'}"))
    return out


@pytest.mark.parametrize("i,M,K,axis,two_d", ragged_nvfp4_cases())
def test_ragged_nvfp4_fuzz(i, M, K, axis, two_d):
    test_nvfp4_fuzz(2000 + i, M, K, axis, two_d)


def ragged_grouped_cases(n=30, seed=20261211):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.integers(1, 9))
        rows = [int(v) for v in rng.integers(0, 1500, G)]
        if all(r % 16 == 0 for r in rows):
            rows[0] += 1
        nv = i % 2 == 0
        K = (16 if nv else 8) * int(rng.integers(1, 80))
        axis = int(rng.integers(1, 4))
        flags = FORMATS[int(rng.integers(0, 4))] | (mx.SCALE_TILED if rng.random() < 0.3 else 0)
        out.append(pytest.param(i, rows, K, axis, flags, nv,
                                id=f"rag{i}-{'nvfp4' if nv else 'mxfp8'}-G{G}-K{K}-a{axis}-f{flags}"))
    return out


@pytest.mark.parametrize("i,rows,K,axis,flags,nv", ragged_grouped_cases())
def test_ragged_grouped_fuzz(i, rows, K, axis, flags, nv):
    test_grouped_fuzz(2000 + i, rows, K, axis, flags, nv)
