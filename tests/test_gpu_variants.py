"""GPU parity of the MXFP8 format variants (flags beside the axis bits): E5M2
elements, the round-up E8M0 rule, and both, against the oracle byte for byte.

An exhaustive tensor drives every (bf16 element, scale byte) pair either rule
can produce through both directions; random shapes cover several tiles and
ragged tails for every kernel family (plain, pre-ops with dbias, gated,
gated backward); the 16384^2 dim0 + dim1 workload runs at full size.
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

MODES = [mx.ELEM_E5M2, mx.SCALE_ROUND_UP, mx.ELEM_E5M2 | mx.SCALE_ROUND_UP]
NAMES = {mx.ELEM_E5M2: "e5m2", mx.SCALE_ROUND_UP: "e4m3-up",
         mx.ELEM_E5M2 | mx.SCALE_ROUND_UP: "e5m2-up"}


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


def every_pair_tensor(width=2048):
    """Blocks of [setter, 31 elements]: for each exponent field E the setter is
    the bf16 magnitude E<<7 | m with m = 0x60 (the largest amax of its binade
    that the round-up rule keeps at the floor byte) or m = 0x7F, and the
    elements run over every finite bf16 of magnitude <= the setter, both
    signs.  Under either rule and either element format this reaches every
    (element, byte) pair a block can produce."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = bits[(bits & 0x7F80) != 0x7F80]
    mag = fin & 0x7FFF
    blocks = []
    for E in range(255):
        for m in (0x60, 0x7F):
            s = (E << 7) | m
            vals = fin[mag <= s]
            pad = (-len(vals)) % 31
            vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
            setter = np.full((vals.shape[0], 1), s, np.uint16)
            blocks.append(np.concatenate([setter, vals], axis=1))
    blk = np.concatenate(blocks)
    per_row = width // 32
    pad = (-blk.shape[0]) % per_row
    blk = np.concatenate([blk, np.zeros((pad, 32), np.uint16)])
    x = blk.reshape(-1, width)
    rows = (-x.shape[0]) % 32
    return np.concatenate([x, np.zeros((rows, width), np.uint16)])


@pytest.fixture(scope="module")
def pairs():
    return every_pair_tensor()


@pytest.mark.parametrize("mode", MODES, ids=lambda m: NAMES[m])
def test_every_element_scale_pair_rowwise(pairs, mode):
    g = mx.mx_quantize(to_dev(pairs), axis=mx.ROWWISE | mode)
    torch.cuda.synchronize()
    o = O.mx_quantize(pairs, axis=mx.ROWWISE | mode)
    mx_outputs_equal(g, o, f"every pair rows {NAMES[mode]}")


@pytest.mark.parametrize("mode", MODES, ids=lambda m: NAMES[m])
def test_every_element_scale_pair_colwise(pairs, mode):
    xt = np.ascontiguousarray(pairs.T)
    g = mx.mx_quantize(to_dev(xt), axis=mx.COLWISE | mode)
    torch.cuda.synchronize()
    o = O.mx_quantize(xt, axis=mx.COLWISE | mode)
    mx_outputs_equal(g, o, f"every pair cols {NAMES[mode]}")


@pytest.mark.parametrize("mode", MODES, ids=lambda m: NAMES[m])
def test_special_and_nonfinite_blocks(mode):
    x = W.special_256x512()
    x[40, 300] = 0x7FC0
    x[200, 7] = 0xFF80
    g = mx.mx_quantize(to_dev(x), axis=3 | mode)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, axis=3 | mode)
    mx_outputs_equal(g, o, f"special {NAMES[mode]}")


@pytest.mark.parametrize("mode", MODES, ids=lambda m: NAMES[m])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", [(32, 32), (96, 288), (160, 800), (416, 1056)])
def test_plain_shapes(M, K, axis, mode):
    x = W.loguniform_rows(M, K, seed=2000 + M + K)
    g = mx.mx_quantize(to_dev(x), axis=axis | mode)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, axis=axis | mode)
    mx_outputs_equal(g, o, f"{M}x{K} axis {axis} {NAMES[mode]}")


@pytest.mark.parametrize("mode", MODES, ids=lambda m: NAMES[m])
@pytest.mark.parametrize("fusion", [mx.FUSE_GELU | mx.FUSE_DBIAS, mx.FUSE_DGELU,
                                    mx.FUSE_DSILU | mx.FUSE_DBIAS, mx.FUSE_DBIAS])
def test_fused_variants(fusion, mode):
    M, K = 288, 544
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    g = mx.mx_quantize(to_dev(x), to_dev(grad), axis=3 | mode, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=3 | mode, fusion=fusion, want_y=True)
    mx_outputs_equal(g, o, f"fusion {fusion} {NAMES[mode]}")
    if fusion & mx.FUSE_DBIAS:
        ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
        assert_dbias_close(g["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("mode", MODES, ids=lambda m: NAMES[m])
@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_gated_variants(act, mode):
    x = W.make("c4_gated_8192", 160, 576)
    g = mx.mx_quantize_gated(to_dev(x), act, axis=3 | mode)
    torch.cuda.synchronize()
    o = O.mx_quantize_gated(x, act, axis=3 | mode)
    mx_outputs_equal(g, o, f"gated {act} {NAMES[mode]}")
    grad, xb = W.make("f1_dgated_8192", 96, 160)
    g = mx.mx_quantize_dgated(to_dev(grad), to_dev(xb), act, axis=3 | mode)
    torch.cuda.synchronize()
    o = O.mx_quantize_dgated(grad, xb, act, axis=3 | mode)
    mx_outputs_equal(g, o, f"dgated {act} {NAMES[mode]}")


@pytest.mark.parametrize("mode", MODES, ids=lambda m: NAMES[m])
def test_dim0_dim1_16384_variants(mode):
    x = W.make("c2_dim1_16384")
    g = mx.mx_quantize(to_dev(x), axis=3 | mode)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, axis=3 | mode)
    mx_outputs_equal(g, o, f"16384 dim0+dim1 {NAMES[mode]}")
