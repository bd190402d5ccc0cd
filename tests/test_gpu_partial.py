"""GPU parity of partial blocks: M a multiple of 16 and K of 8 but not of 32,
so the last block of a row or column holds fewer than 32 elements.  Compared
with the oracle byte for byte (compact and tiled scales), for the plain cast,
the pre-ops with dbias, the gated casts and their backward, and one large
tensor whose edges are partial in both directions."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(16, 8), (48, 40), (80, 200), (112, 264), (400, 1048), (16, 2056), (2064, 24)]


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("layout", [0, mx.SCALE_TILED], ids=["compact", "tiled"])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", SHAPES)
def test_plain_partial(M, K, axis, layout):
    x = W.loguniform_rows(M, K, seed=5000 + M + K)
    g = mx.mx_quantize(to_dev(x), axis=axis | layout)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize(x, axis=axis | layout), f"{M}x{K} axis {axis} {layout}")


@pytest.mark.parametrize("fusion", [mx.FUSE_GELU | mx.FUSE_DBIAS, mx.FUSE_DGELU | mx.FUSE_DBIAS,
                                    mx.FUSE_DSILU, mx.FUSE_DBIAS])
def test_fused_partial(fusion):
    M, K = 400, 1048
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    mode = mx.ELEM_E5M2 if fusion & 1 else 0
    g = mx.mx_quantize(to_dev(x), to_dev(grad), axis=3 | mode, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=3 | mode, fusion=fusion, want_y=True)
    mx_outputs_equal(g, o, f"partial fusion {fusion}")
    if fusion & mx.FUSE_DBIAS:
        ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
        assert_dbias_close(g["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
@pytest.mark.parametrize("M,N", [(48, 40), (112, 72), (400, 264)])
def test_gated_partial(M, N, act):
    x = W.make("c4_gated_8192", M, 2 * N)
    g = mx.mx_quantize_gated(to_dev(x), act, axis=3)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize_gated(x, act, axis=3), f"gated {M}x{N}")
    grad, xb = W.make("f1_dgated_8192", M, N)
    g = mx.mx_quantize_dgated(to_dev(grad), to_dev(xb), act, axis=3 | mx.SCALE_TILED)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize_dgated(grad, xb, act, axis=3 | mx.SCALE_TILED),
                     f"dgated {M}x{N}")


def test_fused_values_partial():
    x, grad = W.make("c3_gelu_dbias_8192", 48, 40)
    y = mx.mx_fused_values(to_dev(x), to_dev(grad), op=mx.FUSE_DGELU)
    torch.cuda.synchronize()
    want = O.mx_quantize(x, grad=grad, fusion=O.FUSE_DGELU, axis=1, want_y=True)["y"]
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("layout", [0, mx.SCALE_TILED], ids=["compact", "tiled"])
def test_large_partial_both_edges(layout):
    x = W.loguniform_rows(8208, 8200, seed=51)
    g = mx.mx_quantize(to_dev(x), axis=3 | layout)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize(x, axis=3 | layout), f"8208x8200 {layout}")


@pytest.mark.parametrize("layout", [0, mx.SCALE_TILED], ids=["compact", "tiled"])
def test_partial_stores_stay_inside_outputs(layout):
    """Outputs placed between guard bands of 0x5A: a partial edge must not
    spill a byte outside its tensor (or into the padding of the next line)."""
    M, K = 400, 1048
    x = W.loguniform_rows(M, K, seed=52)
    guard = 4096
    sizes = dict(q_row=M * K, s_row=mx.mx_scale_size(M, K, 3 | layout), q_col=M * K,
                 s_col=mx.mx_scale_size(K, M, 3 | layout))
    bufs = {n: torch.full((s + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
            for n, s in sizes.items()}
    outs = {n: b[guard:guard + sizes[n]] for n, b in bufs.items()}
    outs["q_row"] = outs["q_row"].view(M, K)
    outs["q_col"] = outs["q_col"].view(K, M)
    if not layout:
        outs["s_row"] = outs["s_row"].view(M, -(-K // 32))
        outs["s_col"] = outs["s_col"].view(K, -(-M // 32))
    mx.mx_quantize(to_dev(x), axis=3 | layout, out=outs)
    torch.cuda.synchronize()
    for n, b in bufs.items():
        assert torch.all(b[:guard] == 0x5A) and torch.all(b[-guard:] == 0x5A), n
    mx_outputs_equal(outs, O.mx_quantize(x, axis=3 | layout), f"guarded {layout}")
