"""GPU parity of the backward casts: the dSiLU pre-op (with and without dbias)
and the gated backward dSwiGLU / dGeGLU, whose quantised tensor is
[d_gate | d_linear].  Fused bf16 values bit-exact over every bf16 input;
bytes and scales bit-exact against the oracle; dbias within 1e-3 relative
(plus the fp32 summation-error term for near-zero sums)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, assert_same, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu


def all_bf16_finite(width=256):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    pad = (-bits.size) % (32 * width)
    bits = np.concatenate([bits, np.zeros(pad, np.uint16)])
    return bits.reshape(-1, width)


def test_dsilu_values_every_bf16_input():
    x = all_bf16_finite()
    for g in (np.full_like(x, 0x3F80), W.normal(*x.shape, seed=50, sigma=3.0)):
        y = mx.mx_fused_values(to_dev(x), to_dev(g), op=mx.FUSE_DSILU)
        torch.cuda.synchronize()
        want = O.mx_quantize(x, grad=g, fusion=O.FUSE_DSILU, axis=1, want_y=True)["y"]
        assert_same(y, want, "dsilu values")


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_gated_backward_values_every_bf16_gate(act):
    gate = all_bf16_finite()
    rng_grads = (np.full_like(gate, 0x3F80), W.normal(*gate.shape, seed=51, sigma=2.0))
    lins = (np.full_like(gate, 0x3F80), W.normal(*gate.shape, seed=52, sigma=2.0))
    for dy in rng_grads:
        for lin in lins:
            x = np.concatenate([gate, lin], axis=1)
            y = mx.mx_fused_values(to_dev(x), to_dev(dy), op=mx.OP_DGATED | act)
            torch.cuda.synchronize()
            want = O.mx_quantize_dgated(dy, x, act, axis=1, want_y=True)["y"]
            assert_same(y, want, f"gated backward values act {act}")


@pytest.mark.parametrize("fusion", [mx.FUSE_DSILU, mx.FUSE_DSILU | mx.FUSE_DBIAS])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", [(64, 96), (256, 512), (416, 800)])
def test_dsilu_cast(M, K, axis, fusion):
    x, grad = W.make("f1_dsilu_dbias_8192", M, K)
    g = mx.mx_quantize(to_dev(x), to_dev(grad), axis=axis, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=axis, fusion=fusion, want_y=True)
    mx_outputs_equal(g, o, f"dsilu {fusion} axis {axis} {M}x{K}")
    if fusion & mx.FUSE_DBIAS:
        ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
        assert_dbias_close(g["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,N", [(32, 32), (96, 160), (128, 256), (256, 544)])
def test_gated_backward_cast(M, N, axis, act):
    """N = 160 and 544 put the gate/linear boundary inside a 256-column strip."""
    grad, x = W.make("f1_dgated_8192", M, N)
    g = mx.mx_quantize_dgated(to_dev(grad), to_dev(x), act, axis=axis)
    torch.cuda.synchronize()
    o = O.mx_quantize_dgated(grad, x, act, axis=axis)
    mx_outputs_equal(g, o, f"dgated {act} axis {axis} {M}x{N}")


def test_gated_backward_halves_in_place():
    """grad = 1 and linear = 1: the gate half holds act'(gate) and the linear
    half act(gate), each the single-input value quantised in place."""
    gate = W.normal(64, 256, seed=53)
    one = np.full_like(gate, 0x3F80)
    x = np.concatenate([gate, one], axis=1)
    g = mx.mx_quantize_dgated(to_dev(one), to_dev(x), mx.GATED_SWIGLU, axis=1)
    torch.cuda.synchronize()
    d_gate = O.mx_quantize(gate, grad=one, fusion=O.FUSE_DSILU, axis=1, want_y=True)["y"]
    d_lin = O.mx_quantize_gated(x, O.GATED_SWIGLU, axis=1, want_y=True)["y"]
    want = O.mx_quantize(np.concatenate([d_gate, d_lin], axis=1), axis=1)
    assert_same(g["q_row"], want["q_row"], "halves")
    assert_same(g["s_row"], want["s_row"], "halves scales")
