"""GPU parity of the fused casts: GELU / dGELU pre-ops with dbias, and the gated
SwiGLU / GeGLU cast.  Bytes and scales bit-exact against the oracle; the fused
bf16 values (mx_fused_values) bit-exact over every bf16 input; dbias within
1e-3 relative (plus the fp32 summation-error term for near-zero sums).
"""
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


def oracle_fused_values(x, grad, op):
    if op & mx.OP_GATED:
        return O.mx_quantize_gated(x, op & 0xF, axis=1, want_y=True)["y"]
    return O.mx_quantize(x, grad=grad, fusion=op, axis=1, want_y=True)["y"]


@pytest.mark.parametrize("op", [mx.FUSE_GELU, mx.FUSE_DGELU])
def test_fused_values_every_bf16_input(op):
    x = all_bf16_finite()
    grads = [np.full_like(x, 0x3F80)]                       # grad = 1: dGELU itself
    if op == mx.FUSE_DGELU:
        grads.append(W.normal(*x.shape, seed=40, sigma=3.0))
    for g in grads:
        y = mx.mx_fused_values(to_dev(x), to_dev(g), op=op)
        torch.cuda.synchronize()
        assert_same(y, oracle_fused_values(x, g, op), f"fused values op {op}")


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_gated_values_every_bf16_gate(act):
    gate = all_bf16_finite()
    for lin in (np.full_like(gate, 0x3F80), W.normal(*gate.shape, seed=41, sigma=2.0)):
        x = np.concatenate([gate, lin], axis=1)
        y = mx.mx_fused_values(to_dev(x), op=mx.OP_GATED | act)
        torch.cuda.synchronize()
        assert_same(y, oracle_fused_values(x, None, mx.OP_GATED | act), f"gated values act {act}")


@pytest.mark.parametrize("fusion", [mx.FUSE_GELU, mx.FUSE_DGELU, mx.FUSE_DBIAS,
                                    mx.FUSE_GELU | mx.FUSE_DBIAS, mx.FUSE_DGELU | mx.FUSE_DBIAS])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,K", [(64, 96), (256, 512), (416, 800)])
def test_fused_cast(M, K, axis, fusion):
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    g = mx.mx_quantize(to_dev(x), to_dev(grad), axis=axis, fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize(x, grad=grad, axis=axis, fusion=fusion, want_y=True)
    mx_outputs_equal(g, o, f"fused {fusion} axis {axis} {M}x{K}")
    if fusion & mx.FUSE_DBIAS:
        ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
        assert_dbias_close(g["dbias"], o["dbias"], ycols)


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("M,N", [(32, 32), (96, 288), (256, 512)])
def test_gated_cast(M, N, axis, act):
    x = W.make("c4_gated_8192", M, 2 * N)
    g = mx.mx_quantize_gated(to_dev(x), act, axis=axis)
    torch.cuda.synchronize()
    o = O.mx_quantize_gated(x, act, axis=axis)
    mx_outputs_equal(g, o, f"gated {act} axis {axis} {M}x{N}")


def test_gated_halves_not_swapped():
    """linear = 1 leaves act(gate): quantising it must equal the plain cast of
    the oracle's act(gate) values, and differ from casting act(linear)."""
    gate = W.normal(64, 256, seed=42)
    x = np.concatenate([gate, np.full_like(gate, 0x3F80)], axis=1)
    g = mx.mx_quantize_gated(to_dev(x), mx.GATED_SWIGLU, axis=1)
    torch.cuda.synchronize()
    y = np.vectorize(lambda a: O.gated(1, int(a), 0x3F80), otypes=[np.uint16])(gate)
    assert_same(g["q_row"], O.mx_quantize(y, axis=1)["q_row"], "gate first")


def test_dbias_deterministic():
    x, grad = W.make("c3_gelu_dbias_8192", 512, 768)
    xd, gd = to_dev(x), to_dev(grad)
    f = mx.FUSE_DGELU | mx.FUSE_DBIAS
    a = mx.mx_quantize(xd, gd, fusion=f)["dbias"].clone()
    b = mx.mx_quantize(xd, gd, fusion=f)["dbias"]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


SPECIALS = [0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80, 0x7F7F, 0xFF7F, 0x5F80, 0xDF80, 0x0001, 0x8000]


def values_match(got, want):
    """bf16 patterns equal, NaN payloads aside: NaN exactly where the oracle
    has NaN, every other pattern identical."""
    g = got.cpu().numpy().view(np.uint16) if isinstance(got, torch.Tensor) else got
    g_nan = (g & 0x7F80) == 0x7F80
    g_nan &= (g & 0x7F) != 0
    w_nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    assert np.array_equal(g_nan, w_nan), np.argwhere(g_nan != w_nan)[:4]
    assert np.array_equal(g[~g_nan], want[~w_nan]), "non-NaN values differ"


@pytest.mark.parametrize("op", [mx.FUSE_GELU, mx.OP_GATED | mx.GATED_SWIGLU,
                                mx.OP_GATED | mx.GATED_GEGLU])
def test_forward_activations_with_nan_and_inf(op):
    """NaN, +-Inf, the largest finite values and inputs whose cube overflows
    (+-2^64), planted among N(0, 1): the cast's bytes equal the oracle's, and
    the fused values are NaN exactly where the oracle's are and equal
    elsewhere."""
    gated = bool(op & mx.OP_GATED)
    M, K = 64, 512
    x = W.normal(M, K, seed=45)
    rng = np.random.default_rng(46)
    for b in SPECIALS:
        for _ in range(6):
            x[rng.integers(M), rng.integers(K)] = b
    xd = to_dev(x)
    if gated:
        g = mx.mx_quantize_gated(xd, op & 0xF)
        o = O.mx_quantize_gated(x, op & 0xF, want_y=True)
    else:
        g = mx.mx_quantize(xd, fusion=op)
        o = O.mx_quantize(x, fusion=op, want_y=True)
    torch.cuda.synchronize()
    mx_outputs_equal(g, o, f"op {op:#x} with NaN / Inf")
    y = mx.mx_fused_values(xd, op=op)
    torch.cuda.synchronize()
    values_match(y, o["y"])
