"""Argument checks of the Python binding (no GPU).

The binding marshals torch tensors into the C ABI, which takes raw pointers
and sizes it cannot check against the memory behind them.  So the binding
itself rejects, before any launch, every tensor whose size disagrees with
the sizes it passes: a gated input of odd width, grouped row counts that do
not sum to the input's rows, a grad of the wrong shape, preallocated outputs
of the wrong dtype, size or device, and host tensors.  These run on CPU
tensors: each malformed call must raise before the device check (which would
reject the CPU tensors anyway), and well-formed CPU calls must raise at the
device check, never reach the library.
"""
import pytest
import torch

import block_scaled_precision_bf16_amd as mx

I16, U8, F32 = torch.int16, torch.uint8, torch.float32


def z(*shape, dtype=I16):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("call", [
    lambda: mx.mx_quantize_gated(z(32, 35), mx.GATED_SWIGLU),
    lambda: mx.mx_quantize_dgated(z(32, 17), z(32, 35), mx.GATED_SWIGLU),
    lambda: mx.mx_fused_values(z(32, 35), op=mx.OP_GATED | mx.GATED_GEGLU),
    lambda: mx.mx_quantize_gated_grouped(z(32, 35), [16, 16], mx.GATED_SWIGLU),
], ids=["gated", "dgated", "fused_values", "gated_grouped"])
def test_odd_gated_width_raises(call):
    """17 gate columns and 17 linear ones would be read with the wrong row
    stride (an odd width is not [gate | linear])."""
    with pytest.raises(ValueError, match="even number of columns"):
        call()


@pytest.mark.parametrize("call", [
    lambda: mx.mx_quantize_grouped(z(64, 32), [16, 16]),
    lambda: mx.mx_quantize_grouped(z(32, 32), [16, 32]),
    lambda: mx.mx_quantize_gated_grouped(z(48, 64), [16, 16], mx.GATED_SWIGLU),
    lambda: mx.nvfp4_quantize_transpose_grouped(z(32, 32), [32, 16], z(2, dtype=F32)),
    lambda: mx.mx_absmax_bf16_grouped(z(32, 32), [48]),
    lambda: mx.mx_quantize_grouped(z(32, 32), [48, -16]),
], ids=["fewer", "more", "gated", "nvfp4", "absmax", "negative"])
def test_group_rows_must_sum_to_input_rows(call):
    with pytest.raises(ValueError, match="group row counts"):
        call()


@pytest.mark.parametrize("call", [
    lambda: mx.mx_quantize(z(32, 64), z(32, 32), fusion=mx.FUSE_DGELU),
    lambda: mx.mx_quantize(z(32, 64), z(16, 64), fusion=mx.FUSE_DSILU | mx.FUSE_DBIAS),
    lambda: mx.mx_quantize_dgated(z(32, 64), z(32, 64), mx.GATED_GEGLU),
    lambda: mx.mx_quantize_grouped(z(32, 64), [32], grad=z(32, 32), fusion=mx.FUSE_DGELU),
    lambda: mx.mx_quantize_gated_grouped(z(32, 64), [32], mx.GATED_SWIGLU, grad=z(32, 64)),
    lambda: mx.mx_fused_values(z(32, 64), z(32, 16), op=mx.FUSE_DGELU),
], ids=["dgelu", "dsilu", "dgated", "grouped", "dgated_grouped", "fused_values"])
def test_grad_shape_is_checked(call):
    with pytest.raises(ValueError, match="grad must have shape"):
        call()


@pytest.mark.parametrize("out", [
    {"q_row": z(32, 64, dtype=F32)},                       # wrong dtype
    {"q_row": z(32, 63, dtype=U8)},                        # too few elements
    {"s_col": z(64, 2, dtype=U8)},                         # [K][M/32] is 64 x 1
    {"q_col": z(64, 64, dtype=U8)[:, :32]},                # not contiguous
])
def test_preallocated_outputs_are_checked(out):
    with pytest.raises(ValueError, match="out\\["):
        mx.mx_quantize(z(32, 64), out=out)


def test_nvfp4_amax_is_checked():
    with pytest.raises(ValueError, match="amax"):
        mx.nvfp4_quantize_transpose(z(32, 32), amax=z(2, dtype=F32))
    with pytest.raises(ValueError, match="amax"):
        mx.nvfp4_quantize_transpose_grouped(z(32, 32), [16, 16], z(1, dtype=F32))


def test_non_2d_input_is_rejected():
    with pytest.raises(ValueError, match="2-D"):
        mx.mx_quantize(z(4, 8, 32))


@pytest.mark.parametrize("call", [
    lambda: mx.mx_quantize(z(32, 64)),
    lambda: mx.mx_quantize(z(32, 64), fusion=mx.FUSE_GELU | mx.FUSE_DBIAS),
    lambda: mx.mx_quantize_gated(z(32, 64), mx.GATED_SWIGLU),
    lambda: mx.mx_quantize_grouped(z(32, 32), [16, 16]),
    lambda: mx.nvfp4_quantize_transpose(z(32, 32), amax=z(1, dtype=F32)),
    lambda: mx.mx_absmax_bf16(z(32, 32)),
], ids=["mx", "dbias", "gated", "grouped", "nvfp4", "absmax"])
def test_host_tensors_never_reach_the_library(call):
    """A host pointer handed to a kernel would fault the GPU: a well-formed
    call on CPU tensors stops at the device check."""
    with pytest.raises(ValueError, match="ROCm"):
        call()
