"""mx_quantize_noalloc (the allocation-free cast) against mx_quantize, through
the C ABI: on two calls in a row, the second with a smaller tensor, every
output must be bit-identical to what mx_quantize writes with a workspace of
its own (the same kernels and summation order), for the dbias casts that use
the static scratch and for a cast that does not.  A dbias request larger than
the scratch is refused with MX_ERR_WORKSPACE and writes nothing.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, assert_same, to_dev

pytestmark = pytest.mark.gpu


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def outputs(M, K, dev="cuda"):
    return dict(q_row=torch.full((M, K), 0x5A, dtype=torch.uint8, device=dev),
                s_row=torch.full((M, -(-K // 32)), 0x5A, dtype=torch.uint8, device=dev),
                q_col=torch.full((K, M), 0x5A, dtype=torch.uint8, device=dev),
                s_col=torch.full((K, -(-M // 32)), 0x5A, dtype=torch.uint8, device=dev),
                dbias=torch.full((K,), float("nan"), dtype=torch.float32, device=dev))


def call_noalloc(x, g, fusion, o):
    M, K = x.shape
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return mx.lib().mx_quantize_noalloc(ptr(x), ptr(g), M, K, 3, fusion, ptr(o["q_row"]),
                                        ptr(o["s_row"]), ptr(o["q_col"]), ptr(o["s_col"]),
                                        ptr(o["dbias"]) if fusion & mx.FUSE_DBIAS else None, s)


def call_with_workspace(x, g, fusion, o):
    M, K = x.shape
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n = mx.mx_quantize_workspace_size(M, K, 3, fusion)
    ws = torch.empty(max(16, n), dtype=torch.uint8, device="cuda")
    st = mx.lib().mx_quantize(ptr(x), ptr(g), M, K, 3, fusion, ptr(o["q_row"]), ptr(o["s_row"]),
                              ptr(o["q_col"]), ptr(o["s_col"]),
                              ptr(o["dbias"]) if fusion & mx.FUSE_DBIAS else None,
                              ptr(ws), n, s)
    return st, ws


@pytest.mark.parametrize("fusion", [mx.FUSE_DGELU | mx.FUSE_DBIAS, mx.FUSE_GELU | mx.FUSE_DBIAS,
                                    mx.FUSE_DSILU | mx.FUSE_DBIAS, mx.FUSE_DBIAS, mx.FUSE_NONE],
                         ids=["dgelu_dbias", "gelu_dbias", "dsilu_dbias", "dbias", "plain"])
def test_noalloc_matches_mx_quantize(fusion):
    # a large call, then a smaller one: the scratch keeps the first call's
    # partials, which the second must not read
    for M, K, seed in ((2048, 4096, 201), (256, 1288, 202)):
        xh = W.normal(M, K, seed=seed, sigma=1.5)
        gh = W.normal(M, K, seed=seed + 50)
        x, g = to_dev(xh), to_dev(gh)
        a, b = outputs(M, K), outputs(M, K)
        assert call_noalloc(x, g, fusion, a) == mx.MX_OK
        st, ws = call_with_workspace(x, g, fusion, b)
        assert st == mx.MX_OK
        torch.cuda.synchronize()
        for k in ("q_row", "s_row", "q_col", "s_col"):
            assert torch.equal(a[k], b[k]), f"{M}x{K} {k}"
        if fusion & mx.FUSE_DBIAS:
            assert torch.equal(a["dbias"].view(torch.int32), b["dbias"].view(torch.int32)), \
                f"{M}x{K} dbias differs from mx_quantize's"
            o = O.mx_quantize(xh, grad=gh, fusion=fusion, want_y=True)
            assert_same(a["q_row"], o["q_row"], f"{M}x{K} q_row vs oracle")
            ycols = np.abs(W.bf16_to_f32(o["y"]).astype(np.float64)).sum(axis=0)
            assert_dbias_close(a["dbias"], o["dbias"], ycols)


def test_noalloc_refuses_more_than_its_scratch():
    M, K = 128, 1 << 21          # one walk of 2^21 partials: 8 MiB > 4 MiB
    x = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    o = outputs(M, K)
    assert call_noalloc(x, None, mx.FUSE_GELU | mx.FUSE_DBIAS, o) == mx.MX_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o["q_row"] == 0x5A).all()) and bool(torch.isnan(o["dbias"]).all())


def test_binding_noalloc_needs_preallocated_outputs():
    x = to_dev(W.normal(64, 256, seed=203))
    with pytest.raises(ValueError, match="allocates nothing"):
        mx.mx_quantize_noalloc(x, out={}, fusion=mx.FUSE_DBIAS)
    o = outputs(64, 256)
    r = mx.mx_quantize_noalloc(x, out=o, fusion=mx.FUSE_GELU | mx.FUSE_DBIAS)
    w = mx.mx_quantize(x, fusion=mx.FUSE_GELU | mx.FUSE_DBIAS)
    torch.cuda.synchronize()
    for k in ("q_row", "s_row", "q_col", "s_col", "dbias"):
        assert torch.equal(r[k], w[k]), k
