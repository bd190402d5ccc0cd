"""GPU parity of the grouped (per-expert) MXFP8 cast against the oracle, byte
for byte: groups of any multiple of 16 rows (empty ones included) stacked
along M, cast in one launch, outputs concatenated group after group; dbias
per group within the dbias tolerance.  Covers walks that end at group
boundaries, groups smaller than a sub-tile, the format and layout flags and
an MoE-like set of eight experts."""
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_dbias_close, mx_outputs_equal, to_dev

pytestmark = pytest.mark.gpu

GROUPS = [([128, 0, 256, 128], 256), ([48, 0, 80, 16], 136), ([16] * 5, 40),
          ([2048, 16, 0, 1520], 1056), ([32], 32)]


@pytest.fixture(scope="module", autouse=True)
def threads():
    O.set_threads(min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("flags", [0, mx.SCALE_TILED, mx.ELEM_E5M2 | mx.SCALE_ROUND_UP],
                         ids=["plain", "tiled", "e5m2-up"])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("rows,K", GROUPS)
def test_grouped_plain(rows, K, axis, flags):
    M = sum(rows)
    x = W.loguniform_rows(M, K, seed=6000 + M + K)
    g = mx.mx_quantize_grouped(to_dev(x), rows, axis=axis | flags)
    torch.cuda.synchronize()
    o = O.mx_quantize_grouped(x, rows, axis=axis | flags)
    mx_outputs_equal(g, o, f"grouped {rows} K={K} axis {axis} flags {flags}")


@pytest.mark.parametrize("fusion", [mx.FUSE_DBIAS, mx.FUSE_GELU | mx.FUSE_DBIAS,
                                    mx.FUSE_DSILU | mx.FUSE_DBIAS, mx.FUSE_DGELU])
def test_grouped_fused(fusion):
    rows, K = [256, 0, 48, 400], 520
    M = sum(rows)
    x, grad = W.make("c3_gelu_dbias_8192", M, K)
    g = mx.mx_quantize_grouped(to_dev(x), rows, grad=to_dev(grad), fusion=fusion)
    torch.cuda.synchronize()
    o = O.mx_quantize_grouped(x, rows, grad=grad, fusion=fusion)
    mx_outputs_equal(g, o, f"grouped fusion {fusion}")
    if fusion & mx.FUSE_DBIAS:
        r0 = 0
        for gi, m in enumerate(rows):
            if m == 0:
                assert torch.all(g["dbias"][gi] == 0)
                continue
            y = O.mx_quantize(np.ascontiguousarray(x[r0:r0 + m]),
                              grad=np.ascontiguousarray(grad[r0:r0 + m]), fusion=fusion,
                              want_y=True)["y"]
            ycols = np.abs(W.bf16_to_f32(y).astype(np.float64)).sum(axis=0)
            assert_dbias_close(g["dbias"][gi], o["dbias"][gi], ycols, f"dbias group {gi}")
            r0 += m


def test_grouped_moe_eight_experts():
    rows = [1024, 512, 0, 2048, 16, 1520, 768, 256]
    K = 2048
    x = W.normal(sum(rows), K, seed=67, sigma=2.0)
    g = mx.mx_quantize_grouped(to_dev(x), rows, axis=3)
    torch.cuda.synchronize()
    mx_outputs_equal(g, O.mx_quantize_grouped(x, rows, axis=3), "moe experts")


def test_grouped_equals_per_group_calls_on_gpu():
    rows, K = [128, 0, 96, 32], 264
    x = W.loguniform_rows(sum(rows), K, seed=68)
    xd = to_dev(x)
    g = mx.mx_quantize_grouped(xd, rows, axis=3)
    r0, qc, sc = 0, [], []
    for m in rows:
        if m:
            p = mx.mx_quantize(xd[r0:r0 + m].contiguous(), axis=3)
            qc.append(p["q_col"].reshape(-1))
            sc.append(p["s_col"].reshape(-1))
        r0 += m
    torch.cuda.synchronize()
    assert torch.equal(g["q_col"], torch.cat(qc)) and torch.equal(g["s_col"], torch.cat(sc))


# --- grouped NVFP4 -------------------------------------------------------------

NV_GROUPS = [([128, 0, 256, 128], 256), ([48, 0, 80, 16], 144), ([16] * 5, 64),
             ([2048, 16, 0, 1520], 1056)]


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
@pytest.mark.parametrize("axis", [1, 2, 3])
@pytest.mark.parametrize("rows,K", NV_GROUPS)
def test_grouped_nvfp4(rows, K, axis, two_d):
    M = sum(rows)
    x = W.student_t_rows(M, K, seed=7000 + M + K)
    xd = to_dev(x)
    amax = mx.mx_absmax_bf16_grouped(xd, rows)
    g = mx.nvfp4_quantize_transpose_grouped(xd, rows, amax, axis=axis, two_d=two_d)
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose_grouped(x, rows, axis=axis, two_d=two_d)
    mx_outputs_equal(g, o, f"grouped nvfp4 {rows} K={K} axis {axis} 2d={two_d}")
    assert np.array_equal(g["sg"].cpu().numpy(), o["sg"])


def test_grouped_absmax_matches_numpy():
    rows, K = [256, 0, 48, 1024, 16], 512
    x = W.student_t_rows(sum(rows), K, seed=74)
    a = mx.mx_absmax_bf16_grouped(to_dev(x), rows).cpu().numpy()
    xf = np.abs(W.bf16_to_f32(x))
    r0 = 0
    for gi, m in enumerate(rows):
        want = xf[r0:r0 + m].max() if m else 0.0
        assert a[gi] == np.float32(want), gi
        r0 += m


def test_grouped_nvfp4_moe_eight_experts():
    rows = [1024, 512, 0, 2048, 16, 1520, 768, 256]
    K = 2048
    x = W.student_t_rows(sum(rows), K, seed=75)
    xd = to_dev(x)
    g = mx.nvfp4_quantize_transpose_grouped(xd, rows, mx.mx_absmax_bf16_grouped(xd, rows))
    torch.cuda.synchronize()
    o = O.nvfp4_quantize_transpose_grouped(x, rows)
    mx_outputs_equal(g, o, "nvfp4 moe experts")


# --- grouped gated casts --------------------------------------------------------

@pytest.mark.parametrize("flags", [0, mx.SCALE_TILED | mx.ELEM_E5M2], ids=["plain", "tiled-e5m2"])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
@pytest.mark.parametrize("rows,N", [([128, 0, 256, 48], 160), ([16] * 5, 40), ([512, 16, 0, 336], 264)])
def test_grouped_gated(rows, N, act, backward, flags):
    M = sum(rows)
    x = W.normal(M, 2 * N, seed=8000 + M + N)
    grad = W.normal(M, N, seed=8001 + M + N) if backward else None
    g = mx.mx_quantize_gated_grouped(to_dev(x), rows, act, grad=to_dev(grad) if backward else None,
                                     axis=3 | flags)
    torch.cuda.synchronize()
    o = O.mx_quantize_gated_grouped(x, rows, act, axis=3 | flags, grad=grad)
    mx_outputs_equal(g, o, f"grouped gated {rows} N={N} act {act} bwd {backward} flags {flags}")
