"""Casts at the largest row length the ABI accepts, with 128 rows, so that the
last row of a sub-tile sits 127 rows (about 2^31 bytes) past the first and the
kernels' 32-bit in-tile offsets run up to the largest buffer descriptor:

  mx_quantize        x [128][2^23]
  mx_quantize_gated  x [128][2^23] = [gate | linear], N = 2^22
  mx_quantize_dgated grad [128][2^22], x [128][2^23] (and the grouped variant)
  nvfp4              x [128][2^23]

The tensors are zero except for seeded N(0, 1) columns at both ends of each
half (for the gated inputs: gate, linear and grad at the same columns), so
the oracle runs on those columns alone: every output block there comes from
those columns only (32-aligned column sets; blocks along M span the 128 rows).
Everything else must come out as zero codes and zero scales.  An access that
fell outside its descriptor would read zeros there and change the codes of
the planted columns (the last row is the one at risk), or drop stores.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_bf16_amd as mx
import oracle as O
import workloads as W
from gpu_util import assert_same, to_host

pytestmark = pytest.mark.gpu

M = 128
WIDE = 1 << 23          # full row length in elements
W_EDGE = 64             # planted columns at each end of a (half) row


def edge_cols(n):
    return np.r_[0:W_EDGE, n - W_EDGE:n]


def plant(t_dev, cols, vals):
    """Write host bf16 bits vals[M][len(cols)] into device t_dev[:, cols]."""
    c = torch.from_numpy(cols.astype(np.int64)).cuda()
    t_dev.index_copy_(1, c, torch.from_numpy(np.ascontiguousarray(vals).view(np.int16)).cuda())


def zero_outside(q_dev, cols, dim, what):
    """Every byte of q_dev outside the given columns (dim 1) / rows (dim 0) is 0."""
    t = q_dev.clone()
    idx = torch.from_numpy(cols.astype(np.int64)).cuda()
    t.index_fill_(dim, idx, 0)
    nz = int(torch.count_nonzero(t).item())
    assert nz == 0, f"{what}: {nz} nonzero bytes outside the planted region"


def blocks_of(cols, size):
    """Scale-block indices (block `size`) covering the 32-aligned column set."""
    return np.unique(cols // size)


def check_mx(g, o, cols, width, what):
    """GPU outputs of a [M][width] quantised tensor vs the oracle's outputs of
    its planted columns (in the order of cols)."""
    q_row = g["q_row"]
    assert_same(to_host(q_row[:, torch.from_numpy(cols).cuda()]), o["q_row"], f"{what} q_row")
    zero_outside(q_row, cols, 1, f"{what} q_row")
    b = blocks_of(cols, 32)
    s_row = g["s_row"]
    assert_same(to_host(s_row[:, torch.from_numpy(b).cuda()]), o["s_row"], f"{what} s_row")
    zero_outside(s_row, b, 1, f"{what} s_row")
    q_col = g["q_col"]
    assert_same(to_host(q_col[torch.from_numpy(cols).cuda()]), o["q_col"], f"{what} q_col")
    zero_outside(q_col, cols, 0, f"{what} q_col")
    s_col = g["s_col"]
    assert_same(to_host(s_col[torch.from_numpy(cols).cuda()]), o["s_col"], f"{what} s_col")
    zero_outside(s_col, cols, 0, f"{what} s_col")
    assert q_row.shape == (M, width)


@pytest.fixture(autouse=True)
def free_memory():
    yield
    torch.cuda.empty_cache()


def test_mx_quantize_longest_rows():
    K = WIDE
    cols = edge_cols(K)
    vals = W.normal(M, cols.size, seed=101)
    x = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    plant(x, cols, vals)
    print(f"[limits] mx_quantize {M}x{K}", flush=True)
    g = mx.mx_quantize(x)
    torch.cuda.synchronize()
    del x
    check_mx(g, O.mx_quantize(vals), cols, K, "mx_quantize 128 x 2^23")


def gated_inputs(N, seed):
    """x [M][2N] zero but for gate / linear columns at both ends of each half,
    grad [M][N] zero but for the same columns; returns device tensors and the
    oracle's small [gate | linear] and grad."""
    cols = edge_cols(N)
    gate = W.normal(M, cols.size, seed=seed)
    lin = W.normal(M, cols.size, seed=seed + 1)
    grad = W.normal(M, cols.size, seed=seed + 2)
    x = torch.zeros((M, 2 * N), dtype=torch.int16, device="cuda")
    plant(x, cols, gate)
    plant(x, N + cols, lin)
    gd = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    plant(gd, cols, grad)
    return x, gd, cols, np.concatenate([gate, lin], axis=1), grad


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_gated_longest_rows(act):
    N = WIDE // 2
    x, gd, cols, xs, _ = gated_inputs(N, 110)
    del gd
    print(f"[limits] mx_quantize_gated {M}x2x{N} act {act}", flush=True)
    g = mx.mx_quantize_gated(x, act)
    torch.cuda.synchronize()
    del x
    check_mx(g, O.mx_quantize_gated(xs, act), cols, N, f"gated act {act}")


@pytest.mark.parametrize("act", [mx.GATED_SWIGLU, mx.GATED_GEGLU])
def test_dgated_longest_rows(act):
    """The gated backward reads the linear half at 2N bytes past the gate; at
    2N = 2^23 the last row's linear loads end 16 bytes short of 2^31."""
    N = WIDE // 2
    x, gd, cols, xs, grads = gated_inputs(N, 120)
    print(f"[limits] mx_quantize_dgated {M}x2x{N} act {act}", flush=True)
    g = mx.mx_quantize_dgated(gd, x, act)
    torch.cuda.synchronize()
    o = O.mx_quantize_dgated(grads, xs, act)
    check_mx(g, o, np.r_[cols, N + cols], 2 * N, f"dgated act {act}")
    # the grouped cast of the same rows as two 64-row groups: each group's
    # outputs are the plain cast's (its rows, and its 64-row column slices)
    print(f"[limits] mx_quantize_dgated_grouped {M}x2x{N} act {act}", flush=True)
    gg = mx.mx_quantize_gated_grouped(x, [64, 64], act, grad=gd)
    torch.cuda.synchronize()
    assert torch.equal(gg["q_row"], g["q_row"])
    assert torch.equal(gg["s_row"].view(M, -1), g["s_row"])
    qc = gg["q_col"].view(2, 2 * N, 64)
    sc = gg["s_col"].view(2, 2 * N, 2)
    for grp in range(2):
        assert torch.equal(qc[grp], g["q_col"][:, 64 * grp:64 * grp + 64]), f"group {grp} q_col"
        assert torch.equal(sc[grp], g["s_col"][:, 2 * grp:2 * grp + 2]), f"group {grp} s_col"


def test_nvfp4_longest_rows():
    K = WIDE
    cols = edge_cols(K)
    vals = W.student_t_rows(M, cols.size, seed=130)
    x = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    plant(x, cols, vals)
    print(f"[limits] nvfp4 {M}x{K}", flush=True)
    amax = mx.mx_absmax_bf16(x)
    g = mx.nvfp4_quantize_transpose(x, amax)
    torch.cuda.synchronize()
    del x
    o = O.nvfp4_quantize_transpose(vals)
    assert g["sg"].item() == o["sg"]
    bcols = np.r_[0:W_EDGE // 2, K // 2 - W_EDGE // 2:K // 2]     # packed bytes
    assert_same(to_host(g["q_row"][:, torch.from_numpy(bcols).cuda()]), o["q_row"], "nvfp4 q_row")
    zero_outside(g["q_row"], bcols, 1, "nvfp4 q_row")
    b = np.r_[0:W_EDGE // 16, K // 16 - W_EDGE // 16:K // 16]
    assert_same(to_host(g["s_row"][:, torch.from_numpy(b).cuda()]), o["s_row"], "nvfp4 s_row")
    zero_outside(g["s_row"], b, 1, "nvfp4 s_row")
    assert_same(to_host(g["q_col"][torch.from_numpy(cols).cuda()]), o["q_col"], "nvfp4 q_col")
    zero_outside(g["q_col"], cols, 0, "nvfp4 q_col")
    assert_same(to_host(g["s_col"][torch.from_numpy(cols).cuda()]), o["s_col"], "nvfp4 s_col")
    zero_outside(g["s_col"], cols, 0, "nvfp4 s_col")
