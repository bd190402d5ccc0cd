"""Pins for the oracle's grouped (per-expert) MXFP8 cast: groups stacked
along rows, each cast as a tensor of its own, outputs concatenated.

  * one group is the plain cast;
  * row-wise outputs equal those of the whole stacked tensor (rows are
    independent), for any group sizes;
  * with group boundaries on multiples of 32 rows no column block crosses a
    boundary, so each group's transposed output is a column slice of the
    stacked tensor's;
  * dbias per group equals numpy's float64 column sums of the group's rows;
  * empty groups take no space and have zero dbias; tiled scales per group.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W


def split(flat, sizes):
    out, o = [], 0
    for n in sizes:
        out.append(flat[o:o + n])
        o += n
    assert o == flat.size
    return out


def test_one_group_is_the_plain_cast():
    x = W.loguniform_rows(96, 200, seed=61)
    g = O.mx_quantize_grouped(x, [96])
    p = O.mx_quantize(x)
    assert np.array_equal(g["q_row"], p["q_row"]) and np.array_equal(g["s_row"], p["s_row"].ravel())
    assert np.array_equal(g["q_col"], p["q_col"].ravel()) and np.array_equal(g["s_col"], p["s_col"].ravel())


@pytest.mark.parametrize("rows", [[32, 64, 16], [48, 0, 80, 16], [16, 16, 16, 16, 16]])
def test_rowwise_equals_stacked(rows):
    M, K = sum(rows), 136
    x = W.loguniform_rows(M, K, seed=62)
    g = O.mx_quantize_grouped(x, rows, axis=O.ROWWISE)
    p = O.mx_quantize(x, axis=O.ROWWISE)
    assert np.array_equal(g["q_row"], p["q_row"]) and np.array_equal(g["s_row"], p["s_row"].ravel())


@pytest.mark.parametrize("mode", [0, O.ELEM_E5M2 | O.SCALE_ROUND_UP])
def test_aligned_groups_are_column_slices(mode):
    rows = [64, 0, 32, 128, 96]
    M, K = sum(rows), 72
    x = W.normal(M, K, seed=63, sigma=3.0)
    g = O.mx_quantize_grouped(x, rows, axis=3 | mode)
    p = O.mx_quantize(x, axis=3 | mode)
    qc = split(g["q_col"], [K * m for m in rows])
    sc = split(g["s_col"], [K * (m // 32) for m in rows])
    r0 = 0
    for m, q, s in zip(rows, qc, sc):
        assert np.array_equal(q.reshape(K, m), p["q_col"][:, r0:r0 + m])
        assert np.array_equal(s.reshape(K, m // 32), p["s_col"][:, r0 // 32:(r0 + m) // 32])
        r0 += m


def test_group_dbias_is_numpy_column_sum():
    rows = [48, 0, 112]
    M, K = sum(rows), 96
    x = W.normal(M, K, seed=64, sigma=2.0)
    g = O.mx_quantize_grouped(x, rows, fusion=O.FUSE_DBIAS)
    xf = W.bf16_to_f32(x).astype(np.float64)
    assert np.array_equal(g["dbias"][0], xf[:48].sum(axis=0).astype(np.float32))
    assert np.all(g["dbias"][1] == 0)
    assert np.array_equal(g["dbias"][2], xf[48:].sum(axis=0).astype(np.float32))


def test_unaligned_groups_have_their_own_partial_blocks():
    rows = [48, 80]            # the boundary at row 48 is inside a 32-row block
    M, K = sum(rows), 40
    x = W.loguniform_rows(M, K, seed=65)
    g = O.mx_quantize_grouped(x, rows, axis=O.COLWISE)
    a = O.mx_quantize(np.ascontiguousarray(x[:48]), axis=O.COLWISE)
    b = O.mx_quantize(np.ascontiguousarray(x[48:]), axis=O.COLWISE)
    assert np.array_equal(g["q_col"], np.concatenate([a["q_col"].ravel(), b["q_col"].ravel()]))
    assert np.array_equal(g["s_col"], np.concatenate([a["s_col"].ravel(), b["s_col"].ravel()]))
    # the group boundary splits what would be one block of the stacked tensor
    p = O.mx_quantize(x, axis=O.COLWISE)
    assert p["s_col"].shape[1] == 4 and a["s_col"].shape[1] + b["s_col"].shape[1] == 5


def test_tiled_scales_per_group():
    rows = [64, 0, 96]
    M, K = sum(rows), 264
    x = W.loguniform_rows(M, K, seed=66)
    g = O.mx_quantize_grouped(x, rows, axis=3 | O.SCALE_TILED)
    srs = split(g["s_row"], [O.tiled_scale_bytes(m, 9) if m else 0 for m in rows])
    scs = split(g["s_col"], [O.tiled_scale_bytes(K, m // 32) if m else 0 for m in rows])
    r0 = 0
    for m, sr, sc in zip(rows, srs, scs):
        if m:
            c = O.mx_quantize(np.ascontiguousarray(x[r0:r0 + m]))
            assert np.array_equal(sr, O.scale_tiles(c["s_row"]))
            assert np.array_equal(sc, O.scale_tiles(c["s_col"]))
        r0 += m


# --- grouped NVFP4 -------------------------------------------------------------

def test_nvfp4_one_group_is_the_plain_cast():
    x = W.student_t_rows(96, 160, seed=71)
    for two_d in (False, True):
        g = O.nvfp4_quantize_transpose_grouped(x, [96], two_d=two_d)
        p = O.nvfp4_quantize_transpose(x, two_d=two_d)
        assert np.array_equal(g["q_row"], p["q_row"]) and np.array_equal(g["s_row"], p["s_row"])
        assert np.array_equal(g["q_col"], p["q_col"].ravel()) and np.array_equal(g["s_col"], p["s_col"].ravel())
        assert g["sg"][0] == p["sg"]


@pytest.mark.parametrize("two_d", [False, True])
def test_nvfp4_equal_amax_groups_are_slices_of_the_stacked_cast(two_d):
    rows = [48, 0, 16, 96]
    M, K = sum(rows), 80
    x = W.student_t_rows(M, K, seed=72)
    # give every group the same largest magnitude, so every S_g is the stack's
    big = np.uint16(0x4500)          # 2048, larger than any drawn value
    r0 = 0
    for m in rows:
        if m:
            x[r0, 0] = big
        r0 += m
    g = O.nvfp4_quantize_transpose_grouped(x, rows, two_d=two_d)
    p = O.nvfp4_quantize_transpose(x, two_d=two_d)
    assert np.all(g["sg"][[0, 2, 3]] == p["sg"]) and g["sg"][1] == 1.0
    assert np.array_equal(g["q_row"], p["q_row"]) and np.array_equal(g["s_row"], p["s_row"])
    qc = split(g["q_col"], [K * m // 2 for m in rows])
    sc = split(g["s_col"], [K * m // 16 for m in rows])
    r0 = 0
    for m, q, s in zip(rows, qc, sc):
        assert np.array_equal(q.reshape(K, m // 2), p["q_col"][:, r0 // 2:(r0 + m) // 2])
        assert np.array_equal(s.reshape(K, m // 16), p["s_col"][:, r0 // 16:(r0 + m) // 16])
        r0 += m


def test_nvfp4_group_global_scales_follow_group_amax():
    rows = [32, 64]
    x = W.student_t_rows(96, 48, seed=73)
    g = O.nvfp4_quantize_transpose_grouped(x, rows)
    xf = np.abs(W.bf16_to_f32(x))
    for gi, (a, b) in enumerate([(0, 32), (32, 96)]):
        A = np.float32(xf[a:b].max())
        assert g["sg"][gi] == np.float32(A / np.float32(2688.0))
    # a given amax array overrides the groups' own
    g2 = O.nvfp4_quantize_transpose_grouped(x, rows, amax=[1.0, 2.0])
    assert list(g2["sg"]) == [np.float32(1.0 / 2688.0), np.float32(2.0 / 2688.0)]


# --- grouped gated casts ------------------------------------------------------

@pytest.mark.parametrize("backward", [False, True])
def test_gated_grouped_rowwise_equals_stacked_and_aligned_slices(backward):
    rows = [64, 0, 32, 96]
    M, N = sum(rows), 80
    x = W.normal(M, 2 * N, seed=76)
    grad = W.normal(M, N, seed=77) if backward else None
    g = O.mx_quantize_gated_grouped(x, rows, O.GATED_SWIGLU, grad=grad)
    if backward:
        p = O.mx_quantize_dgated(grad, x, O.GATED_SWIGLU)
    else:
        p = O.mx_quantize_gated(x, O.GATED_SWIGLU)
    Wd = 2 * N if backward else N
    assert np.array_equal(g["q_row"], p["q_row"]) and np.array_equal(g["s_row"], p["s_row"].ravel())
    qc = split(g["q_col"], [Wd * m for m in rows])
    sc = split(g["s_col"], [Wd * (m // 32) for m in rows])
    r0 = 0
    for m, q, s in zip(rows, qc, sc):
        assert np.array_equal(q.reshape(Wd, m), p["q_col"][:, r0:r0 + m])
        assert np.array_equal(s.reshape(Wd, m // 32), p["s_col"][:, r0 // 32:(r0 + m) // 32])
        r0 += m
