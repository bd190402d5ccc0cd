"""Pins for partial blocks (lines whose length is not a multiple of 32):

  * a hand-worked partial block;
  * every output of an M x K cast equals the corresponding part of the cast of
    the tensor zero-padded to multiples of 32 -- zeros never change an amax
    and encode to zero, so a partial block must behave as the full block it
    would be with zero padding; the full-block rule is pinned elsewhere;
  * transposition and the tiled layout at partial sizes.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W


def test_hand_worked_partial_block():
    # row 0: 32 zeros, then the 3-element block [6, -1.5, 0.25]:
    # amax 6 -> byte 2 - 8 + 127 = 0x79, X = 2^-6: 384 -> e15 m4 (0x7C),
    # -96 -> e13 m4 with sign (0xEC), 16 -> e11 (0x58)
    x = np.zeros((32, 35), np.uint16)
    x[0, 32:35] = [0x40C0, 0xBFC0, 0x3E80]
    o = O.mx_quantize(x)
    assert o["s_row"].shape == (32, 2) and o["s_row"][0, 1] == 0x79
    assert list(o["q_row"][0, 32:35]) == [0x7C, 0xEC, 0x58]
    # column-wise: each of those columns has one non-zero element in a
    # 32-row block, so it is its own block amax
    assert o["s_col"].shape == (35, 1)
    assert list(o["s_col"][32:35, 0]) == [0x79, 0x77, 0x75]   # 6, 1.5, 0.25


@pytest.mark.parametrize("mode", [0, O.ELEM_E5M2 | O.SCALE_ROUND_UP])
@pytest.mark.parametrize("M,K", [(16, 8), (48, 40), (80, 200), (112, 264), (33, 31), (1, 1), (17, 9),
                                 (3, 70), (70, 3)])
def test_partial_equals_zero_padded(M, K, mode):
    x = W.loguniform_rows(M, K, seed=4000 + M + K)
    Mp, Kp = -(-M // 32) * 32, -(-K // 32) * 32
    xp = np.zeros((Mp, Kp), np.uint16)
    xp[:M, :K] = x
    o = O.mx_quantize(x, axis=3 | mode)
    p = O.mx_quantize(xp, axis=3 | mode)
    assert np.array_equal(o["q_row"], p["q_row"][:M, :K])
    assert np.array_equal(o["s_row"], p["s_row"][:M, :])
    assert np.array_equal(o["q_col"], p["q_col"][:K, :M])
    assert np.array_equal(o["s_col"], p["s_col"][:K, :])


def test_partial_fused_and_gated_equal_zero_padded():
    M, K = 48, 72
    x, g = W.make("c3_gelu_dbias_8192", M, K)
    xp, gp = np.zeros((64, 96), np.uint16), np.zeros((64, 96), np.uint16)
    xp[:M, :K], gp[:M, :K] = x, g
    o = O.mx_quantize(x, grad=g, fusion=O.FUSE_DGELU | O.FUSE_DBIAS)
    p = O.mx_quantize(xp, grad=gp, fusion=O.FUSE_DGELU | O.FUSE_DBIAS)
    assert np.array_equal(o["q_row"], p["q_row"][:M, :K]) and np.array_equal(o["s_col"], p["s_col"][:K])
    assert np.array_equal(o["dbias"], p["dbias"][:K])
    gx = W.make("c4_gated_8192", 48, 2 * 40)
    gxp = np.zeros((64, 2 * 64), np.uint16)
    gxp[:48, :40], gxp[:48, 64:104] = gx[:, :40], gx[:, 40:]
    og = O.mx_quantize_gated(gx, O.GATED_GEGLU)
    pg = O.mx_quantize_gated(gxp, O.GATED_GEGLU)
    assert np.array_equal(og["q_row"], pg["q_row"][:48, :40]) and np.array_equal(og["s_row"], pg["s_row"][:48])
    assert np.array_equal(og["q_col"], pg["q_col"][:40, :48]) and np.array_equal(og["s_col"], pg["s_col"][:40])


def test_partial_transpose_and_tiles():
    x = W.normal(80, 200, seed=41, sigma=4.0)
    a = O.mx_quantize(x)
    t = O.mx_quantize(np.ascontiguousarray(x.T))
    assert np.array_equal(a["q_col"], t["q_row"]) and np.array_equal(a["s_col"], t["s_row"])
    tl = O.mx_quantize(x, axis=3 | O.SCALE_TILED)
    assert tl["s_row"].size == O.tiled_scale_bytes(80, 7) == 3 * 1 * 256
    assert np.array_equal(tl["s_row"], O.scale_tiles(a["s_row"]))
    assert np.array_equal(tl["s_col"], O.scale_tiles(a["s_col"]))
