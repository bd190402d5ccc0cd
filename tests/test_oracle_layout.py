"""Pins for the oracle's GEMM-ready (MFMA tile) scale layout.

  * a hand-worked tile (tests/golden/scale_tiles.txt);
  * a block-scaled matrix product computed the way a 32x32x64 MFMA wave walks
    the tiled scales (tile by tile, lane by lane, step by step) equals the same
    product with the compact scales -- the layout is checked against the
    consumer it is for, not against its own formula;
  * padding to whole tiles with zero bytes, sizes, and the tensor entry points
    writing exactly the tiled form of their compact scales.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_tile():
    s = (8 * np.arange(32)[:, None] + np.arange(8)[None, :]).astype(np.uint8)
    t = O.scale_tiles(s)
    assert t.size == 256
    for line in open(os.path.join(GOLDEN, "scale_tiles.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lane, b = [f.strip() for f in line.split("|")]
        want = [int(h, 16) for h in b.split(",")]
        L = int(lane)
        assert list(t[4 * L:4 * L + 4]) == want, L


def test_sizes_and_padding():
    assert O.tiled_scale_bytes(32, 8) == 256
    assert O.tiled_scale_bytes(64, 12) == 2 * 2 * 256
    assert O.tiled_scale_bytes(16384, 512) == 512 * 64 * 256       # no padding at 16384^2
    assert O.tiled_scale_bytes(16384, 512) == 16384 * 512
    rng = np.random.default_rng(3)
    s = rng.integers(1, 255, (64, 12), dtype=np.uint8)        # no zero scales
    t = O.scale_tiles(s)
    assert np.count_nonzero(t) == s.size                       # every pad byte is 0
    assert sorted(t[t != 0].tolist()) == sorted(s.ravel().tolist())


def dequant_rows(q, s):
    """Compact layout: value[m][k] = e4m3(q[m][k]) * 2^(s[m][k / 32] - 127)."""
    v = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    return v * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)


def mfma_walk_product(qa, ta, qb, tb, M, N, K):
    """C = A B^T the way a 32x32x64 block-scaled MFMA wave reads the tiled
    scales: for each 32 x 32 output tile and each 64-wide K step, lane L's
    scale -- byte (step % 4) of its word in tile (block tile, row tile) --
    scales row L % 32 of A (and of B) over K block L / 32 of the step.  (On
    the hardware the lane's operand bytes hold 16 K values of each of the
    step's two blocks; which lane carries an element does not change the
    product, the scale of each (row, block) does.)"""
    a = torch.from_numpy(qa).view(torch.float8_e4m3fn).double().numpy()
    b = torch.from_numpy(qb).view(torch.float8_e4m3fn).double().numpy()
    RA, RB = M // 32, N // 32
    C = np.zeros((M, N))
    for mt in range(M // 32):
        for nt in range(N // 32):
            acc = np.zeros((32, 32))
            for step in range(K // 64):
                bt, j = step // 4, step % 4
                wa = ta[(bt * RA + mt) * 256:(bt * RA + mt + 1) * 256].reshape(64, 4)
                wb = tb[(bt * RB + nt) * 256:(bt * RB + nt + 1) * 256].reshape(64, 4)
                for L in range(64):
                    r, h = L % 32, L // 32
                    k0 = 64 * step + 32 * h
                    av = a[32 * mt + r, k0:k0 + 32] * 2.0 ** (int(wa[L, j]) - 127)
                    for L2 in range(64):
                        if L2 // 32 != h:
                            continue
                        r2 = L2 % 32
                        bv = b[32 * nt + r2, k0:k0 + 32] * 2.0 ** (int(wb[L2, j]) - 127)
                        acc[r, r2] += float(np.dot(av, bv))
            C[32 * mt:32 * mt + 32, 32 * nt:32 * nt + 32] = acc
    return C


def test_mfma_consumer_sees_the_compact_scales():
    M, N, K = 64, 32, 512
    xa = W.loguniform_rows(M, K, seed=21)
    xb = W.loguniform_rows(N, K, seed=22)
    ca = O.mx_quantize(xa, axis=O.ROWWISE)
    cb = O.mx_quantize(xb, axis=O.ROWWISE)
    ta = O.mx_quantize(xa, axis=O.ROWWISE | O.SCALE_TILED)
    tb = O.mx_quantize(xb, axis=O.ROWWISE | O.SCALE_TILED)
    assert np.array_equal(ta["q_row"], ca["q_row"]) and np.array_equal(tb["q_row"], cb["q_row"])
    ref = dequant_rows(ca["q_row"], ca["s_row"]) @ dequant_rows(cb["q_row"], cb["s_row"]).T
    got = mfma_walk_product(ta["q_row"], ta["s_row"], tb["q_row"], tb["s_row"], M, N, K)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    # a wrong layout (steps and halves swapped inside the word) is caught
    bad = ta["s_row"].reshape(-1, 64, 4)[:, :, ::-1].ravel().copy()
    wrong = mfma_walk_product(ta["q_row"], bad, tb["q_row"], tb["s_row"], M, N, K)
    assert not np.allclose(wrong, ref, rtol=1e-6)


@pytest.mark.parametrize("mode", [0, O.ELEM_E5M2 | O.SCALE_ROUND_UP])
def test_tensor_entry_points_write_the_tiled_form(mode):
    x = W.loguniform_rows(96, 800, seed=23)
    c = O.mx_quantize(x, axis=3 | mode)
    t = O.mx_quantize(x, axis=3 | mode | O.SCALE_TILED)
    assert np.array_equal(t["q_row"], c["q_row"]) and np.array_equal(t["q_col"], c["q_col"])
    assert np.array_equal(t["s_row"], O.scale_tiles(c["s_row"]))
    assert np.array_equal(t["s_col"], O.scale_tiles(c["s_col"]))
    g = W.make("c4_gated_8192", 64, 576)
    cg = O.mx_quantize_gated(g, O.GATED_SWIGLU, axis=3 | mode)
    tg = O.mx_quantize_gated(g, O.GATED_SWIGLU, axis=3 | mode | O.SCALE_TILED)
    assert np.array_equal(tg["s_col"], O.scale_tiles(cg["s_col"]))
    grad, xb = W.make("f1_dgated_8192", 64, 160)
    cd = O.mx_quantize_dgated(grad, xb, O.GATED_GEGLU, axis=3 | mode)
    td = O.mx_quantize_dgated(grad, xb, O.GATED_GEGLU, axis=3 | mode | O.SCALE_TILED)
    assert np.array_equal(td["s_row"], O.scale_tiles(cd["s_row"]))
