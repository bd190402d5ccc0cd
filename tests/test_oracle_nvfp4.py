"""Pins for the oracle's NVFP4 quantize-transpose (CPU only).

  * hand-derived blocks with tensor scale 1 (tests/golden/nvfp4_blocks.txt);
  * an independent implementation of the same scale chain in numpy float32
    arithmetic (IEEE single operations, not the oracle's double-then-round
    route) with a brute-force E2M1 encoder, compared on whole tensors;
  * invariants: dequantisation within half an E2M1 ulp at the block scale,
    the E4M3 block scale is the nearest to b/6/S_g, transpose, sign symmetry.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def load_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "nvfp4_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, xin, s, q = [f.strip() for f in line.split("|")]
        rows.append((tag, [int(h, 16) for h in xin.split(",")], int(s, 16),
                     [int(h, 16) for h in q.split(",")]))
    return rows


@pytest.mark.parametrize("tag,xin,scale,nibbles", load_golden())
def test_golden_block(tag, xin, scale, nibbles):
    x = np.zeros((16, 16), np.uint16)
    x[0, :len(xin)] = xin
    out = O.nvfp4_quantize_transpose(x, tensor_amax=2688.0)
    assert out["sg"] == 1.0
    assert out["s_row"][0, 0] == scale, tag
    want = np.zeros(16, np.uint8)
    want[:len(nibbles)] = nibbles
    packed = want[0::2] | (want[1::2] << 4)
    assert list(out["q_row"][0]) == list(packed), tag
    # the same block as column 0 of the transpose
    outT = O.nvfp4_quantize_transpose(np.ascontiguousarray(x.T), tensor_amax=2688.0)
    assert outT["s_col"][0, 0] == scale and list(outT["q_col"][0]) == list(packed)


def test_golden_ties_packing_literal():
    """Byte packing of the first golden block, written out: element 2j low nibble."""
    tag, xin, scale, nib = load_golden()[0]
    x = np.zeros((16, 16), np.uint16)
    x[0] = xin
    out = O.nvfp4_quantize_transpose(x, tensor_amax=2688.0)
    assert bytes(out["q_row"][0]).hex() == "6746240 2f880 5624".replace(" ", "")


def brute_e2m1(v):
    a = np.abs(v)
    d = np.abs(a[..., None] - E2M1)
    best = d.min(-1, keepdims=True)
    hit = d == best
    idx = np.argmax(hit, -1)
    two = hit.sum(-1) == 2
    idx = np.where(two & (idx % 2 == 1), idx + 1, idx)
    idx = np.where(a >= 6, 7, idx)
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def numpy_nvfp4_rows(bits, A):
    """Independent row-wise NVFP4 in numpy float32 arithmetic."""
    x = W.bf16_to_f32(bits)
    M, K = x.shape
    f32 = np.float32
    Sg = f32(1.0) if A == 0 else f32(A) / f32(2688.0)
    blk = x.reshape(M, K // 16, 16)
    b = np.abs(blk).max(-1)
    sq = (b / f32(6.0)) / Sg
    sbyte = torch.from_numpy(np.minimum(sq, f32(448.0))).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    d = torch.from_numpy(sbyte).view(torch.float8_e4m3fn).float().numpy()
    den = d * Sg
    with np.errstate(divide="ignore"):
        inv = np.where(den == 0, f32(0.0), f32(1.0) / den).astype(np.float32)
    v = blk * inv[..., None]
    codes = brute_e2m1(v.astype(np.float64)).reshape(M, K)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), sbyte, Sg


@pytest.mark.parametrize("case", ["student_t", "normal", "loguniform", "tiny"])
def test_tensor_matches_numpy_float32_chain(case):
    if case == "student_t":
        x = W.student_t_rows(128, 160, seed=31)
    elif case == "normal":
        x = W.normal(64, 96, seed=32)
    elif case == "loguniform":
        x = W.loguniform_rows(96, 64, seed=33)
    else:
        x = W.normal(32, 64, seed=34, sigma=1e-20)
    out = O.nvfp4_quantize_transpose(x)
    A = float(np.abs(W.bf16_to_f32(x)).max())
    q, s, Sg = numpy_nvfp4_rows(x, A)
    assert out["sg"] == float(Sg)
    assert np.array_equal(out["q_row"], q) and np.array_equal(out["s_row"], s)
    qt, st, _ = numpy_nvfp4_rows(np.ascontiguousarray(x.T), A)
    assert np.array_equal(out["q_col"], qt) and np.array_equal(out["s_col"], st)


def test_global_scale():
    assert O.nvfp4_global_scale(0.0) == 1.0
    assert O.nvfp4_global_scale(2688.0) == 1.0
    rng = np.random.default_rng(35)
    for A in W.bf16_to_f32(W.bf16_bits(rng.uniform(1e-3, 1e4, 200).astype(np.float32))):
        assert O.nvfp4_global_scale(float(A)) == float(np.float32(A) / np.float32(2688.0))


def e2m1_half_ulp(v):
    a = np.abs(v)
    return np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))


def test_dequantisation_bound_and_scale_choice():
    x = W.student_t_rows(256, 256, seed=36)
    out = O.nvfp4_quantize_transpose(x)
    xf = W.bf16_to_f32(x).astype(np.float64)
    Sg = out["sg"]
    d = torch.from_numpy(out["s_row"]).view(torch.float8_e4m3fn).double().numpy()
    den = np.repeat(d * Sg, 16, axis=1)
    codes = np.stack([out["q_row"] & 0xF, out["q_row"] >> 4], -1).reshape(x.shape)
    val = np.array([O.e2m1_value(c) for c in range(16)])[codes]
    v = xf / den
    sat = np.abs(v) > 6 * (1 + 2.0 ** -21)
    slack = 1 + 2.0 ** -21
    ok = np.abs(val * den - xf) <= e2m1_half_ulp(v) * den * slack + 1e-300
    assert np.all(ok[~sat])
    assert np.all(np.abs(val[sat]) == 6)
    # the stored block scale is the E4M3 value nearest to (b/6)/S_g (fp32 rounding aside)
    b = np.abs(xf).reshape(256, 16, 16).max(-1)
    ideal = b / 6 / Sg
    near = O.e4m3_encode_array(ideal)
    assert np.mean(near == out["s_row"]) > 0.999


def test_transpose_and_sign_invariants():
    x = W.student_t_rows(64, 96, seed=37)
    a = O.nvfp4_quantize_transpose(x)
    t = O.nvfp4_quantize_transpose(np.ascontiguousarray(x.T))
    assert np.array_equal(a["q_col"], t["q_row"]) and np.array_equal(a["s_col"], t["s_row"])
    n = O.nvfp4_quantize_transpose(x ^ np.uint16(0x8000))
    assert np.array_equal(n["s_row"], a["s_row"])
    assert np.array_equal(n["q_row"], a["q_row"] ^ 0x88)


def test_zero_tensor_and_shape_errors():
    z = np.zeros((16, 32), np.uint16)
    out = O.nvfp4_quantize_transpose(z)
    assert out["sg"] == 1.0 and not out["q_row"].any() and not out["s_row"].any()
    with pytest.raises(ValueError):
        O.nvfp4_quantize_transpose(np.zeros((0, 32), np.uint16))


def test_hand_worked_odd_row():
    """One row [6, -3, 1]: amax 6, S_g = 6/2688; the block's b/6 = 1 over S_g
    is 448 -> scale byte 0x7E, multiplier 1/(448 S_g) = 1; codes E2M1(6) = 7,
    E2M1(-3) = 0x8 | 5, E2M1(1) = 2, packed into ceil(3/2) = 2 bytes with the
    missing fourth code 0.  Transposed, each column is a block of one
    element: 6 as above; 3: 0.5 / S_g = 224 -> byte 0x76, multiplier 2, -6 ->
    0x8 | 7; 1: (1/6) / S_g = 74.67 -> nearest E4M3 72 (0x69), multiplier
    2688 / 432 = 6.22, which saturates to code 7."""
    x = np.array([[0x40C0, 0xC040, 0x3F80]], np.uint16)
    o = O.nvfp4_quantize_transpose(x)
    assert o["q_row"].shape == (1, 2) and o["s_row"].shape == (1, 1)
    assert list(o["q_row"][0]) == [0xD7, 0x02] and o["s_row"][0, 0] == 0x7E
    assert o["q_col"].shape == (3, 1) and list(o["q_col"][:, 0]) == [0x07, 0x0F, 0x07]
    assert list(o["s_col"][:, 0]) == [0x7E, 0x76, 0x69]


@pytest.mark.parametrize("two_d", [False, True], ids=["1d", "2d"])
@pytest.mark.parametrize("M,K", [(1, 1), (17, 9), (5, 31), (33, 50), (40, 7), (16, 24), (3, 16)])
def test_partial_blocks_equal_zero_padded(M, K, two_d):
    """Any M, K: every output equals the matching bytes of the cast of the
    tensor zero-padded to multiples of 16 (zeros change no amax, no block
    maximum, and code to 0, which also fills the high nibble of an odd row's
    last byte); the full-block chain is pinned by the tests above."""
    x = W.student_t_rows(M, K, seed=300 + M + K)
    Mp, Kp = -(-M // 16) * 16, -(-K // 16) * 16
    xp = np.zeros((Mp, Kp), np.uint16)
    xp[:M, :K] = x
    o = O.nvfp4_quantize_transpose(x, two_d=two_d)
    p = O.nvfp4_quantize_transpose(xp, two_d=two_d)
    assert o["sg"] == p["sg"]
    assert np.array_equal(o["q_row"], p["q_row"][:M, :-(-K // 2)])
    assert np.array_equal(o["s_row"], p["s_row"][:M, :-(-K // 16)])
    assert np.array_equal(o["q_col"], p["q_col"][:K, :-(-M // 2)])
    assert np.array_equal(o["s_col"], p["s_col"][:K, :-(-M // 16)])


def test_grouped_any_rows_equal_per_group_casts():
    rows, K = [5, 0, 33, 16, 1], 19
    x = W.student_t_rows(sum(rows), K, seed=310)
    for two_d in (False, True):
        g = O.nvfp4_quantize_transpose_grouped(x, rows, two_d=two_d)
        r0 = qc = sc = 0
        for gi, m in enumerate(rows):
            if m == 0:
                assert g["sg"][gi] == 1.0
                continue
            o = O.nvfp4_quantize_transpose(np.ascontiguousarray(x[r0:r0 + m]), two_d=two_d)
            assert g["sg"][gi] == o["sg"]
            assert np.array_equal(g["q_row"][r0:r0 + m], o["q_row"])
            assert np.array_equal(g["s_row"][r0:r0 + m], o["s_row"])
            assert np.array_equal(g["q_col"][qc:qc + o["q_col"].size], o["q_col"].ravel())
            assert np.array_equal(g["s_col"][sc:sc + o["s_col"].size], o["s_col"].ravel())
            r0, qc, sc = r0 + m, qc + o["q_col"].size, sc + o["s_col"].size
        assert qc == g["q_col"].size and sc == g["s_col"].size


# --- NVFP4 with 2D (16 x 16 block) scaling ------------------------------------

def test_2d_transposes_like_the_transpose():
    """A 16 x 16 block is its own transpose's block: the column-wise outputs of
    x equal the row-wise outputs of x^T (same tensor scale)."""
    x = W.student_t_rows(96, 160, seed=61)
    a = O.nvfp4_quantize_transpose(x, two_d=True)
    b = O.nvfp4_quantize_transpose(np.ascontiguousarray(x.T), two_d=True)
    assert a["sg"] == b["sg"]
    assert np.array_equal(a["q_col"], b["q_row"]) and np.array_equal(a["s_col"], b["s_row"])
    assert np.array_equal(a["q_row"], b["q_col"]) and np.array_equal(a["s_row"], b["s_col"])


def test_2d_scale_is_one_per_block_replicated():
    x = W.student_t_rows(64, 128, seed=62)
    a = O.nvfp4_quantize_transpose(x, two_d=True)
    s = a["s_row"].reshape(4, 16, 8)
    assert np.all(s == s[:, :1, :])                       # same for the 16 rows of a block
    assert np.array_equal(a["s_col"][::16, :], a["s_row"][::16, :].T)


def test_2d_equals_1d_when_the_rows_of_a_block_are_equal():
    base = W.student_t_rows(4, 256, seed=63)
    x = np.repeat(base, 16, axis=0)                       # each 16-row group is one row repeated
    a = O.nvfp4_quantize_transpose(x, axis=1, two_d=True)
    b = O.nvfp4_quantize_transpose(x, axis=1)
    assert np.array_equal(a["q_row"], b["q_row"]) and np.array_equal(a["s_row"], b["s_row"])


def test_2d_block_amax_spans_rows():
    """One element of 6.0 in a block of 0.5s, tensor scale 1 (amax 2688 given):
    b = 6 gives scale E4M3(1) = 0x38 and multiplier 1 for all 256 elements, so
    every 0.5 codes as E2M1 0x1 -- in 1D, the rows without the 6.0 would get
    their own (smaller) scale instead."""
    x = np.full((16, 16), 0x3F00, np.uint16)              # 0.5
    x[3, 7] = 0x40C0                                      # 6.0
    a = O.nvfp4_quantize_transpose(x, tensor_amax=2688.0, two_d=True)
    assert a["sg"] == 1.0
    assert np.all(a["s_row"] == 0x38) and np.all(a["s_col"] == 0x38)
    codes = np.stack([a["q_row"] & 0xF, a["q_row"] >> 4], axis=-1).reshape(16, 16)
    want = np.full((16, 16), 0x1, np.uint8)
    want[3, 7] = 0x7
    assert np.array_equal(codes, want)
    one_d = O.nvfp4_quantize_transpose(x, tensor_amax=2688.0)
    assert one_d["s_row"][0, 0] != 0x38                   # row 0 has no 6.0


def _poisoned(M, K, seed, where, bits):
    x = W.normal(M, K, seed=seed)
    for (r, c), b in zip(where, bits):
        x[r, c] = b
    return x


@pytest.mark.parametrize("bits,kind", [((0x7FC0,), "nan"), ((0xFFC1,), "nan"), ((0x7F80,), "inf"),
                                       ((0xFF80,), "inf"), ((0xFF80, 0x7FC0), "nan")])
def test_nonfinite_tensor_amax(bits, kind):
    """The tensor amax is NaN when an element is NaN, else Inf when one is
    infinite (a NaN outranks an Inf), as numpy finds them."""
    x = _poisoned(32, 48, 5, [(5, 7), (30, 1)][:len(bits)], bits)
    A = O.absmax(x)
    f = W.bf16_to_f32(x).astype(np.float64)
    assert np.isnan(A) == np.isnan(f).any()
    assert (np.isinf(A) and A > 0) == (not np.isnan(f).any() and np.isinf(f).any())
    assert kind == ("nan" if np.isnan(A) else "inf")


@pytest.mark.parametrize("bits", [0x7FC0, 0xFF80])
@pytest.mark.parametrize("two_d", [False, True])
def test_nonfinite_tensor_has_nan_scales_and_zero_codes(bits, two_d):
    """R16: a tensor holding a NaN or an Inf has a non-finite amax A and so no
    usable global scale: S_g = A/2688 stays NaN or Inf, every scale byte is
    0x7F (the E4M3 NaN) and every element code 0, in both layouts."""
    x = _poisoned(48, 80, 6, [(17, 33)], [bits])
    o = O.nvfp4_quantize_transpose(x, two_d=two_d)
    assert np.isnan(o["sg"]) if bits == 0x7FC0 else (np.isinf(o["sg"]) and o["sg"] > 0)
    for k in ("s_row", "s_col"):
        assert o[k].shape == ((48, 5) if k == "s_row" else (80, 3))
        assert (o[k] == 0x7F).all(), k
    for k in ("q_row", "q_col"):
        assert (o[k] == 0).all(), k
    # one output direction at a time gives the same bytes
    r = O.nvfp4_quantize_transpose(x, axis=1, two_d=two_d)
    assert (r["s_row"] == 0x7F).all() and (r["q_row"] == 0).all()
    # a given non-finite amax does the same to a finite tensor
    f = O.nvfp4_quantize_transpose(W.normal(48, 80, seed=6), tensor_amax=float("inf"), two_d=two_d)
    assert (f["s_row"] == 0x7F).all() and (f["q_col"] == 0).all() and np.isinf(f["sg"])


def test_nonfinite_group_leaves_the_other_groups_alone():
    rows = [32, 16, 0, 48]
    x = W.normal(96, 64, seed=7)
    x[40, 3] = 0x7FC0                      # a NaN in group 1 (rows 32..47)
    o = O.nvfp4_quantize_transpose_grouped(x, rows)
    assert np.isnan(o["sg"][1]) and o["sg"][2] == 1.0
    assert np.isfinite(o["sg"][[0, 3]]).all()
    assert (o["s_row"][32:48] == 0x7F).all() and (o["q_row"][32:48] == 0).all()
    # group 1's transposed outputs: [64][16/2] at byte 64*32/2, [64][16/16] at 64*32/16
    assert (o["q_col"][64 * 16:64 * 16 + 64 * 8] == 0).all()
    assert (o["s_col"][64 * 2:64 * 2 + 64] == 0x7F).all()
    for g, (r0, m) in enumerate(((0, 32), (48, 48))):
        own = O.nvfp4_quantize_transpose(x[r0:r0 + m])
        gi = (0, 3)[g]
        assert own["sg"] == o["sg"][gi]
        assert np.array_equal(own["s_row"], o["s_row"][r0:r0 + m])
        assert np.array_equal(own["q_row"], o["q_row"][r0:r0 + m])
