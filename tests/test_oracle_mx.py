"""Pins for the oracle's MXFP8 block and tensor quantisation (CPU only).

  * hand-derived blocks (tests/golden/mx_blocks.txt, derivations inline there);
  * an independent implementation built from torch primitives (log2 for the
    shared exponent, torch's own float8_e4m3fn conversion for the elements),
    compared on whole tensors in both directions;
  * invariants that hold at any size: dequantisation error within half an
    E4M3 ulp at the block scale, transpose, sign symmetry, power-of-two
    equivariance, and the divide -> multiply-by-inverse swap being exact.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, xin, s, q = [f.strip() for f in line.split("|")]
        rows.append((tag, [int(h, 16) for h in xin.split(",")], int(s, 16),
                     [int(h, 16) for h in q.split(",")]))
    return rows


@pytest.mark.parametrize("tag,xin,scale,codes", load_golden("mx_blocks.txt"))
def test_golden_block(tag, xin, scale, codes):
    bits = np.zeros(32, np.uint16)
    bits[:len(xin)] = xin
    vals = [O.bf16_value(int(b)) for b in bits]
    q, s = O.mx_block(vals)
    assert s == scale, tag
    want = np.zeros(32, np.uint8)
    want[:len(codes)] = codes if len(codes) > 1 else codes * len(xin)
    assert list(q) == list(want), tag


@pytest.mark.parametrize("tag,xin,scale,codes", load_golden("mx_blocks.txt"))
def test_golden_block_through_tensor_both_axes(tag, xin, scale, codes):
    """The same block placed in row 0 of a 32x32 tensor (row-wise) and in
    column 0 (column-wise) must give the same bytes."""
    x = np.zeros((32, 32), np.uint16)
    x[0, :len(xin)] = xin
    r = O.mx_quantize(x, axis=O.ROWWISE)
    xt = np.ascontiguousarray(x.T)
    c = O.mx_quantize(xt, axis=O.COLWISE)
    assert r["s_row"][0, 0] == scale and c["s_col"][0, 0] == scale
    assert np.array_equal(r["q_row"][0], c["q_col"][0])


def torch_mx_rows(bits):
    """Independent row-wise MX cast from torch primitives."""
    x = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16).double()
    M, K = x.shape
    blk = x.view(M, K // 32, 32)
    amax = blk.abs().amax(-1)
    e = torch.floor(torch.log2(amax))
    byte = torch.where(amax == 0, torch.zeros_like(e), torch.clamp(e - 8 + 127, 0, 254))
    X = torch.pow(2.0, byte - 127).unsqueeze(-1)
    v = (blk / X).float().clamp(-448.0, 448.0)
    q = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(M, K).numpy()
    return q, byte.to(torch.uint8).numpy()


@pytest.mark.parametrize("case", ["special", "loguniform", "normal", "tiny"])
def test_tensor_matches_torch_pipeline(case):
    if case == "special":
        x = W.special_256x512()
    elif case == "loguniform":
        x = W.loguniform_rows(96, 224, seed=7)
    elif case == "normal":
        x = W.normal(64, 160, seed=8, sigma=3.0)
    else:
        x = W.bf16_bits(np.random.default_rng(9).standard_normal((32, 64)).astype(np.float32)
                        * np.float32(1e-38))
    out = O.mx_quantize(x)
    q, s = torch_mx_rows(x)
    assert np.array_equal(out["q_row"], q) and np.array_equal(out["s_row"], s)
    qt, st = torch_mx_rows(np.ascontiguousarray(x.T))
    assert np.array_equal(out["q_col"], qt) and np.array_equal(out["s_col"], st)


def test_special_tiles_hit_their_cases():
    x = W.special_256x512()
    out = O.mx_quantize(x)
    assert np.all(out["s_row"][0:32, 0] == 0) and np.all(out["q_row"][0:32, 0:32] == 0)
    assert np.all(out["s_row"][32:64, 1] == 122)          # amax exactly 2^3
    assert np.all(out["s_col"][32:64, 1] == 122)
    assert np.all(out["s_row"][96:128, 3] == 246)         # near +-3e38
    assert np.all((out["q_row"][96:128, 96:128] & 0x7F) >= 0x7C)


def e4m3_half_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)          # subnormal spacing 2^-9 below 2^-6


def test_dequantisation_error_bound():
    x = W.loguniform_rows(128, 256, seed=10)
    out = O.mx_quantize(x)
    xv = W.bf16_to_f32(x).astype(np.float64)
    X = np.repeat(2.0 ** (out["s_row"].astype(np.float64) - 127), 32, axis=1)
    dq = torch.from_numpy(out["q_row"]).view(torch.float8_e4m3fn).double().numpy() * X
    v = xv / X
    sat = np.abs(v) > 448
    assert np.all(np.abs(dq[sat]) == 448 * X[sat])
    assert np.all(np.abs(dq - xv)[~sat] <= e4m3_half_ulp(v[~sat]) * X[~sat])
    assert sat.mean() > 0.001     # the floor rule does saturate some amax elements


def test_transpose_sign_and_power_of_two_invariants():
    x = W.normal(64, 96, seed=14, sigma=5.0)
    a = O.mx_quantize(x)
    # transpose: the column output of X is the row output of X^T
    t = O.mx_quantize(np.ascontiguousarray(x.T))
    assert np.array_equal(a["q_col"], t["q_row"]) and np.array_equal(a["s_col"], t["s_row"])
    # sign symmetry: same scales, element sign bit flipped (zero -> -0 too)
    n = O.mx_quantize(x ^ np.uint16(0x8000))
    assert np.array_equal(n["s_row"], a["s_row"]) and np.array_equal(n["q_row"], a["q_row"] ^ 0x80)
    assert np.array_equal(n["q_col"], a["q_col"] ^ 0x80)
    # 2^j scaling: scales shift by j, elements unchanged (no clamp reached)
    for j in (-20, 5, 60):
        xs = W.bf16_bits(W.bf16_to_f32(x) * np.float32(2.0 ** j))
        s = O.mx_quantize(xs)
        assert np.array_equal(s["s_row"].astype(int), a["s_row"].astype(int) + j)
        assert np.array_equal(s["q_row"], a["q_row"]) and np.array_equal(s["q_col"], a["q_col"])


def test_division_by_scale_equals_multiply_by_inverse():
    """The torchao PR replaces 32 divisions per block by one inverse and 32
    multiplies.  With a power-of-two scale both are exact, so the swap cannot
    change a code: check x / X == x * (1/X) in fp32 for every reachable pair."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    xf = W.bf16_to_f32(bits)
    ef = (bits.astype(np.int64) >> 7) & 0xFF
    for b in range(0, 247, 7):
        sel = ef <= b + 8
        X = np.float32(2.0 ** (b - 127)) if b >= 1 else np.float32(2.0 ** -127)
        inv = np.float32(2.0 ** (127 - b))
        assert np.array_equal((xf[sel] / X).view(np.uint32), (xf[sel] * inv).view(np.uint32))


def test_nonfinite_block_reading():
    x = np.zeros((32, 64), np.uint16)
    x[0, 3] = 0x7F80          # +Inf in row 0, block 0
    x[5, 40] = 0x7FC1         # NaN in row 5, block 1
    out = O.mx_quantize(x)
    assert out["s_row"][0, 0] == 0xFF and np.all(out["q_row"][0, :32] == 0x7F)
    assert out["s_row"][0, 1] == 0 and out["s_row"][5, 1] == 0xFF
    assert out["s_col"][3, 0] == 0xFF and np.all(out["q_col"][3, :] == 0x7F)


def test_shape_errors():
    # any positive size is a valid tensor (partial blocks); empty ones are not
    with pytest.raises(ValueError):
        O.mx_quantize(np.zeros((0, 32), np.uint16))
    with pytest.raises(ValueError):
        O.mx_quantize(np.zeros((16, 0), np.uint16))


def test_dbias_is_column_sum_of_fused_values():
    x, g = W.make("c3_gelu_dbias_8192", 64, 96)
    for fusion in (O.FUSE_DBIAS, O.FUSE_GELU | O.FUSE_DBIAS, O.FUSE_DGELU | O.FUSE_DBIAS):
        out = O.mx_quantize(x, grad=g, fusion=fusion, want_y=True)
        ref = W.bf16_to_f32(out["y"]).astype(np.float64).sum(axis=0)
        assert np.array_equal(out["dbias"], ref.astype(np.float32))
    # closed form: a constant tensor sums to M * c
    c = np.full((64, 32), 0x3FC0, np.uint16)   # 1.5
    assert np.all(O.mx_quantize(c, fusion=O.FUSE_DBIAS)["dbias"] == 96.0)
