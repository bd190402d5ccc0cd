"""Pins for the oracle's MX format variants (CPU only): E5M2 elements and the
round-up E8M0 rule, selected by flags beside the axis bits.

  * E5M2 decoding equals IEEE half precision's top byte (numpy float16), and
    encoding equals RNE rounding of the half-precision bit pattern for every
    finite half value, and torch's float8_e5m2 conversion on every bf16 value
    in range;
  * the two scale rules over every positive finite bf16 amax, checked by what
    each rule promises (floor: amax / X lands in the element format's largest
    binade; round-up: amax / X <= max and halving X would overflow) and by the
    mantissa threshold 96 that follows from max = 1.75 * 2^emax;
  * hand-worked blocks (tests/golden/mx_variant_blocks.txt);
  * whole tensors against a pipeline built from torch primitives (log2 / ceil
    for the byte, torch's float8 conversions for the elements), both axes.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MODES = [0, O.ELEM_E5M2, O.SCALE_ROUND_UP, O.ELEM_E5M2 | O.SCALE_ROUND_UP]


def fmt(mode):
    """(emax, max finite, torch dtype) of the element format."""
    if mode & O.ELEM_E5M2:
        return 15, 57344.0, torch.float8_e5m2
    return 8, 448.0, torch.float8_e4m3fn


def test_e5m2_decode_is_half_precision_top_byte():
    for c in range(256):
        h = np.array([c << 8], np.uint16).view(np.float16)[0]
        v = O.e5m2_value(c)
        if np.isnan(h):
            assert np.isnan(v), c
        else:
            assert v == float(h), (c, v, float(h))


def test_e5m2_encode_every_finite_half():
    """E5M2 is half precision with 8 fewer significand bits, so the nearest
    code (ties to even) is the half bit pattern rounded at bit 8."""
    bits = np.arange(65536, dtype=np.uint32)
    bits = bits[(bits & 0x7C00) != 0x7C00].astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    mag = bits.astype(np.uint32) & 0x7FFF
    r = (mag + 0x7F + ((mag >> 8) & 1)) >> 8
    want = (np.minimum(r, 0x7B) | ((bits >> 8) & 0x80)).astype(np.uint8)
    got = O.e5m2_encode_array(vals)
    assert np.array_equal(got, want)


def test_e5m2_encode_matches_torch_on_every_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    f = W.bf16_to_f32(bits)
    got = O.e5m2_encode_array(f.astype(np.float64))
    inr = np.abs(f) <= 57344.0
    want = torch.from_numpy(f[inr]).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(got[inr], want)
    assert np.all((got[~inr] & 0x7F) == 0x7B)
    assert np.array_equal(got[~inr] >> 7, (f[~inr] < 0).astype(np.uint8))


def test_e5m2_specials():
    assert O.e5m2_encode(float("inf")) == 0x7B and O.e5m2_encode(-float("inf")) == 0xFB
    assert O.e5m2_encode(float("nan")) == 0x7F
    assert O.e5m2_encode(-0.0) == 0x80 and O.e5m2_encode(0.0) == 0x00
    assert O.e5m2_encode(61439.0) == 0x7B and O.e5m2_encode(2.0 ** -17) == 0x00
    assert O.e5m2_encode(2.0 ** -17 * 1.0000001) == 0x01


@pytest.mark.parametrize("mode", MODES)
def test_scale_rule_every_bf16_amax(mode):
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    amax = W.bf16_to_f32(bits).astype(np.float64)
    emax, vmax, _ = fmt(mode)
    b = np.array([O.e8m0_byte_mode(float(a), mode) for a in amax], np.int64)
    r = amax / 2.0 ** (b - 127)                # exact: X is a power of two
    live = b > 0
    if mode & O.SCALE_ROUND_UP:
        assert np.all(r <= vmax)
        assert np.all(2.0 * r[live] > vmax)
    else:
        lo, hi = 2.0 ** emax, 2.0 ** (emax + 1)
        assert np.all((r[live] >= lo) & (r[live] < hi))
        assert np.all(r[~live] < hi)
    # mantissa threshold: the two rules differ exactly when amax > 1.75 * 2^E
    # (bf16 mantissa above 96), because max = 1.75 * 2^emax for both formats
    floor_b = np.array([O.e8m0_byte_mode(float(a), mode & ~O.SCALE_ROUND_UP) for a in amax])
    normal = (bits >> 7) > 0
    up = np.array([O.e8m0_byte_mode(float(a), mode | O.SCALE_ROUND_UP) for a in amax])
    sel = normal & (floor_b > 0)
    inc = ((bits & 0x7F) > 0x60).astype(np.int64)
    assert np.array_equal(up[sel].astype(np.int64), floor_b[sel].astype(np.int64) + inc[sel])


def test_scale_rule_specials():
    for mode in MODES:
        assert O.e8m0_byte_mode(0.0, mode) == 0
        assert O.e8m0_byte_mode(float("inf"), mode) == 0xFF
        assert O.e8m0_byte_mode(float("nan"), mode) == 0xFF
    assert O.e8m0_byte_mode(1.0, 0) == O.e8m0_byte(1.0) == 119
    assert O.e8m0_byte_mode(2.0 ** 200, O.SCALE_ROUND_UP) == 254      # clamp
    assert O.e8m0_byte_mode(2.0 ** 200 * 1.8, O.ELEM_E5M2) == 254


def load_variant_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "mx_variant_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tag, mode, xin, s, q = [f.strip() for f in line.split("|")]
        rows.append((tag, int(mode), [int(h, 16) for h in xin.split(",")], int(s, 16),
                     [int(h, 16) for h in q.split(",")]))
    return rows


@pytest.mark.parametrize("tag,mode,xin,scale,codes", load_variant_golden())
def test_golden_variant_block(tag, mode, xin, scale, codes):
    bits = np.zeros(32, np.uint16)
    bits[:len(xin)] = xin
    vals = [O.bf16_value(int(b)) for b in bits]
    q, s = O.mx_block(vals, mode=mode)
    assert s == scale, tag
    want = np.zeros(32, np.uint8)
    want[:len(codes)] = codes
    assert list(q) == list(want), tag
    # the same block through the tensor path, row-wise and column-wise
    x = np.zeros((32, 32), np.uint16)
    x[0] = bits
    r = O.mx_quantize(x, axis=O.ROWWISE | mode)
    c = O.mx_quantize(np.ascontiguousarray(x.T), axis=O.COLWISE | mode)
    assert r["s_row"][0, 0] == scale and c["s_col"][0, 0] == scale
    assert np.array_equal(r["q_row"][0], want) and np.array_equal(c["q_col"][0], want)


def torch_mx_rows(bits, mode):
    """Independent row-wise MX cast from torch primitives."""
    emax, vmax, dt = fmt(mode)
    x = torch.from_numpy(bits.astype(np.int32)).to(torch.int16).view(torch.bfloat16).double()
    M, K = x.shape
    blk = x.view(M, K // 32, 32)
    amax = blk.abs().amax(-1)
    if mode & O.SCALE_ROUND_UP:
        e = torch.ceil(torch.log2(amax / vmax))
    else:
        e = torch.floor(torch.log2(amax)) - emax
    byte = torch.where(amax == 0, torch.zeros_like(e), torch.clamp(e + 127, 0, 254))
    X = torch.pow(2.0, byte - 127).unsqueeze(-1)
    v = (blk / X).float().clamp(-vmax, vmax)
    q = v.to(dt).view(torch.uint8).reshape(M, K).numpy()
    return q, byte.to(torch.uint8).numpy()


@pytest.mark.parametrize("mode", MODES[1:])
@pytest.mark.parametrize("case", ["special", "loguniform", "normal", "tiny"])
def test_variant_tensor_matches_torch_pipeline(case, mode):
    if case == "special":
        x = W.special_256x512()
    elif case == "loguniform":
        x = W.loguniform_rows(96, 224, seed=7)
    elif case == "normal":
        x = W.normal(64, 160, seed=8, sigma=3.0)
    else:
        x = W.bf16_bits(np.random.default_rng(9).standard_normal((32, 64)).astype(np.float32)
                        * np.float32(1e-38))
    out = O.mx_quantize(x, axis=O.ROWWISE | O.COLWISE | mode)
    q, s = torch_mx_rows(x, mode)
    assert np.array_equal(out["s_row"], s) and np.array_equal(out["q_row"], q)
    qt, st = torch_mx_rows(np.ascontiguousarray(x.T), mode)
    assert np.array_equal(out["s_col"], st) and np.array_equal(out["q_col"], qt)


def test_round_up_never_saturates_and_floor_does():
    x = W.loguniform_rows(128, 256, seed=10)
    xv = W.bf16_to_f32(x).astype(np.float64)
    for mode in MODES:
        _, vmax, dt = fmt(mode)
        out = O.mx_quantize(x, axis=O.ROWWISE | mode)
        X = np.repeat(2.0 ** (out["s_row"].astype(np.float64) - 127), 32, axis=1)
        v = xv / X
        sat = np.abs(v) > vmax
        if mode & O.SCALE_ROUND_UP:
            assert not sat.any()
        else:
            assert sat.mean() > 0.001
        dq = torch.from_numpy(out["q_row"]).view(dt).double().numpy()
        assert np.all(np.abs(dq) <= vmax)


def test_variant_nonfinite_block_and_enum():
    x = np.zeros((32, 64), np.uint16)
    x[0, 3] = 0x7F80
    for mode in MODES:
        out = O.mx_quantize(x, axis=O.ROWWISE | O.COLWISE | mode)
        assert out["s_row"][0, 0] == 0xFF and np.all(out["q_row"][0, :32] == 0x7F)
        assert out["s_col"][3, 0] == 0xFF and np.all(out["q_col"][3, :] == 0x7F)
    with pytest.raises(ValueError):
        O.mx_quantize(x, axis=0x23)
    for act in (O.GATED_SWIGLU, O.GATED_GEGLU):
        g = O.mx_quantize_gated(np.zeros((32, 64), np.uint16), act, axis=3 | O.ELEM_E5M2)
        assert np.all(g["s_row"] == 0) and np.all(g["q_row"] == 0)


def test_variants_compose_with_fusions():
    """A fused variant cast equals the variant cast of the fused bf16 tensor."""
    x, g = W.make("c3_gelu_dbias_8192", 64, 96)
    for mode in MODES[1:]:
        for fusion in (O.FUSE_GELU, O.FUSE_DGELU | O.FUSE_DBIAS):
            f = O.mx_quantize(x, grad=g, fusion=fusion, axis=3 | mode, want_y=True)
            p = O.mx_quantize(f["y"], axis=3 | mode)
            for k in ("q_row", "s_row", "q_col", "s_col"):
                assert np.array_equal(f[k], p[k]), (mode, fusion, k)
