"""Pins for the oracle's fused pre-op arithmetic (CPU only).

The fp32 sequences (own exp, logistic form of tanh-GELU) are a reading: the
pages name gelu / dgelu / swiglu / geglu fusions (tables "MXFP8 generic
quantize kernel", "MXFP8 gated (swiglu / geglu) kernel") but fix no
arithmetic.  They are pinned here against float64 closed forms written the
textbook way (tanh, 1/(1+exp)), against a finite difference for the
derivative, and by the compositions the fused casts rely on.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W

K0_32 = float(np.float32(math.sqrt(2.0 / math.pi)))
K1_32 = float(np.float32(0.044715))


def all_finite_bf16_f32():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    return W.bf16_to_f32(bits)


def one_plus_tanh(u):
    """1 + tanh(u) in float64 without cancellation: for u < 0 use
    2 e^(2u) / (1 + e^(2u))."""
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(2.0 * np.minimum(u, 0.0))
        return np.where(u >= 0, 1.0 + np.tanh(u), 2.0 * e / (1.0 + e))


def one_minus_tanh_sq(u):
    """1 - tanh(u)^2 = 4 e^(-2|u|) / (1 + e^(-2|u|))^2, cancellation free."""
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(-2.0 * np.abs(u))
        return 4.0 * e / (1.0 + e) ** 2


def gelu64(x, k0=math.sqrt(2 / math.pi), k1=0.044715):
    """tanh-form GELU 0.5 x (1 + tanh(k0 (x + k1 x^3))) in float64."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        u = k0 * (x + k1 * x ** 3)
        return 0.5 * x * one_plus_tanh(u)


def dgelu64(x, k0=math.sqrt(2 / math.pi), k1=0.044715):
    """Its derivative 0.5 (1 + t) + 0.5 x (1 - t^2) k0 (1 + 3 k1 x^2)."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        u = k0 * (x + k1 * x ** 3)
        d = 0.5 * one_plus_tanh(u) + 0.5 * x * one_minus_tanh_sq(u) * k0 * (1 + 3 * k1 * x * x)
    return np.where(np.isfinite(d), d, np.where(x > 0, 1.0, 0.0))


def cond_ulps(x):
    """Error budget in fp32 ulps: a few roundings, plus the amplification of
    u's rounding (about 3 ulps relative) by e^(2u), i.e. 3 |2u|."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        u = K0_32 * (x + K1_32 * x ** 3)
    return 8.0 + 3.0 * np.abs(2.0 * u)


def silu64(x):
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def ulp32(v):
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 23)


def test_exp32_accuracy_and_range():
    a = np.linspace(-103.0, 88.72, 2_000_001).astype(np.float32)
    got = O.unary32("exp", a).astype(np.float64)
    want = np.exp(a.astype(np.float64))
    normal = want >= 2.0 ** -126
    err = np.abs(got - want)[normal] / ulp32(want[normal])
    assert err.max() <= 2.0, err.max()
    # subnormal results: within one unit of the least subnormal
    assert np.all(np.abs(got - want)[~normal] <= 2.0 ** -149)
    assert O.unary32("exp", [0.0])[0] == 1.0
    assert np.isfinite(O.unary32("exp", [88.72283172607421875])[0])
    assert np.isinf(O.unary32("exp", [88.7228393554687])[0])
    assert O.unary32("exp", [-104.5])[0] == 0.0


def test_gelu32_against_tanh_form():
    x = all_finite_bf16_f32()
    got = O.unary32("gelu", x).astype(np.float64)
    want = gelu64(x, K0_32, K1_32)                 # same constants, tanh route
    fin = np.isfinite(want)
    assert np.all(np.isfinite(got[fin]))
    err = np.abs(got - want)[fin]
    tol = cond_ulps(x[fin]) * ulp32(want[fin]) + 2.0 ** -148
    assert np.all(err <= tol), (x[fin][err > tol][:5], got[fin][err > tol][:5], want[fin][err > tol][:5])
    # the fp32 constants cost at most ~1e-5 relative against the exact ones
    mid = np.abs(x) < 8
    rel = np.abs(got[mid] - gelu64(x[mid])) / np.maximum(np.abs(gelu64(x[mid])), 1e-30)
    assert np.all(rel[np.abs(gelu64(x[mid])) > 1e-30] < 1e-5)
    # rounded to bf16 (what the fused casts quantise), the fp32 sequence gives
    # the bf16 rounding of the float64 function on every finite bf16 input,
    # with the exact constants as well as with their fp32 roundings
    gb = O.bf16_round_array(got)
    assert np.array_equal(gb, O.bf16_round_array(want))
    assert np.array_equal(gb, O.bf16_round_array(gelu64(x)))


def test_dgelu32_against_analytic_derivative():
    x = all_finite_bf16_f32()
    got = O.unary32("dgelu", x).astype(np.float64)
    want = dgelu64(x, K0_32, K1_32)
    err = np.abs(got - want)
    # gelu' has a zero near x = -0.75 where its two O(1) terms cancel, so the
    # budget also allows a few ulps of 1 in absolute terms
    tol = cond_ulps(x) * ulp32(want) + 16 * 2.0 ** -24
    assert np.all(err <= tol), (x[err > tol][:5], got[err > tol][:5], want[err > tol][:5])
    away = np.abs(want) > 0.05
    assert np.all(err[away] <= cond_ulps(x[away]) * ulp32(want[away]) * 4)


def test_dgelu_analytic_form_is_the_derivative_of_gelu():
    x = np.linspace(-6, 6, 4001)
    h = 1e-6
    fd = (gelu64(x + h) - gelu64(x - h)) / (2 * h)
    assert np.max(np.abs(fd - dgelu64(x))) < 1e-8


def test_silu32_against_closed_form():
    x = all_finite_bf16_f32()
    got = O.unary32("silu", x).astype(np.float64)
    want = silu64(x)
    err = np.abs(got - want)
    tol = (8.0 + 2.0 * np.abs(x)) * ulp32(want) + 2.0 ** -148
    assert np.all(err <= tol), (x[err > tol][:5], got[err > tol][:5], want[err > tol][:5])
    # rounded to bf16: the bf16 rounding of the float64 function, everywhere
    assert np.array_equal(O.bf16_round_array(got), O.bf16_round_array(want))


@pytest.mark.parametrize("which,ref", [("dgelu", "dgelu64"), ("dsilu", "dsilu64")])
def test_derivatives_rounded_to_bf16(which, ref):
    """gelu' and silu' rounded to bf16 equal the bf16 rounding of the float64
    derivative on every finite bf16 input, but for two kinds of input:
      - deep in the negative tail, where the derivative is a tiny negative
        number (|d| below half the least bf16 subnormal, so float64 rounds it
        to -0): the fp32 sequence gives +0 there, because its second term is
        taken as 0 once sigma (1 - sigma) underflows;
      - exactly one input each where the exact derivative lies a few fp32
        ulps from the midpoint of two bf16 values, closer than the fp32
        sequence's error budget (the fp32 result lands on or just before the
        midpoint, the float64 value just past it); the two differ by one
        bf16 ulp."""
    x = all_finite_bf16_f32()
    got = O.unary32(which, x).astype(np.float64)
    want = globals()[ref](x)
    gb, wb = O.bf16_round_array(got), O.bf16_round_array(want)
    diff = gb != wb
    zero = diff & (gb == 0) & (wb == 0x8000)
    assert np.all(x[zero] < 0) and np.all(np.abs(want[zero]) < 2.0 ** -134)
    rest = np.flatnonzero(diff & ~zero)
    assert rest.size == 1, x[rest][:8]
    i = rest[0]
    assert abs(int(gb[i]) - int(wb[i])) == 1
    mid = (O.bf16_value(int(gb[i])) + O.bf16_value(int(wb[i]))) / 2
    budget = 64 * ulp32(mid)
    assert abs(got[i] - mid) <= budget and abs(want[i] - mid) <= budget, (x[i], got[i], want[i])


def test_special_values():
    g = O.unary32("gelu", [0.0, -0.0, 1e30, -1e30, 3.0e38, -3.0e38])
    assert list(g[:2]) == [0.0, 0.0] and g[2] == np.float32(1e30) and g[4] == np.float32(3e38)
    assert g[3] == 0.0 and np.signbit(g[3]) and g[5] == 0.0
    d = O.unary32("dgelu", [0.0, 1e30, -1e30, 3e38])
    assert list(d) == [0.5, 1.0, 0.0, 1.0]
    s = O.unary32("silu", [0.0, 1e30, -1e30])
    assert s[0] == 0.0 and s[1] == np.float32(1e30) and s[2] == 0.0


def test_preop_and_gated_compositions():
    rng = np.random.default_rng(21)
    xs = W.bf16_bits(rng.standard_normal(2000).astype(np.float32) * 3)
    one, two = 0x3F80, 0x4000
    for x in xs[:500]:
        x = int(x)
        xf = O.bf16_value(x)
        g = float(O.unary32("gelu", [xf])[0])
        assert O.preop(O.FUSE_GELU, x) == O.bf16_round(g)
        d = float(O.unary32("dgelu", [xf])[0])
        assert O.preop(O.FUSE_DGELU, x, one) == O.bf16_round(d)
        assert O.preop(O.FUSE_NONE, x) == x
        s = float(O.unary32("silu", [xf])[0])
        # linear = 1 leaves act(gate): gate and linear are not swapped
        assert O.gated(O.GATED_SWIGLU, x, one) == O.bf16_round(s)
        assert O.gated(O.GATED_GEGLU, x, one) == O.bf16_round(g)
        # linear = 2 doubles exactly
        assert O.bf16_value(O.gated(O.GATED_SWIGLU, x, two)) == 2 * O.bf16_value(O.bf16_round(s))
        # gate = 0 gives +-0 whatever the linear half
        assert O.bf16_value(O.gated(O.GATED_SWIGLU, 0, x)) == 0.0


def test_fused_tensor_equals_plain_cast_of_fused_values():
    x, g = W.make("c3_gelu_dbias_8192", 64, 64)
    for fusion in (O.FUSE_GELU, O.FUSE_DGELU):
        f = O.mx_quantize(x, grad=g, fusion=fusion, want_y=True)
        p = O.mx_quantize(f["y"])
        for k in ("q_row", "s_row", "q_col", "s_col"):
            assert np.array_equal(f[k], p[k])
    xg = W.make("c4_gated_8192", 64, 128)
    for act in (O.GATED_SWIGLU, O.GATED_GEGLU):
        f = O.mx_quantize_gated(xg, act, want_y=True)
        p = O.mx_quantize(f["y"])
        for k in ("q_row", "s_row", "q_col", "s_col"):
            assert np.array_equal(f[k], p[k])
        # y[m][n] = act(x[m][n]) * x[m][N + n]
        m, n = 5, 17
        assert f["y"][m, n] == O.gated(act, int(xg[m, n]), int(xg[m, 64 + n]))


def dsilu64(x):
    """d/dx x sigma(x) = sigma(x) (1 + x (1 - sigma(x))), with sigma and
    1 - sigma from e^-|x| (no overflow, no cancellation)."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(-np.abs(x))
        s = np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
        sc = np.where(x >= 0, e / (1.0 + e), 1.0 / (1.0 + e))
        d = s * (1.0 + x * sc)
    return np.where(np.isfinite(d), d, np.where(x > 0, 1.0, 0.0))


def test_dsilu_closed_form_is_the_derivative_of_silu():
    x = np.linspace(-12, 12, 4801)
    h = 1e-6
    fd = (silu64(x + h) - silu64(x - h)) / (2 * h)
    assert np.max(np.abs(fd - dsilu64(x))) < 1e-8


def test_dsilu32_against_closed_form():
    x = all_finite_bf16_f32()
    got = O.unary32("dsilu", x).astype(np.float64)
    want = dsilu64(x)
    err = np.abs(got - want)
    # silu' has a zero near x = -1.28 where sigma and x sigma (1 - sigma)
    # cancel, hence the absolute term (a few ulps of 1)
    tol = (8.0 + 2.0 * np.abs(x)) * ulp32(want) + 16 * 2.0 ** -24
    assert np.all(err <= tol), (x[err > tol][:5], got[err > tol][:5], want[err > tol][:5])
    away = np.abs(want) > 0.05
    with np.errstate(over="ignore"):
        assert np.all(err[away] <= (8.0 + 2.0 * np.abs(x[away])) * ulp32(want[away]) * 4)
    d = O.unary32("dsilu", [0.0, 1e30, -1e30, 3e38])
    assert list(d) == [0.5, 1.0, 0.0, 1.0]


def test_dsilu_preop_and_gated_backward_compositions():
    rng = np.random.default_rng(22)
    v = W.bf16_bits(rng.standard_normal(1500).astype(np.float32) * 3)
    one = 0x3F80
    for i in range(500):
        gate, lin, dy = int(v[i]), int(v[500 + i]), int(v[1000 + i])
        gf, lf = O.bf16_value(gate), O.bf16_value(lin)
        ds = float(O.unary32("dsilu", [gf])[0])
        dg = float(O.unary32("dgelu", [gf])[0])
        # single-input dSiLU: grad = 1 leaves dsilu(x)
        assert O.preop(O.FUSE_DSILU, gate, one) == O.bf16_round(ds)
        for act, da, pre in ((O.GATED_SWIGLU, ds, O.FUSE_DSILU), (O.GATED_GEGLU, dg, O.FUSE_DGELU)):
            d_gate, d_lin = O.gated_bwd(act, gate, lin, dy)
            # d_lin = act(gate) * grad is the forward gated value with linear := grad
            assert d_lin == O.gated(act, gate, dy)
            # linear = 1: d_gate = act'(gate) * grad, the single-input backward
            assert O.gated_bwd(act, gate, one, dy)[0] == O.preop(pre, gate, dy)
            # grad = 1: d_gate = fl32(act'(gate) * linear), one fp32 rounding
            want = np.float32(np.float32(da) * np.float32(lf))
            assert O.gated_bwd(act, gate, lin, one)[0] == O.bf16_round(float(want))
            # gate = 0: act(0) = 0, so d_lin = +-0
            assert O.bf16_value(O.gated_bwd(act, 0, lin, dy)[1]) == 0.0


def test_backward_tensors_equal_plain_cast_of_their_values():
    x, g = W.make("c3_gelu_dbias_8192", 64, 64)
    f = O.mx_quantize(x, grad=g, fusion=O.FUSE_DSILU | O.FUSE_DBIAS, want_y=True)
    p = O.mx_quantize(f["y"])
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert np.array_equal(f[k], p[k])
    assert f["y"][3, 7] == O.preop(O.FUSE_DSILU, int(x[3, 7]), int(g[3, 7]))
    xg = W.make("c4_gated_8192", 64, 128)
    dy = W.normal(64, 64, seed=9)
    for act in (O.GATED_SWIGLU, O.GATED_GEGLU):
        f = O.mx_quantize_dgated(dy, xg, act, want_y=True)
        p = O.mx_quantize(f["y"])
        for k in ("q_row", "s_row", "q_col", "s_col"):
            assert np.array_equal(f[k], p[k])
        assert f["q_row"].shape == (64, 128) and f["s_col"].shape == (128, 2)
        # dx[m][n] = d_gate, dx[m][N + n] = d_lin of element pair n
        m, n = 5, 17
        d_gate, d_lin = O.gated_bwd(act, int(xg[m, n]), int(xg[m, 64 + n]), int(dy[m, n]))
        assert f["y"][m, n] == d_gate and f["y"][m, 64 + n] == d_lin
