"""CPU oracle for block-scaled quantisation (MXFP8 and NVFP4) -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The product path (block_scaled_precision_bf16_amd) never does,
and this package never imports it.

All arrays are numpy: bf16 tensors are uint16 bit patterns, E4M3 / E8M0 /
packed-E2M1 outputs are uint8.  The arithmetic lives in mx_oracle.c; this file
only marshals arguments.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64

FUSE_NONE, FUSE_GELU, FUSE_DGELU, FUSE_DSILU, FUSE_DBIAS = 0, 1, 2, 3, 0x10
GATED_SWIGLU, GATED_GEGLU = 1, 2
ROWWISE, COLWISE = 1, 2
ELEM_E5M2, SCALE_ROUND_UP = 4, 8     # variant flags OR-ed into axis (MXFP8 only)
SCALE_TILED = 16                     # GEMM-ready (MFMA tile) scale layout flag


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        L = ctypes.CDLL(LIB)
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e2m1_encode.argtypes = [ctypes.c_double]
        L.orc_e8m0_byte.restype = ctypes.c_uint8
        L.orc_e8m0_byte.argtypes = [ctypes.c_double]
        L.orc_e8m0_byte_mode.restype = ctypes.c_uint8
        L.orc_e8m0_byte_mode.argtypes = [ctypes.c_double, ctypes.c_uint]
        L.orc_e5m2_value.restype = ctypes.c_double
        L.orc_e5m2_value.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_encode.restype = ctypes.c_uint8
        L.orc_e5m2_encode.argtypes = [ctypes.c_double]
        L.orc_mx_block_mode.restype = None
        L.orc_mx_block_mode.argtypes = [_f64p, ctypes.c_int, _u8p, _i64, _u8p, ctypes.c_uint]
        L.orc_e5m2_encode_array.restype = None
        L.orc_e5m2_encode_array.argtypes = [_f64p, _u8p, _i64]
        L.orc_tiled_scale_bytes.restype = ctypes.c_int64
        L.orc_tiled_scale_bytes.argtypes = [_i64, _i64]
        L.orc_scale_tiles.restype = None
        L.orc_scale_tiles.argtypes = [_u8p, _i64, _i64, _u8p]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
        L.orc_mx_block.restype = None
        L.orc_mx_block.argtypes = [_f64p, ctypes.c_int, _u8p, _i64, _u8p]
        L.orc_exp32.restype = ctypes.c_float
        L.orc_exp32.argtypes = [ctypes.c_float]
        for f in ("orc_gelu32", "orc_dgelu32", "orc_silu32", "orc_dsilu32"):
            getattr(L, f).restype = ctypes.c_float
            getattr(L, f).argtypes = [ctypes.c_float]
        L.orc_preop.restype = ctypes.c_uint16
        L.orc_preop.argtypes = [ctypes.c_int, ctypes.c_uint16, ctypes.c_uint16]
        L.orc_gated.restype = ctypes.c_uint16
        L.orc_gated.argtypes = [ctypes.c_int, ctypes.c_uint16, ctypes.c_uint16]
        L.orc_mx_quantize.restype = ctypes.c_int
        L.orc_mx_quantize.argtypes = [_u16p, _u16p, _i64, _i64, ctypes.c_uint, ctypes.c_int,
                                      _u8p, _u8p, _u8p, _u8p, _f32p, _u16p]
        L.orc_gated_bwd.restype = ctypes.c_int
        L.orc_gated_bwd.argtypes = [ctypes.c_int, ctypes.c_uint16, ctypes.c_uint16,
                                    ctypes.c_uint16, _u16p, _u16p]
        L.orc_mx_quantize_dgated.restype = ctypes.c_int
        L.orc_mx_quantize_dgated.argtypes = [_u16p, _u16p, _i64, _i64, ctypes.c_uint,
                                             ctypes.c_int, _u8p, _u8p, _u8p, _u8p, _u16p]
        L.orc_mx_quantize_grouped.restype = ctypes.c_int
        L.orc_mx_quantize_grouped.argtypes = [_u16p, _u16p, _i64, ctypes.POINTER(ctypes.c_int64),
                                              ctypes.c_int, ctypes.c_uint, ctypes.c_int,
                                              _u8p, _u8p, _u8p, _u8p, _f32p]
        L.orc_mx_quantize_gated_grouped.restype = ctypes.c_int
        L.orc_mx_quantize_gated_grouped.argtypes = [_u16p, _u16p, _i64,
                                                    ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                                    ctypes.c_uint, ctypes.c_int, _u8p, _u8p, _u8p,
                                                    _u8p]
        L.orc_mx_quantize_gated.restype = ctypes.c_int
        L.orc_mx_quantize_gated.argtypes = [_u16p, _i64, _i64, ctypes.c_uint, ctypes.c_int,
                                            _u8p, _u8p, _u8p, _u8p, _u16p]
        L.orc_nvfp4_quantize_transpose_2d.restype = ctypes.c_int
        L.orc_nvfp4_quantize_transpose_2d.argtypes = [_u16p, _i64, _i64, ctypes.c_uint,
                                                      ctypes.c_float, _u8p, _u8p, _u8p, _u8p,
                                                      _f32p]
        L.orc_nvfp4_quantize_transpose_grouped.restype = ctypes.c_int
        L.orc_nvfp4_quantize_transpose_grouped.argtypes = [
            _u16p, _i64, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, _f32p, ctypes.c_int,
            ctypes.c_uint, _u8p, _u8p, _u8p, _u8p, _f32p]
        L.orc_absmax.restype = ctypes.c_float
        L.orc_absmax.argtypes = [_u16p, _i64]
        L.orc_nvfp4_global_scale.restype = ctypes.c_float
        L.orc_nvfp4_global_scale.argtypes = [ctypes.c_float]
        L.orc_nvfp4_quantize_transpose.restype = ctypes.c_int
        L.orc_nvfp4_quantize_transpose.argtypes = [_u16p, _i64, _i64, ctypes.c_uint,
                                                   ctypes.c_float, _u8p, _u8p, _u8p, _u8p,
                                                   _f32p]
        L.orc_e4m3_encode_array.restype = None
        L.orc_e4m3_encode_array.argtypes = [_f64p, _u8p, _i64]
        L.orc_e2m1_encode_array.restype = None
        L.orc_e2m1_encode_array.argtypes = [_f64p, _u8p, _i64]
        L.orc_bf16_round_array.restype = None
        L.orc_bf16_round_array.argtypes = [_f64p, _u16p, _i64]
        L.orc_unary32_array.restype = None
        L.orc_unary32_array.argtypes = [ctypes.c_int, _f32p, _f32p, _i64]
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_get_threads.restype = ctypes.c_int
        L.orc_get_threads.argtypes = []
        L.orc_init()
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


_CHECKS = {"bf16_round": ctypes.POINTER(ctypes.c_uint16), "e2m1": _u8p, "e4m3": _u8p,
           "exp32": ctypes.POINTER(ctypes.c_uint32)}


def check_range(which: str, got: np.ndarray, first: int):
    """Compare device results for the fp32 patterns first, first + 1, ...
    with the oracle's rule `which` (bf16_round, e2m1, e4m3, exp32).  got holds
    one result per input (e2m1: one byte per input pair).  Returns (number of
    differing inputs, first differing input index or -1)."""
    fn = getattr(lib(), "orc_check_" + which)
    fn.restype = ctypes.c_int64
    fn.argtypes = [_CHECKS[which], ctypes.c_uint64, ctypes.c_int64,
                   ctypes.POINTER(ctypes.c_int64)]
    got = np.ascontiguousarray(got)
    n = got.size * (2 if which == "e2m1" else 1)
    fb = ctypes.c_int64()
    bad = fn(got.ctypes.data_as(_CHECKS[which]), first, n, ctypes.byref(fb))
    return int(bad), int(fb.value)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return lib().orc_get_threads()


# --- scalar codecs (exact decoders, nearest-value encoders) -------------------

def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(b)


def bf16_round(v: float) -> int:
    return lib().orc_bf16_round(v)


def e4m3_value(c: int) -> float:
    return lib().orc_e4m3_value(c)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def e2m1_value(c: int) -> float:
    return lib().orc_e2m1_value(c)


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(v)


def e8m0_byte(amax: float) -> int:
    return lib().orc_e8m0_byte(amax)


def e8m0_byte_mode(amax: float, mode: int) -> int:
    """E8M0 byte under the variant flags (ELEM_E5M2, SCALE_ROUND_UP)."""
    return lib().orc_e8m0_byte_mode(amax, mode)


def e5m2_value(c: int) -> float:
    return lib().orc_e5m2_value(c)


def e5m2_encode(v: float) -> int:
    return lib().orc_e5m2_encode(v)


def e5m2_encode_array(v) -> np.ndarray:
    v = _c(np.asarray(v, dtype=np.float64), np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e5m2_encode_array(_p(v, _f64p), _p(out, _u8p), v.size)
    return out


def e8m0_value(b: int) -> float:
    return lib().orc_e8m0_value(b)


def tiled_scale_bytes(R: int, C: int) -> int:
    return lib().orc_tiled_scale_bytes(R, C)


def scale_tiles(s) -> np.ndarray:
    """Compact scales s[R][C] -> the flat tiled (GEMM-ready) layout."""
    s = _c(s, np.uint8)
    R, C = s.shape
    out = np.empty(tiled_scale_bytes(R, C), np.uint8)
    lib().orc_scale_tiles(_p(s, _u8p), R, C, _p(out, _u8p))
    return out


def _scales(axis, rows, blocks):
    """Output buffer for one direction's scales: [rows][blocks], or flat tiled."""
    if axis & SCALE_TILED:
        return np.zeros(tiled_scale_bytes(rows, blocks), np.uint8)
    return np.zeros((rows, blocks), np.uint8)


def e4m3_encode_array(v) -> np.ndarray:
    v = _c(np.asarray(v, dtype=np.float64), np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(v, _f64p), _p(out, _u8p), v.size)
    return out


def e2m1_encode_array(v) -> np.ndarray:
    v = _c(np.asarray(v, dtype=np.float64), np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e2m1_encode_array(_p(v, _f64p), _p(out, _u8p), v.size)
    return out


def bf16_round_array(v) -> np.ndarray:
    v = _c(np.asarray(v, dtype=np.float64), np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_round_array(_p(v, _f64p), _p(out, _u16p), v.size)
    return out


def mx_block(values, mode=0):
    """One MX block: exact values -> (element codes, E8M0 byte); mode holds the
    variant flags (ELEM_E5M2, SCALE_ROUND_UP), 0 = E4M3 with the floor rule."""
    v = _c(np.asarray(values, dtype=np.float64), np.float64)
    q = np.empty(v.size, np.uint8)
    s = np.empty(1, np.uint8)
    if mode:
        lib().orc_mx_block_mode(_p(v, _f64p), v.size, _p(q, _u8p), 1, _p(s, _u8p), mode)
    else:
        lib().orc_mx_block(_p(v, _f64p), v.size, _p(q, _u8p), 1, _p(s, _u8p))
    return q, int(s[0])


# --- fused pre-op arithmetic (fp32 sequences) ---------------------------------

_UNARY = {"exp": 0, "gelu": 1, "dgelu": 2, "silu": 3, "dsilu": 4}


def unary32(which: str, v) -> np.ndarray:
    v = _c(np.asarray(v, dtype=np.float32), np.float32)
    out = np.empty(v.shape, np.float32)
    lib().orc_unary32_array(_UNARY[which], _p(v, _f32p), _p(out, _f32p), v.size)
    return out


def preop(pre: int, x: int, grad: int = 0) -> int:
    return lib().orc_preop(pre, x, grad)


def gated(act: int, gate: int, lin: int) -> int:
    return lib().orc_gated(act, gate, lin)


def gated_bwd(act: int, gate: int, lin: int, grad: int):
    """(d_gate, d_lin) bf16 bits of the gated backward for one element pair."""
    dg, dl = ctypes.c_uint16(), ctypes.c_uint16()
    rc = lib().orc_gated_bwd(act, gate, lin, grad, ctypes.byref(dg), ctypes.byref(dl))
    if rc != 0:
        raise ValueError(f"oracle gated_bwd failed with code {rc}")
    return dg.value, dl.value


# --- tensor entry points --------------------------------------------------------

def mx_quantize(x, grad=None, axis=ROWWISE | COLWISE, fusion=FUSE_NONE, want_y=False):
    """MXFP8 cast of bf16 bits x[M][K]. Returns dict of numpy outputs."""
    x = _c(x, np.uint16)
    M, K = x.shape
    g = _c(grad, np.uint16) if grad is not None else None
    out = {}
    q_row = np.zeros((M, K), np.uint8) if axis & ROWWISE else None
    s_row = _scales(axis, M, -(-K // 32)) if axis & ROWWISE else None
    q_col = np.zeros((K, M), np.uint8) if axis & COLWISE else None
    s_col = _scales(axis, K, -(-M // 32)) if axis & COLWISE else None
    dbias = np.zeros(K, np.float32) if fusion & FUSE_DBIAS else None
    y = np.zeros((M, K), np.uint16) if want_y else None
    rc = lib().orc_mx_quantize(_p(x, _u16p), _p(g, _u16p), M, K, axis, fusion,
                               _p(q_row, _u8p), _p(s_row, _u8p), _p(q_col, _u8p),
                               _p(s_col, _u8p), _p(dbias, _f32p), _p(y, _u16p))
    if rc != 0:
        raise ValueError(f"oracle mx_quantize failed with code {rc}")
    out.update(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col, dbias=dbias, y=y)
    return out


def _scale_len(rows, cols, axis):
    if rows == 0:
        return 0
    blocks = -(-cols // 32)
    return tiled_scale_bytes(rows, blocks) if axis & SCALE_TILED else rows * blocks


def mx_quantize_grouped(x, group_rows, grad=None, axis=ROWWISE | COLWISE, fusion=FUSE_NONE):
    """Grouped MXFP8 cast: x[M][K] stacks len(group_rows) tensors along rows.
    Returns flat per-group-concatenated s_row / q_col / s_col, q_row[M][K] and
    dbias[G][K]."""
    x = _c(x, np.uint16)
    M, K = x.shape
    rows = np.ascontiguousarray(group_rows, dtype=np.int64)
    G = rows.size
    assert rows.sum() == M
    g = _c(grad, np.uint16) if grad is not None else None
    sr = sum(_scale_len(int(m), K, axis) for m in rows)
    sc = sum(_scale_len(K, int(m), axis) for m in rows)
    q_row = np.zeros((M, K), np.uint8) if axis & ROWWISE else None
    s_row = np.zeros(sr, np.uint8) if axis & ROWWISE else None
    q_col = np.zeros(K * M, np.uint8) if axis & COLWISE else None
    s_col = np.zeros(sc, np.uint8) if axis & COLWISE else None
    dbias = np.zeros((G, K), np.float32) if fusion & FUSE_DBIAS else None
    rc = lib().orc_mx_quantize_grouped(_p(x, _u16p), _p(g, _u16p), K,
                                       rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), G,
                                       axis, fusion, _p(q_row, _u8p), _p(s_row, _u8p),
                                       _p(q_col, _u8p), _p(s_col, _u8p), _p(dbias, _f32p))
    if rc != 0:
        raise ValueError(f"oracle mx_quantize_grouped failed with code {rc}")
    return dict(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col, dbias=dbias)


def mx_quantize_gated_grouped(x, group_rows, act, axis=ROWWISE | COLWISE, grad=None):
    """Grouped gated cast: x[M][2N] = [gate | linear] stacked by group; with
    grad ([M][N]) the gated backward.  Flat per-group-concatenated outputs
    (q_row [M][W], W = N forward or 2N backward)."""
    x = _c(x, np.uint16)
    M, N2 = x.shape
    N = N2 // 2
    rows = np.ascontiguousarray(group_rows, dtype=np.int64)
    assert rows.sum() == M
    g = _c(grad, np.uint16) if grad is not None else None
    W = N2 if grad is not None else N
    sr = sum(_scale_len(int(m), W, axis) for m in rows)
    sc = sum(_scale_len(W, int(m), axis) for m in rows)
    q_row = np.zeros((M, W), np.uint8) if axis & ROWWISE else None
    s_row = np.zeros(sr, np.uint8) if axis & ROWWISE else None
    q_col = np.zeros(W * M, np.uint8) if axis & COLWISE else None
    s_col = np.zeros(sc, np.uint8) if axis & COLWISE else None
    rc = lib().orc_mx_quantize_gated_grouped(_p(g, _u16p), _p(x, _u16p), N,
                                             rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                             rows.size, axis, act, _p(q_row, _u8p), _p(s_row, _u8p),
                                             _p(q_col, _u8p), _p(s_col, _u8p))
    if rc != 0:
        raise ValueError(f"oracle mx_quantize_gated_grouped failed with code {rc}")
    return dict(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col)


def mx_quantize_gated(x, act, axis=ROWWISE | COLWISE, want_y=False):
    """Gated MXFP8 cast of x[M][2N] = [gate | linear]."""
    x = _c(x, np.uint16)
    M, N2 = x.shape
    N = N2 // 2
    q_row = np.zeros((M, N), np.uint8) if axis & ROWWISE else None
    s_row = _scales(axis, M, -(-N // 32)) if axis & ROWWISE else None
    q_col = np.zeros((N, M), np.uint8) if axis & COLWISE else None
    s_col = _scales(axis, N, -(-M // 32)) if axis & COLWISE else None
    y = np.zeros((M, N), np.uint16) if want_y else None
    rc = lib().orc_mx_quantize_gated(_p(x, _u16p), M, N, axis, act, _p(q_row, _u8p),
                                     _p(s_row, _u8p), _p(q_col, _u8p), _p(s_col, _u8p),
                                     _p(y, _u16p))
    if rc != 0:
        raise ValueError(f"oracle mx_quantize_gated failed with code {rc}")
    return dict(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col, y=y)


def mx_quantize_dgated(grad, x, act, axis=ROWWISE | COLWISE, want_y=False):
    """Gated backward MXFP8 cast: grad[M][N], x[M][2N] = [gate | linear]; the
    quantised tensor is dx[M][2N] = [d_gate | d_lin]."""
    grad = _c(grad, np.uint16)
    x = _c(x, np.uint16)
    M, N2 = x.shape
    N = N2 // 2
    assert grad.shape == (M, N)
    q_row = np.zeros((M, N2), np.uint8) if axis & ROWWISE else None
    s_row = _scales(axis, M, -(-N2 // 32)) if axis & ROWWISE else None
    q_col = np.zeros((N2, M), np.uint8) if axis & COLWISE else None
    s_col = _scales(axis, N2, -(-M // 32)) if axis & COLWISE else None
    y = np.zeros((M, N2), np.uint16) if want_y else None
    rc = lib().orc_mx_quantize_dgated(_p(grad, _u16p), _p(x, _u16p), M, N, axis, act,
                                      _p(q_row, _u8p), _p(s_row, _u8p), _p(q_col, _u8p),
                                      _p(s_col, _u8p), _p(y, _u16p))
    if rc != 0:
        raise ValueError(f"oracle mx_quantize_dgated failed with code {rc}")
    return dict(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col, y=y)


def absmax(x) -> float:
    x = _c(x, np.uint16)
    return lib().orc_absmax(_p(x, _u16p), x.size)


def nvfp4_global_scale(A: float) -> float:
    return lib().orc_nvfp4_global_scale(A)


def nvfp4_quantize_transpose(x, axis=ROWWISE | COLWISE, tensor_amax=None, two_d=False):
    """NVFP4 of x[M][K] and of its transpose. tensor_amax overrides max|x|.
    two_d: one scale per 16 x 16 block (written per row / per column)."""
    x = _c(x, np.uint16)
    M, K = x.shape
    q_row = np.zeros((M, -(-K // 2)), np.uint8) if axis & ROWWISE else None
    s_row = np.zeros((M, -(-K // 16)), np.uint8) if axis & ROWWISE else None
    q_col = np.zeros((K, -(-M // 2)), np.uint8) if axis & COLWISE else None
    s_col = np.zeros((K, -(-M // 16)), np.uint8) if axis & COLWISE else None
    sg = np.zeros(1, np.float32)
    A = -1.0 if tensor_amax is None else float(tensor_amax)
    fn = lib().orc_nvfp4_quantize_transpose_2d if two_d else lib().orc_nvfp4_quantize_transpose
    rc = fn(_p(x, _u16p), M, K, axis, A, _p(q_row, _u8p), _p(s_row, _u8p), _p(q_col, _u8p),
            _p(s_col, _u8p), _p(sg, _f32p))
    if rc != 0:
        raise ValueError(f"oracle nvfp4_quantize_transpose failed with code {rc}")
    return dict(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col, sg=float(sg[0]))


def nvfp4_quantize_transpose_grouped(x, group_rows, axis=ROWWISE | COLWISE, amax=None, two_d=False):
    """Grouped NVFP4: x[M][K] stacks len(group_rows) tensors along rows, each
    with its own tensor amax (amax[g], or its own max |x|) and global scale."""
    x = _c(x, np.uint16)
    M, K = x.shape
    rows = np.ascontiguousarray(group_rows, dtype=np.int64)
    G = rows.size
    assert rows.sum() == M
    q_row = np.zeros((M, -(-K // 2)), np.uint8) if axis & ROWWISE else None
    s_row = np.zeros((M, -(-K // 16)), np.uint8) if axis & ROWWISE else None
    q_col = np.zeros(K * int(sum(-(-int(m) // 2) for m in rows)), np.uint8) if axis & COLWISE else None
    s_col = np.zeros(K * int(sum(-(-int(m) // 16) for m in rows)), np.uint8) if axis & COLWISE else None
    sg = np.zeros(G, np.float32)
    a = None if amax is None else _c(np.asarray(amax, dtype=np.float32), np.float32)
    rc = lib().orc_nvfp4_quantize_transpose_grouped(
        _p(x, _u16p), K, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), G, _p(a, _f32p),
        int(two_d), axis, _p(q_row, _u8p), _p(s_row, _u8p), _p(q_col, _u8p), _p(s_col, _u8p),
        _p(sg, _f32p))
    if rc != 0:
        raise ValueError(f"oracle nvfp4_quantize_transpose_grouped failed with code {rc}")
    return dict(q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col, sg=sg)
