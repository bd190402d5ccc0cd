"""C-ABI contract tests that need no GPU.

libmxcast.so loads on a machine without a GPU (the HIP runtime is only
initialised by a launch), exports every function include/mxcast.h declares,
and rejects every malformed call with its status code before touching any
memory.  The "device pointers" below are host buffers with canary bytes:
validation never dereferences them, so they must come back unchanged.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import block_scaled_precision_bf16_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxcast.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert set(header_functions()) == set(mx.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = mx.lib()
    for name in header_functions():
        assert hasattr(L, name), name


def header_abi_version():
    text = open(os.path.join(ROOT, "include", "mxcast.h")).read()
    return int(re.search(r"#define MXCAST_ABI_VERSION (\d+)", text).group(1))


def test_version_and_status_strings():
    assert mx.mx_abi_version() == header_abi_version() == 10
    for code in range(9):
        assert mx.mx_status_str(code).startswith("MX_")
    assert "unknown" in mx.mx_status_str(99)


def walks(M, K, target=512):
    """Workgroup walks along M: sub-tiles are 128 x 256; a walk takes the deepest
    power of two <= 16 sub-tiles that still leaves >= target workgroups (512
    for the plain cast and casts with dbias, 1024 for the other fused casts)."""
    tm, tk = -(-M // 128), -(-K // 256)
    g = 16
    while g > 1 and -(-tm // g) * tk < target:
        g //= 2
    return -(-tm // g)


def test_workspace_size():
    ws = mx.mx_quantize_workspace_size
    assert ws(8192, 8192, 3, mx.FUSE_NONE) == 0
    assert walks(8192, 8192) == 16 and walks(16384, 16384) == 8 and walks(96, 32) == 1
    assert walks(8192, 8192, 1024) == 32
    assert ws(8192, 8192, 3, mx.FUSE_DBIAS) == 16 * 8192 * 4
    assert ws(8192, 8192, 3, mx.FUSE_GELU | mx.FUSE_DBIAS) == 16 * 8192 * 4
    assert ws(200 * 32, 96, 3, mx.FUSE_GELU | mx.FUSE_DBIAS) == 50 * 96 * 4
    for M, K in ((32, 32), (4096, 14336), (16384, 5120), (8192, 28672)):
        assert ws(M, K, 3, mx.FUSE_DBIAS) == walks(M, K) * K * 4
        for pre in (mx.FUSE_GELU, mx.FUSE_DGELU, mx.FUSE_DSILU):
            assert ws(M, K, 3, pre | mx.FUSE_DBIAS) == walks(M, K) * K * 4
    assert ws(0, 64, 3, mx.FUSE_DBIAS) == 0       # invalid shape
    assert ws(40, 64, 3, mx.FUSE_DBIAS) == 64 * 4  # any-shape kernel: one walk
    assert ws(16383, 16383, 3, mx.FUSE_DBIAS) == 32 * 16383 * 4   # walks of 8 x 64 rows
    assert ws(48, 72, 3, mx.FUSE_DBIAS) == 72 * 4  # partial blocks: one walk
    assert ws(64, 64, 0, mx.FUSE_DBIAS) == 0      # invalid axis
    assert ws(64, 64, 3, 0x14) == 0               # invalid pre-op
    assert ws(8192, 8192, 3 | mx.ELEM_E5M2 | mx.SCALE_ROUND_UP, mx.FUSE_DBIAS) == 16 * 8192 * 4
    assert ws(64, 64, 0x23, mx.FUSE_DBIAS) == 0   # unknown flag
    # the tile layout makes every walk at least two sub-tiles long
    assert walks(1024, 4096) == 8
    assert ws(1024, 4096, 3, mx.FUSE_DBIAS) == 8 * 4096 * 4
    assert ws(1024, 4096, 3 | mx.SCALE_TILED, mx.FUSE_DBIAS) == 4 * 4096 * 4
    assert ws(8192, 8192, 3 | mx.SCALE_TILED, mx.FUSE_DBIAS) == 16 * 8192 * 4


def test_scale_size():
    sz = mx.mx_scale_size
    assert sz(16384, 16384, 3) == 16384 * 512
    assert sz(16384, 16384, 3 | mx.SCALE_TILED) == 16384 * 512       # whole tiles
    assert sz(64, 96, 1) == 64 * 3
    assert sz(64, 96, 1 | mx.SCALE_TILED) == 2 * 1 * 256              # 3 blocks pad to 8
    assert sz(96, 800, 2 | mx.SCALE_TILED) == 3 * 4 * 256             # 25 blocks -> 4 tiles
    assert sz(0, 64, 3) == 0 and sz(64, 64, 0) == 0 and sz(64, 64, 0x43) == 0
    assert sz(48, 72, 3) == 48 * 3 and sz(72, 48, 3) == 72 * 2         # partial blocks
    assert sz(48, 72, 3 | mx.SCALE_TILED) == 2 * 1 * 256


def test_tiled_scales_alias_check_uses_tiled_size():
    b = Bufs(64, 96)
    # compact s_row is 64 * 3 = 192 bytes; tiled it is 512, so an s_col that
    # starts 256 bytes after s_row overlaps it (rejected before any launch)
    assert q(b, axis=3 | mx.SCALE_TILED, s_col=b.p("s_row", 256)) == mx.MX_ERR_ALIAS
    assert b.untouched()


class Bufs:
    """16-byte aligned host buffers standing in for device memory, with canaries."""

    def __init__(self, M, K):
        self.M, self.K = M, K
        self.arrays = {}
        for name, nbytes in dict(x=2 * M * K, g=2 * M * K, q_row=M * K, s_row=M * K // 32,
                                 q_col=M * K, s_col=M * K // 32, dbias=4 * K,
                                 ws=4 * K * ((M + 127) // 128), amax=16).items():
            raw = np.full(nbytes + 64, 0xA5, np.uint8)
            off = (-raw.ctypes.data) % 16
            self.arrays[name] = (raw, off)

    def p(self, name, shift=0):
        raw, off = self.arrays[name]
        return ctypes.c_void_p(raw.ctypes.data + off + shift)

    def untouched(self):
        return all(np.all(raw == 0xA5) for raw, _ in self.arrays.values())


def q(b, x=None, grad=None, M=None, K=None, axis=3, fusion=0, q_row=None, s_row=None,
      q_col=None, s_col=None, dbias=None, ws=None, ws_bytes=None):
    L = mx.lib()
    M = b.M if M is None else M
    K = b.K if K is None else K
    x = b.p("x") if x is None else x
    grad = b.p("g") if grad is None else grad
    q_row = b.p("q_row") if q_row is None else q_row
    s_row = b.p("s_row") if s_row is None else s_row
    q_col = b.p("q_col") if q_col is None else q_col
    s_col = b.p("s_col") if s_col is None else s_col
    dbias = b.p("dbias") if dbias is None else dbias
    ws = b.p("ws") if ws is None else ws
    ws_bytes = 4 * K * ((M + 127) // 128) if ws_bytes is None else ws_bytes
    return L.mx_quantize(x, grad, M, K, axis, fusion, q_row, s_row, q_col, s_col, dbias, ws,
                         ws_bytes, None)


NULL = ctypes.c_void_p(0)


@pytest.mark.parametrize("kw,code", [
    (dict(axis=0), mx.MX_ERR_ENUM),
    (dict(axis=4), mx.MX_ERR_ENUM),            # a format flag without an axis
    (dict(axis=12), mx.MX_ERR_ENUM),
    (dict(axis=0x23), mx.MX_ERR_ENUM),
    (dict(axis=0x10), mx.MX_ERR_ENUM),
    (dict(axis=3 | mx.SCALE_TILED, x=NULL), mx.MX_ERR_NULL),
    (dict(axis=3 | mx.ELEM_E5M2 | mx.SCALE_ROUND_UP, x=NULL), mx.MX_ERR_NULL),  # flags accepted
    (dict(axis=1 | mx.ELEM_E5M2, M=0), mx.MX_ERR_SHAPE),
    (dict(fusion=5), mx.MX_ERR_ENUM),
    (dict(fusion=0x20), mx.MX_ERR_ENUM),
    (dict(fusion=4), mx.MX_ERR_ENUM),
    (dict(fusion=mx.FUSE_DSILU, grad=NULL), mx.MX_ERR_NULL),
    (dict(x=NULL), mx.MX_ERR_NULL),
    (dict(fusion=mx.FUSE_DGELU, grad=NULL), mx.MX_ERR_NULL),
    (dict(axis=1, s_row=NULL), mx.MX_ERR_NULL),
    (dict(axis=2, q_col=NULL), mx.MX_ERR_NULL),
    (dict(fusion=mx.FUSE_DBIAS, dbias=NULL), mx.MX_ERR_NULL),
    (dict(M=0), mx.MX_ERR_SHAPE),              # any M, K >= 1 (up to the limits) is a shape
    (dict(K=-8), mx.MX_ERR_SHAPE),
    (dict(K=0), mx.MX_ERR_SHAPE),
    (dict(M=-32), mx.MX_ERR_SHAPE),
    (dict(M=1 << 31), mx.MX_ERR_SHAPE),
    (dict(M=1 << 26, K=1 << 26), mx.MX_ERR_SHAPE),
    (dict(M=(1 << 23) + 32), mx.MX_ERR_SHAPE),
    (dict(K=(1 << 23) + 32), mx.MX_ERR_SHAPE),
    (dict(fusion=mx.FUSE_DBIAS, ws=NULL), mx.MX_ERR_WORKSPACE),
    (dict(fusion=mx.FUSE_DBIAS, ws_bytes=16), mx.MX_ERR_WORKSPACE),
])
def test_mx_quantize_rejects(kw, code):
    b = Bufs(64, 96)
    assert q(b, **kw) == code
    assert b.untouched()


def test_mx_quantize_alignment_and_alias():
    b = Bufs(64, 96)
    assert q(b, x=b.p("x", 8)) == mx.MX_ERR_ALIGN
    assert q(b, q_col=b.p("q_col", 4)) == mx.MX_ERR_ALIGN
    assert q(b, fusion=mx.FUSE_DGELU, grad=b.p("g", 2)) == mx.MX_ERR_ALIGN
    # an output inside the input, an output overlapping another output
    assert q(b, q_row=b.p("x", 16)) == mx.MX_ERR_ALIAS
    assert q(b, q_col=b.p("q_row", 32)) == mx.MX_ERR_ALIAS
    assert q(b, fusion=mx.FUSE_DGELU, s_row=b.p("g", 64)) == mx.MX_ERR_ALIAS
    assert q(b, fusion=mx.FUSE_DBIAS, dbias=b.p("ws", 0)) == mx.MX_ERR_ALIAS
    assert b.untouched()


def test_gated_and_fused_values_reject():
    b = Bufs(64, 128)
    L = mx.lib()
    g = lambda **kw: L.mx_quantize_gated(kw.get("x", b.p("x")), kw.get("M", 64), kw.get("N", 64),
                                         kw.get("axis", 3), kw.get("act", 1),
                                         kw.get("q_row", b.p("q_row")), kw.get("s_row", b.p("s_row")),
                                         kw.get("q_col", b.p("q_col")), kw.get("s_col", b.p("s_col")),
                                         None)
    assert g(act=0) == mx.MX_ERR_ENUM and g(act=3) == mx.MX_ERR_ENUM
    assert g(axis=0) == mx.MX_ERR_ENUM and g(axis=8) == mx.MX_ERR_ENUM and g(axis=0x23) == mx.MX_ERR_ENUM
    assert g(axis=3 | mx.ELEM_E5M2 | mx.SCALE_ROUND_UP, x=NULL) == mx.MX_ERR_NULL
    assert g(x=NULL) == mx.MX_ERR_NULL
    assert g(N=0) == mx.MX_ERR_SHAPE and g(M=-16) == mx.MX_ERR_SHAPE and g(N=1 << 23) == mx.MX_ERR_SHAPE
    assert g(x=b.p("x", 4)) == mx.MX_ERR_ALIGN
    assert g(q_row=b.p("x", 32)) == mx.MX_ERR_ALIAS
    f = lambda **kw: L.mx_fused_values(kw.get("x", b.p("x")), kw.get("g", b.p("g")), kw.get("M", 64),
                                       kw.get("K", 64), kw.get("op", mx.FUSE_GELU),
                                       kw.get("y", b.p("q_row")), None)
    assert f(op=0) == mx.MX_ERR_ENUM and f(op=mx.FUSE_DBIAS) == mx.MX_ERR_ENUM
    assert f(op=mx.OP_GATED | 3) == mx.MX_ERR_ENUM
    assert f(y=NULL) == mx.MX_ERR_NULL and f(op=mx.FUSE_DGELU, g=NULL) == mx.MX_ERR_NULL
    assert f(K=0) == mx.MX_ERR_SHAPE and f(M=-1) == mx.MX_ERR_SHAPE
    assert f(y=b.p("q_row", 2)) == mx.MX_ERR_ALIGN
    assert f(y=b.p("x", 16)) == mx.MX_ERR_ALIAS
    assert b.untouched()


def test_dgated_and_backward_values_reject():
    b = Bufs(64, 128)        # x [64][128] = [gate | linear], grad in "g", outputs [64][128]
    L = mx.lib()
    d = lambda **kw: L.mx_quantize_dgated(kw.get("g", b.p("g")), kw.get("x", b.p("x")),
                                          kw.get("M", 64), kw.get("N", 64), kw.get("axis", 3),
                                          kw.get("act", 1), kw.get("q_row", b.p("q_row")),
                                          kw.get("s_row", b.p("s_row")), kw.get("q_col", b.p("q_col")),
                                          kw.get("s_col", b.p("s_col")), None)
    assert d(act=0) == mx.MX_ERR_ENUM and d(act=3) == mx.MX_ERR_ENUM and d(axis=4) == mx.MX_ERR_ENUM
    assert d(axis=0x43) == mx.MX_ERR_ENUM and d(axis=2 | mx.ELEM_E5M2, x=NULL) == mx.MX_ERR_NULL
    assert d(g=NULL) == mx.MX_ERR_NULL and d(x=NULL) == mx.MX_ERR_NULL
    assert d(axis=1, s_row=NULL) == mx.MX_ERR_NULL
    assert d(N=0) == mx.MX_ERR_SHAPE and d(M=0) == mx.MX_ERR_SHAPE and d(N=1 << 23) == mx.MX_ERR_SHAPE
    assert d(g=b.p("g", 2)) == mx.MX_ERR_ALIGN and d(s_col=b.p("s_col", 8)) == mx.MX_ERR_ALIGN
    assert d(q_col=b.p("g", 16)) == mx.MX_ERR_ALIAS and d(q_row=b.p("x", 64)) == mx.MX_ERR_ALIAS
    f = lambda **kw: L.mx_fused_values(kw.get("x", b.p("x")), kw.get("g", b.p("g")), 64, 64,
                                       kw.get("op", mx.FUSE_DSILU), kw.get("y", b.p("q_row")), None)
    assert f(op=mx.OP_DGATED | 3) == mx.MX_ERR_ENUM and f(op=mx.OP_DGATED) == mx.MX_ERR_ENUM
    assert f(g=NULL) == mx.MX_ERR_NULL and f(op=mx.OP_DGATED | 1, g=NULL) == mx.MX_ERR_NULL
    assert f(y=b.p("x", 32)) == mx.MX_ERR_ALIAS
    assert b.untouched()


def test_nvfp4_and_absmax_reject():
    b = Bufs(64, 128)
    L = mx.lib()
    n = lambda **kw: L.nvfp4_quantize_transpose(kw.get("x", b.p("x")), kw.get("M", 64),
                                                kw.get("K", 128), kw.get("amax", b.p("amax")),
                                                kw.get("axis", 3), kw.get("q_row", b.p("q_row")),
                                                kw.get("s_row", b.p("s_row")),
                                                kw.get("q_col", b.p("q_col")),
                                                kw.get("s_col", b.p("s_col")),
                                                kw.get("sg", NULL), None)
    assert n(axis=0) == mx.MX_ERR_ENUM
    assert n(axis=3 | mx.ELEM_E5M2) == mx.MX_ERR_ENUM      # NVFP4 has no format flags
    assert n(axis=1 | mx.SCALE_ROUND_UP) == mx.MX_ERR_ENUM
    assert n(amax=NULL) == mx.MX_ERR_NULL and n(x=NULL) == mx.MX_ERR_NULL
    assert n(M=0) == mx.MX_ERR_SHAPE and n(K=-16) == mx.MX_ERR_SHAPE   # any M, K >= 1 is a shape
    assert n(s_col=b.p("s_col", 1)) == mx.MX_ERR_ALIGN
    assert n(sg=b.p("x", 4)) == mx.MX_ERR_ALIAS
    assert n(amax=b.p("q_row", 0)) == mx.MX_ERR_ALIAS
    a = lambda **kw: L.mx_absmax_bf16(kw.get("x", b.p("x")), kw.get("n", 100),
                                      kw.get("amax", b.p("amax")), None)
    assert a(n=0) == mx.MX_ERR_SHAPE and a(x=NULL) == mx.MX_ERR_NULL
    assert a(x=b.p("x", 2)) == mx.MX_ERR_ALIGN
    assert a(amax=b.p("x", 16)) == mx.MX_ERR_ALIAS
    assert b.untouched()


def test_grouped_sizes():
    ws, sz = mx.mx_quantize_grouped_workspace_size, mx.mx_grouped_scale_size
    # walks per group with the walk length of the whole stack (here 1 sub-tile)
    assert walks(512, 256) == 4
    assert ws(256, [128, 0, 256, 128], 3, mx.FUSE_DBIAS) == (1 + 0 + 2 + 1) * 256 * 4
    assert ws(256, [128, 0, 256, 128], 3, mx.FUSE_NONE) == 0
    # tiled: walks of at least 2 sub-tiles
    assert ws(256, [128, 0, 256, 128], 3 | mx.SCALE_TILED, mx.FUSE_DBIAS) == 3 * 256 * 4
    assert sz(96, [48, 0, 80], 3, False) == 128 * 3
    assert sz(96, [48, 0, 80], 3, True) == 96 * 2 + 96 * 3
    assert sz(96, [48, 0, 80], 3 | mx.SCALE_TILED, True) == 3 * 1 * 256 + 3 * 1 * 256
    assert sz(96, [40], 3, False) == 40 * 3 and sz(96, [40, 8], 3, True) == 96 * 2 + 96 * 1
    assert sz(96, [-16], 3, False) == 0 and sz(96, [0, 0], 3, False) == 0 and sz(96, [], 3, False) == 0


def test_grouped_rejects():
    b = Bufs(64, 96)
    L = mx.lib()

    def gq(rows=(32, 0, 32), G=None, **kw):
        arr = (ctypes.c_int64 * max(1, len(rows)))(*rows)
        return L.mx_quantize_grouped(kw.get("x", b.p("x")), kw.get("g", b.p("g")), kw.get("K", 96),
                                     kw.get("rows_p", ctypes.cast(arr, ctypes.c_void_p)),
                                     len(rows) if G is None else G, kw.get("axis", 3),
                                     kw.get("fusion", 0), kw.get("q_row", b.p("q_row")),
                                     kw.get("s_row", b.p("s_row")), kw.get("q_col", b.p("q_col")),
                                     kw.get("s_col", b.p("s_col")), kw.get("dbias", b.p("dbias")),
                                     kw.get("ws", b.p("ws")), kw.get("ws_bytes", 4096), None)
    assert gq(axis=0) == mx.MX_ERR_ENUM and gq(fusion=5) == mx.MX_ERR_ENUM
    assert gq(x=NULL) == mx.MX_ERR_NULL and gq(rows_p=NULL) == mx.MX_ERR_NULL
    assert gq(fusion=mx.FUSE_DGELU, g=NULL) == mx.MX_ERR_NULL
    assert gq(rows=(32, -16, 48)) == mx.MX_ERR_SHAPE
    assert gq(rows=(0, 0)) == mx.MX_ERR_SHAPE            # no rows at all
    assert gq(rows=(32,), G=0) == mx.MX_ERR_SHAPE
    assert gq(rows=tuple([16] * 65)) == mx.MX_ERR_SHAPE   # more than 64 groups
    assert gq(K=0) == mx.MX_ERR_SHAPE and gq(rows=(32, (1 << 23) + 1)) == mx.MX_ERR_SHAPE
    assert gq(x=b.p("x", 8)) == mx.MX_ERR_ALIGN
    assert gq(fusion=mx.FUSE_DBIAS, ws=NULL) == mx.MX_ERR_WORKSPACE
    assert gq(fusion=mx.FUSE_DBIAS, ws_bytes=16) == mx.MX_ERR_WORKSPACE
    assert gq(q_col=b.p("x", 16)) == mx.MX_ERR_ALIAS
    assert gq(fusion=mx.FUSE_DBIAS, dbias=b.p("ws", 0)) == mx.MX_ERR_ALIAS
    assert b.untouched()


def test_grouped_gated_rejects():
    b = Bufs(64, 128)          # x [64][128] = [gate | linear] (N = 64), grad in "g"
    L = mx.lib()

    def gg(rows=(32, 0, 32), bwd=False, **kw):
        arr = (ctypes.c_int64 * max(1, len(rows)))(*rows)
        args = [kw.get("x", b.p("x")), kw.get("N", 64), ctypes.cast(arr, ctypes.c_void_p),
                kw.get("G", len(rows)), kw.get("axis", 3), kw.get("act", 1),
                kw.get("q_row", b.p("q_row")), kw.get("s_row", b.p("s_row")),
                kw.get("q_col", b.p("q_col")), kw.get("s_col", b.p("s_col")), None]
        if bwd:
            return L.mx_quantize_dgated_grouped(kw.get("g", b.p("g")), *args)
        return L.mx_quantize_gated_grouped(*args)
    for bwd in (False, True):
        assert gg(bwd=bwd, act=0) == mx.MX_ERR_ENUM and gg(bwd=bwd, axis=0x40 | 3) == mx.MX_ERR_ENUM
        assert gg(bwd=bwd, x=NULL) == mx.MX_ERR_NULL
        assert gg(bwd=bwd, rows=(32, -16)) == mx.MX_ERR_SHAPE and gg(bwd=bwd, N=0) == mx.MX_ERR_SHAPE
        assert gg(bwd=bwd, G=0) == mx.MX_ERR_SHAPE
        assert gg(bwd=bwd, x=b.p("x", 4)) == mx.MX_ERR_ALIGN
        assert gg(bwd=bwd, q_row=b.p("x", 16)) == mx.MX_ERR_ALIAS
    assert gg(bwd=True, g=NULL) == mx.MX_ERR_NULL
    assert gg(bwd=True, q_col=b.p("g", 32)) == mx.MX_ERR_ALIAS
    assert b.untouched()


def test_grouped_nvfp4_rejects():
    b = Bufs(64, 96)
    L = mx.lib()

    def nq(rows=(32, 0, 32), G=None, **kw):
        arr = (ctypes.c_int64 * max(1, len(rows)))(*rows)
        return L.nvfp4_quantize_transpose_grouped(
            kw.get("x", b.p("x")), kw.get("K", 96), kw.get("rows_p", ctypes.cast(arr, ctypes.c_void_p)),
            len(rows) if G is None else G, kw.get("amax", b.p("amax")), kw.get("two_d", 0),
            kw.get("axis", 3), kw.get("q_row", b.p("q_row")), kw.get("s_row", b.p("s_row")),
            kw.get("q_col", b.p("q_col")), kw.get("s_col", b.p("s_col")), kw.get("sg", NULL), None)

    def am(rows=(32, 0, 32), **kw):
        arr = (ctypes.c_int64 * len(rows))(*rows)
        return L.mx_absmax_bf16_grouped(kw.get("x", b.p("x")), kw.get("K", 96),
                                        ctypes.cast(arr, ctypes.c_void_p), len(rows),
                                        kw.get("amax", b.p("amax")), None)
    assert nq(axis=0) == mx.MX_ERR_ENUM and nq(axis=3 | mx.ELEM_E5M2) == mx.MX_ERR_ENUM
    assert nq(two_d=2) == mx.MX_ERR_ENUM
    assert nq(x=NULL) == mx.MX_ERR_NULL and nq(amax=NULL) == mx.MX_ERR_NULL
    assert nq(rows_p=NULL) == mx.MX_ERR_NULL
    assert nq(rows=(32, -16)) == mx.MX_ERR_SHAPE and nq(K=0) == mx.MX_ERR_SHAPE
    assert nq(rows=(0,)) == mx.MX_ERR_SHAPE and nq(rows=tuple([16] * 65)) == mx.MX_ERR_SHAPE
    assert nq(s_col=b.p("s_col", 4)) == mx.MX_ERR_ALIGN
    assert nq(sg=b.p("x", 0)) == mx.MX_ERR_ALIAS
    assert am(x=NULL) == mx.MX_ERR_NULL and am(rows=(-8,)) == mx.MX_ERR_SHAPE
    assert am(amax=b.p("x", 16)) == mx.MX_ERR_ALIAS
    assert b.untouched()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mx, "_lib", None)
    monkeypatch.setattr(mx, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        mx.lib()


def test_noalloc_rejects_before_any_launch():
    """The allocation-free cast validates like mx_quantize (no workspace
    arguments) and refuses a dbias cast whose partials exceed its static
    scratch, before touching the runtime."""
    b = Bufs(64, 96)
    L = mx.lib()

    def qn(**kw):
        a = dict(x=b.p("x"), grad=b.p("g"), M=64, K=96, axis=3, fusion=0, q_row=b.p("q_row"),
                 s_row=b.p("s_row"), q_col=b.p("q_col"), s_col=b.p("s_col"), dbias=b.p("dbias"))
        a.update(kw)
        return L.mx_quantize_noalloc(a["x"], a["grad"], a["M"], a["K"], a["axis"], a["fusion"],
                                     a["q_row"], a["s_row"], a["q_col"], a["s_col"], a["dbias"],
                                     None)

    assert qn(axis=0) == mx.MX_ERR_ENUM
    assert qn(x=NULL) == mx.MX_ERR_NULL
    assert qn(fusion=mx.FUSE_DBIAS, dbias=NULL) == mx.MX_ERR_NULL
    assert qn(M=0) == mx.MX_ERR_SHAPE
    assert qn(x=b.p("x", 8)) == mx.MX_ERR_ALIGN
    assert qn(q_row=b.p("x", 16)) == mx.MX_ERR_ALIAS
    # 128 x 2^21 with dbias: one walk of 2^21 fp32 partials = 8 MiB > 4 MiB
    assert mx.mx_quantize_workspace_size(128, 1 << 21, 3, mx.FUSE_GELU | mx.FUSE_DBIAS) == 8 << 20
    assert qn(M=128, K=1 << 21, fusion=mx.FUSE_GELU | mx.FUSE_DBIAS) == mx.MX_ERR_WORKSPACE
    assert mx.mx_quantize_workspace_size(128, 1 << 20, 3, mx.FUSE_DBIAS) == mx.NOALLOC_SCRATCH_BYTES
    assert b.untouched()
