"""Python binding of libmxcast (include/mxcast.h): block-scaled quantisation of
bf16 tensors on MI355X.

Argument marshalling only.  Every step of the cast runs in the HIP kernels of
libmxcast.so; PyTorch provides device memory and the stream.  If the library
is not built, importing a function raises -- there is no fallback path.

The same names as the C ABI:
    mx_quantize, mx_quantize_workspace_size, mx_scale_size, mx_quantize_grouped,
    mx_quantize_grouped_workspace_size, mx_grouped_scale_size, mx_quantize_gated,
    mx_fused_values, mx_absmax_bf16, nvfp4_quantize_transpose,
    mx_status_str, mx_abi_version
take torch tensors (bf16 inputs, or int16/uint16 holding bf16 bits, on a ROCm
device) and return dicts of uint8 / float32 torch tensors on the same device.
The MXFP8 casts take the format flags ELEM_E5M2 / SCALE_ROUND_UP and the
layout flag SCALE_TILED OR-ed into `axis`, as the C ABI does.
`lib()` returns the raw ctypes library for callers that pass pointers
themselves.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxcast.so")

ROWWISE, COLWISE = 1, 2
ELEM_E5M2, SCALE_ROUND_UP = 4, 8     # MXFP8 format flags, OR-ed into axis
SCALE_TILED = 16                     # GEMM-ready scale layout flag, OR-ed into axis
FUSE_NONE, FUSE_GELU, FUSE_DGELU, FUSE_DSILU, FUSE_DBIAS = 0, 1, 2, 3, 0x10
GATED_SWIGLU, GATED_GEGLU = 1, 2
OP_GATED, OP_DGATED = 0x100, 0x200
(MX_OK, MX_ERR_NULL, MX_ERR_ENUM, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_WORKSPACE,
 MX_ERR_ALIAS, MX_ERR_HIP, MX_ERR_UNSUPPORTED) = range(9)

EXPORTS = ("mx_quantize", "mx_quantize_workspace_size", "mx_scale_size", "mx_quantize_grouped",
           "mx_quantize_grouped_workspace_size", "mx_grouped_scale_size", "mx_quantize_gated",
           "mx_quantize_gated_grouped", "mx_quantize_dgated_grouped",
           "mx_quantize_dgated", "mx_fused_values",
           "mx_absmax_bf16", "nvfp4_quantize_transpose", "nvfp4_quantize_transpose_2d",
           "mx_absmax_bf16_grouped", "nvfp4_quantize_transpose_grouped",
           "mx_status_str", "mx_abi_version")


class MxError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {mx_status_str(status)} (status {status})")


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


def lib():
    """The loaded libmxcast.so with argument types set (raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        L.mx_quantize.restype = ctypes.c_int
        L.mx_quantize.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_uint, ctypes.c_int,
                                  _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.mx_quantize_workspace_size.restype = ctypes.c_size_t
        L.mx_quantize_workspace_size.argtypes = [_i64, _i64, ctypes.c_uint, ctypes.c_int]
        L.mx_scale_size.restype = ctypes.c_size_t
        L.mx_scale_size.argtypes = [_i64, _i64, ctypes.c_uint]
        L.mx_quantize_grouped.restype = ctypes.c_int
        L.mx_quantize_grouped.argtypes = [_vp, _vp, _i64, _vp, ctypes.c_int, ctypes.c_uint,
                                          ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.c_size_t, _vp]
        L.mx_quantize_grouped_workspace_size.restype = ctypes.c_size_t
        L.mx_quantize_grouped_workspace_size.argtypes = [_i64, _vp, ctypes.c_int, ctypes.c_uint,
                                                         ctypes.c_int]
        L.mx_grouped_scale_size.restype = ctypes.c_size_t
        L.mx_grouped_scale_size.argtypes = [_i64, _vp, ctypes.c_int, ctypes.c_uint, ctypes.c_int]
        L.mx_quantize_gated_grouped.restype = ctypes.c_int
        L.mx_quantize_gated_grouped.argtypes = [_vp, _i64, _vp, ctypes.c_int, ctypes.c_uint,
                                                ctypes.c_int, _vp, _vp, _vp, _vp, _vp]
        L.mx_quantize_dgated_grouped.restype = ctypes.c_int
        L.mx_quantize_dgated_grouped.argtypes = [_vp, _vp, _i64, _vp, ctypes.c_int, ctypes.c_uint,
                                                 ctypes.c_int, _vp, _vp, _vp, _vp, _vp]
        L.mx_quantize_gated.restype = ctypes.c_int
        L.mx_quantize_gated.argtypes = [_vp, _i64, _i64, ctypes.c_uint, ctypes.c_int,
                                        _vp, _vp, _vp, _vp, _vp]
        L.mx_quantize_dgated.restype = ctypes.c_int
        L.mx_quantize_dgated.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_uint, ctypes.c_int,
                                         _vp, _vp, _vp, _vp, _vp]
        L.mx_fused_values.restype = ctypes.c_int
        L.mx_fused_values.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_int, _vp, _vp]
        L.mx_absmax_bf16.restype = ctypes.c_int
        L.mx_absmax_bf16.argtypes = [_vp, _i64, _vp, _vp]
        L.nvfp4_quantize_transpose.restype = ctypes.c_int
        L.nvfp4_quantize_transpose.argtypes = [_vp, _i64, _i64, _vp, ctypes.c_uint,
                                               _vp, _vp, _vp, _vp, _vp, _vp]
        L.nvfp4_quantize_transpose_2d.restype = ctypes.c_int
        L.nvfp4_quantize_transpose_2d.argtypes = L.nvfp4_quantize_transpose.argtypes
        L.mx_absmax_bf16_grouped.restype = ctypes.c_int
        L.mx_absmax_bf16_grouped.argtypes = [_vp, _i64, _vp, ctypes.c_int, _vp, _vp]
        L.nvfp4_quantize_transpose_grouped.restype = ctypes.c_int
        L.nvfp4_quantize_transpose_grouped.argtypes = [_vp, _i64, _vp, ctypes.c_int, _vp,
                                                       ctypes.c_int, ctypes.c_uint, _vp, _vp,
                                                       _vp, _vp, _vp, _vp]
        L.mx_status_str.restype = ctypes.c_char_p
        L.mx_status_str.argtypes = [ctypes.c_int]
        L.mx_abi_version.restype = ctypes.c_int
        L.mx_abi_version.argtypes = []
        _lib = L
    return _lib


def mx_status_str(status: int) -> str:
    return lib().mx_status_str(int(status)).decode()


def mx_abi_version() -> int:
    return lib().mx_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _bf16_bits(t):
    if t is None:
        return None
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected bf16 (or int16/uint16 bf16 bits), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t


def _check(status, where):
    if status != MX_OK:
        raise MxError(status, where)


def _u8(shape, dev):
    return torch.empty(shape, dtype=torch.uint8, device=dev)


def mx_quantize_workspace_size(M: int, K: int, axis: int = ROWWISE | COLWISE,
                               fusion: int = FUSE_NONE) -> int:
    return lib().mx_quantize_workspace_size(M, K, axis, fusion)


def mx_scale_size(rows: int, cols: int, axis: int = ROWWISE | COLWISE) -> int:
    return lib().mx_scale_size(rows, cols, axis)


def _scales(rows, cols, axis, dev):
    """One direction's scale tensor: [rows][ceil(cols/32)], or flat in the tile
    layout."""
    if axis & SCALE_TILED:
        return _u8((mx_scale_size(rows, cols, axis),), dev)
    return _u8((rows, -(-cols // 32)), dev)


def mx_quantize(x, grad=None, axis=ROWWISE | COLWISE, fusion=FUSE_NONE, out=None,
                workspace=None, stream=None):
    """MXFP8 cast of x[M][K].  Returns {q_row, s_row, q_col, s_col, dbias}
    (None where not requested).  `out` may hold preallocated outputs and
    `workspace` a preallocated uint8 buffer (needed only with FUSE_DBIAS)."""
    x = _bf16_bits(x)
    grad = _bf16_bits(grad) if (fusion & 0xF) in (FUSE_DGELU, FUSE_DSILU) else None
    M, K = x.shape
    dev = x.device
    o = dict(out or {})
    if axis & ROWWISE:
        o.setdefault("q_row", _u8((M, K), dev))
        o.setdefault("s_row", _scales(M, K, axis, dev))
    if axis & COLWISE:
        o.setdefault("q_col", _u8((K, M), dev))
        o.setdefault("s_col", _scales(K, M, axis, dev))
    ws_bytes = 0
    if fusion & FUSE_DBIAS:
        o.setdefault("dbias", torch.empty(K, dtype=torch.float32, device=dev))
        ws_bytes = mx_quantize_workspace_size(M, K, axis, fusion)
        if workspace is None:
            workspace = _u8((max(ws_bytes, 16),), dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().mx_quantize(_ptr(x), _ptr(grad), M, K, axis, fusion,
                           _ptr(o.get("q_row")), _ptr(o.get("s_row")), _ptr(o.get("q_col")),
                           _ptr(o.get("s_col")), _ptr(o.get("dbias")),
                           _ptr(workspace) if fusion & FUSE_DBIAS else None, ws_bytes,
                           _stream(dev, stream))
    _check(st, "mx_quantize")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col", "dbias")}


def _rows_arg(group_rows):
    """Host int64 array of group row counts (kept alive by the caller)."""
    return (ctypes.c_int64 * len(group_rows))(*[int(r) for r in group_rows])


def mx_quantize_grouped_workspace_size(K: int, group_rows, axis: int = ROWWISE | COLWISE,
                                       fusion: int = FUSE_NONE) -> int:
    rows = _rows_arg(group_rows)
    return lib().mx_quantize_grouped_workspace_size(K, ctypes.cast(rows, _vp), len(group_rows),
                                                    axis, fusion)


def mx_grouped_scale_size(K: int, group_rows, axis: int, colwise: bool) -> int:
    rows = _rows_arg(group_rows)
    return lib().mx_grouped_scale_size(K, ctypes.cast(rows, _vp), len(group_rows), axis,
                                       int(colwise))


def mx_quantize_grouped(x, group_rows, grad=None, axis=ROWWISE | COLWISE, fusion=FUSE_NONE,
                        out=None, workspace=None, stream=None):
    """Grouped MXFP8 cast of x[M][K] = len(group_rows) tensors stacked along
    rows.  Returns q_row [M][K], flat s_row / q_col / s_col holding the groups'
    outputs one after the other, and dbias [G][K] (None where not requested)."""
    x = _bf16_bits(x)
    grad = _bf16_bits(grad) if (fusion & 0xF) in (FUSE_DGELU, FUSE_DSILU) else None
    M, K = x.shape
    G = len(group_rows)
    dev = x.device
    o = dict(out or {})
    if axis & ROWWISE:
        o.setdefault("q_row", _u8((M, K), dev))
        o.setdefault("s_row", _u8((max(1, mx_grouped_scale_size(K, group_rows, axis, False)),), dev))
    if axis & COLWISE:
        o.setdefault("q_col", _u8((M * K,), dev))
        o.setdefault("s_col", _u8((max(1, mx_grouped_scale_size(K, group_rows, axis, True)),), dev))
    ws_bytes = 0
    if fusion & FUSE_DBIAS:
        o.setdefault("dbias", torch.empty((G, K), dtype=torch.float32, device=dev))
        ws_bytes = mx_quantize_grouped_workspace_size(K, group_rows, axis, fusion)
        if workspace is None:
            workspace = _u8((max(ws_bytes, 16),), dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    rows = _rows_arg(group_rows)
    st = lib().mx_quantize_grouped(_ptr(x), _ptr(grad), K, ctypes.cast(rows, _vp), G, axis, fusion,
                                   _ptr(o.get("q_row")), _ptr(o.get("s_row")),
                                   _ptr(o.get("q_col")), _ptr(o.get("s_col")),
                                   _ptr(o.get("dbias")),
                                   _ptr(workspace) if fusion & FUSE_DBIAS else None, ws_bytes,
                                   _stream(dev, stream))
    _check(st, "mx_quantize_grouped")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col", "dbias")}


def mx_quantize_gated(x, act, axis=ROWWISE | COLWISE, out=None, stream=None):
    """Gated MXFP8 cast of x[M][2N] = [gate | linear] -> y[M][N] = act(gate)*linear."""
    x = _bf16_bits(x)
    M, N2 = x.shape
    N = N2 // 2
    dev = x.device
    o = dict(out or {})
    if axis & ROWWISE:
        o.setdefault("q_row", _u8((M, N), dev))
        o.setdefault("s_row", _scales(M, N, axis, dev))
    if axis & COLWISE:
        o.setdefault("q_col", _u8((N, M), dev))
        o.setdefault("s_col", _scales(N, M, axis, dev))
    st = lib().mx_quantize_gated(_ptr(x), M, N, axis, act, _ptr(o.get("q_row")),
                                 _ptr(o.get("s_row")), _ptr(o.get("q_col")),
                                 _ptr(o.get("s_col")), _stream(dev, stream))
    _check(st, "mx_quantize_gated")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col")}


def mx_quantize_dgated(grad, x, act, axis=ROWWISE | COLWISE, out=None, stream=None):
    """Gated backward MXFP8 cast: grad[M][N], x[M][2N] = [gate | linear] ->
    quantised dx[M][2N] = [d_gate | d_linear]."""
    grad = _bf16_bits(grad)
    x = _bf16_bits(x)
    M, N2 = x.shape
    N = N2 // 2
    dev = x.device
    o = dict(out or {})
    if axis & ROWWISE:
        o.setdefault("q_row", _u8((M, N2), dev))
        o.setdefault("s_row", _scales(M, N2, axis, dev))
    if axis & COLWISE:
        o.setdefault("q_col", _u8((N2, M), dev))
        o.setdefault("s_col", _scales(N2, M, axis, dev))
    st = lib().mx_quantize_dgated(_ptr(grad), _ptr(x), M, N, axis, act, _ptr(o.get("q_row")),
                                  _ptr(o.get("s_row")), _ptr(o.get("q_col")),
                                  _ptr(o.get("s_col")), _stream(dev, stream))
    _check(st, "mx_quantize_dgated")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col")}


def mx_fused_values(x, grad=None, op=FUSE_GELU, out=None, stream=None):
    """The bf16 values the fused casts quantise (returned as int16 bits).
    Gated ops (OP_GATED | act) take x[M][2K] and give [M][K]; gated backward
    ops (OP_DGATED | act) take x[M][2K] and grad[M][K] and give [M][2K]."""
    x = _bf16_bits(x)
    gated = bool(op & (OP_GATED | OP_DGATED))
    M, W = x.shape
    K = W // 2 if gated else W
    dev = x.device
    shape = (M, 2 * K) if op & OP_DGATED else (M, K)
    y = out if out is not None else torch.empty(shape, dtype=torch.int16, device=dev)
    g = _bf16_bits(grad) if (op in (FUSE_DGELU, FUSE_DSILU) or op & OP_DGATED) else None
    st = lib().mx_fused_values(_ptr(x), _ptr(g), M, K, op, _ptr(y), _stream(dev, stream))
    _check(st, "mx_fused_values")
    return y


def mx_absmax_bf16(x, out=None, stream=None):
    """Tensor absmax as a one-element float32 device tensor."""
    x = _bf16_bits(x)
    amax = out if out is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    st = lib().mx_absmax_bf16(_ptr(x), x.numel(), _ptr(amax), _stream(x.device, stream))
    _check(st, "mx_absmax_bf16")
    return amax


def nvfp4_quantize_transpose(x, amax=None, axis=ROWWISE | COLWISE, out=None, stream=None,
                             two_d=False):
    """NVFP4 of x[M][K] and its transpose.  amax: one-element float32 device
    tensor (computed with mx_absmax_bf16 when None).  two_d: one scale per
    16 x 16 block.  Returns {q_row, s_row, q_col, s_col, sg}."""
    x = _bf16_bits(x)
    M, K = x.shape
    dev = x.device
    if amax is None:
        amax = mx_absmax_bf16(x, stream=stream)
    o = dict(out or {})
    if axis & ROWWISE:
        o.setdefault("q_row", _u8((M, K // 2), dev))
        o.setdefault("s_row", _u8((M, K // 16), dev))
    if axis & COLWISE:
        o.setdefault("q_col", _u8((K, M // 2), dev))
        o.setdefault("s_col", _u8((K, M // 16), dev))
    o.setdefault("sg", torch.empty(1, dtype=torch.float32, device=dev))
    fn = lib().nvfp4_quantize_transpose_2d if two_d else lib().nvfp4_quantize_transpose
    st = fn(_ptr(x), M, K, _ptr(amax), axis, _ptr(o.get("q_row")), _ptr(o.get("s_row")),
            _ptr(o.get("q_col")), _ptr(o.get("s_col")), _ptr(o["sg"]), _stream(dev, stream))
    _check(st, "nvfp4_quantize_transpose_2d" if two_d else "nvfp4_quantize_transpose")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col", "sg")}


def mx_absmax_bf16_grouped(x, group_rows, out=None, stream=None):
    """Per-group max |x| (fp32 [G]) of x[M][K] = len(group_rows) stacked tensors."""
    x = _bf16_bits(x)
    M, K = x.shape
    G = len(group_rows)
    amax = out if out is not None else torch.empty(G, dtype=torch.float32, device=x.device)
    rows = _rows_arg(group_rows)
    st = lib().mx_absmax_bf16_grouped(_ptr(x), K, ctypes.cast(rows, _vp), G, _ptr(amax),
                                      _stream(x.device, stream))
    _check(st, "mx_absmax_bf16_grouped")
    return amax


def nvfp4_quantize_transpose_grouped(x, group_rows, amax, axis=ROWWISE | COLWISE, two_d=False,
                                     out=None, stream=None):
    """Grouped NVFP4 of x[M][K] = len(group_rows) stacked tensors, each with its
    own tensor amax (device fp32 [G]).  Returns q_row [M][K/2], s_row
    [M][K/16], flat q_col / s_col (the groups' transposes one after the
    other) and the groups' global scales sg [G]."""
    x = _bf16_bits(x)
    M, K = x.shape
    G = len(group_rows)
    dev = x.device
    o = dict(out or {})
    if axis & ROWWISE:
        o.setdefault("q_row", _u8((M, K // 2), dev))
        o.setdefault("s_row", _u8((M, K // 16), dev))
    if axis & COLWISE:
        o.setdefault("q_col", _u8((M * K // 2,), dev))
        o.setdefault("s_col", _u8((M * K // 16,), dev))
    o.setdefault("sg", torch.empty(G, dtype=torch.float32, device=dev))
    rows = _rows_arg(group_rows)
    st = lib().nvfp4_quantize_transpose_grouped(_ptr(x), K, ctypes.cast(rows, _vp), G, _ptr(amax),
                                                int(two_d), axis, _ptr(o.get("q_row")),
                                                _ptr(o.get("s_row")), _ptr(o.get("q_col")),
                                                _ptr(o.get("s_col")), _ptr(o["sg"]),
                                                _stream(dev, stream))
    _check(st, "nvfp4_quantize_transpose_grouped")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col", "sg")}


def mx_quantize_gated_grouped(x, group_rows, act, grad=None, axis=ROWWISE | COLWISE, out=None,
                              stream=None):
    """Grouped gated MXFP8 cast of x[M][2N] = [gate | linear] stacked by group
    (with grad [M][N]: the gated backward).  q_row [M][W] (W = N, or 2N
    backward) and flat s_row / q_col / s_col, the groups one after the other."""
    x = _bf16_bits(x)
    M, N2 = x.shape
    N = N2 // 2
    W = N2 if grad is not None else N
    G = len(group_rows)
    dev = x.device
    o = dict(out or {})
    if axis & ROWWISE:
        o.setdefault("q_row", _u8((M, W), dev))
        o.setdefault("s_row", _u8((max(1, mx_grouped_scale_size(W, group_rows, axis, False)),), dev))
    if axis & COLWISE:
        o.setdefault("q_col", _u8((M * W,), dev))
        o.setdefault("s_col", _u8((max(1, mx_grouped_scale_size(W, group_rows, axis, True)),), dev))
    rows = _rows_arg(group_rows)
    ptrs = (_ptr(o.get("q_row")), _ptr(o.get("s_row")), _ptr(o.get("q_col")), _ptr(o.get("s_col")))
    if grad is None:
        st = lib().mx_quantize_gated_grouped(_ptr(x), N, ctypes.cast(rows, _vp), G, axis, act,
                                             *ptrs, _stream(dev, stream))
    else:
        grad = _bf16_bits(grad)
        st = lib().mx_quantize_dgated_grouped(_ptr(grad), _ptr(x), N, ctypes.cast(rows, _vp), G,
                                              axis, act, *ptrs, _stream(dev, stream))
    _check(st, "mx_quantize_gated_grouped")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col")}
