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

EXPORTS = ("mx_quantize", "mx_quantize_workspace_size", "mx_quantize_noalloc", "mx_scale_size", "mx_quantize_grouped",
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
        L.mx_quantize_noalloc.restype = ctypes.c_int
        L.mx_quantize_noalloc.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_uint, ctypes.c_int,
                                          _vp, _vp, _vp, _vp, _vp, _vp]
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


def _2d(t, name):
    """A bf16-bits input that must be a contiguous 2-D tensor."""
    t = _bf16_bits(t)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t


def _half_width(W, name):
    """N of a gated row [gate | linear] of W elements (W must be even)."""
    if W % 2:
        raise ValueError(f"{name}: a [gate | linear] row has an even number of columns, got {W}")
    return W // 2


def _want_shape(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _group_total(group_rows, M):
    if any(int(r) < 0 for r in group_rows):
        raise ValueError("group row counts must be non-negative")
    if sum(int(r) for r in group_rows) != M:
        raise ValueError(f"group row counts sum to {sum(int(r) for r in group_rows)}, "
                         f"but the input has {M} rows")


def _outputs(o, need, dev):
    """Allocate the outputs the caller did not pass and check those it did.
    need maps name -> (shape, dtype).  A passed tensor must be a contiguous
    tensor of that dtype on the input's device with exactly as many elements
    as the library writes."""
    o = dict(o or {})
    for k, (shape, dtype) in need.items():
        t = o.get(k)
        if t is None:
            o[k] = torch.empty(shape, dtype=dtype, device=dev)
            continue
        numel = 1
        for d in shape:
            numel *= int(d)
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"out[{k!r}] must be a tensor")
        if t.dtype != dtype or t.numel() != numel or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"out[{k!r}] must be a contiguous {dtype} tensor of {numel} elements "
                             f"on {dev}; got {t.dtype}, {t.numel()} elements on {t.device}"
                             f"{'' if t.is_contiguous() else ', not contiguous'}")
    return o


def _on_device(dev, *tensors):
    """Every tensor the library reads or writes lives on one ROCm device (a
    host pointer handed to a kernel would fault the GPU)."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a ROCm (cuda) device, got {dev}")
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError(f"all tensors must be on {dev}; got one on {t.device}")


def _f32_vec(t, n, name, dev):
    """A float32 device vector of n elements (amax, global scales)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() != n \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    return t


U8, F32, I16 = torch.uint8, torch.float32, torch.int16


def mx_quantize_workspace_size(M: int, K: int, axis: int = ROWWISE | COLWISE,
                               fusion: int = FUSE_NONE) -> int:
    return lib().mx_quantize_workspace_size(M, K, axis, fusion)


def mx_scale_size(rows: int, cols: int, axis: int = ROWWISE | COLWISE) -> int:
    return lib().mx_scale_size(rows, cols, axis)


def _scale_shape(rows, cols, axis):
    """One direction's scale tensor: [rows][ceil(cols/32)], or flat in the tile
    layout."""
    if axis & SCALE_TILED:
        return (max(1, mx_scale_size(rows, cols, axis)),)
    return (rows, -(-cols // 32))


def _mx_need(M, K, axis):
    """Outputs of an MXFP8 cast of a quantised [M][K] tensor."""
    need = {}
    if axis & ROWWISE:
        need["q_row"] = ((M, K), U8)
        need["s_row"] = (_scale_shape(M, K, axis), U8)
    if axis & COLWISE:
        need["q_col"] = ((K, M), U8)
        need["s_col"] = (_scale_shape(K, M, axis), U8)
    return need


def _workspace(workspace, need_bytes, dev):
    if workspace is None:
        return torch.empty(max(need_bytes, 16), dtype=U8, device=dev)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous() \
            or workspace.device != dev:
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    return workspace


def mx_quantize(x, grad=None, axis=ROWWISE | COLWISE, fusion=FUSE_NONE, out=None,
                workspace=None, stream=None):
    """MXFP8 cast of x[M][K].  Returns {q_row, s_row, q_col, s_col, dbias}
    (None where not requested).  `out` may hold preallocated outputs and
    `workspace` a preallocated device buffer (needed only with FUSE_DBIAS)."""
    x = _2d(x, "x")
    M, K = x.shape
    grad = _2d(grad, "grad") if (fusion & 0xF) in (FUSE_DGELU, FUSE_DSILU) else None
    _want_shape(grad, (M, K), "grad")
    dev = x.device
    need = _mx_need(M, K, axis)
    if fusion & FUSE_DBIAS:
        need["dbias"] = ((K,), F32)
    o = _outputs(out, need, dev)
    ws_bytes = 0
    if fusion & FUSE_DBIAS:
        workspace = _workspace(workspace, mx_quantize_workspace_size(M, K, axis, fusion), dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    _on_device(dev, grad, *o.values(), workspace if fusion & FUSE_DBIAS else None)
    st = lib().mx_quantize(_ptr(x), _ptr(grad), M, K, axis, fusion,
                           _ptr(o.get("q_row")), _ptr(o.get("s_row")), _ptr(o.get("q_col")),
                           _ptr(o.get("s_col")), _ptr(o.get("dbias")),
                           _ptr(workspace) if fusion & FUSE_DBIAS else None, ws_bytes,
                           _stream(dev, stream))
    _check(st, "mx_quantize")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col", "dbias")}


NOALLOC_SCRATCH_BYTES = 4 << 20     # MX_NOALLOC_SCRATCH_BYTES


def mx_quantize_noalloc(x, out, grad=None, axis=ROWWISE | COLWISE, fusion=FUSE_NONE,
                        stream=None):
    """mx_quantize without any device allocation: `out` must hold every
    requested output (q_row, s_row, q_col, s_col, and dbias with FUSE_DBIAS)
    preallocated; dbias partials use the library's static device scratch
    (calls with FUSE_DBIAS that overlap on one GPU race; see mxcast.h)."""
    x = _2d(x, "x")
    M, K = x.shape
    grad = _2d(grad, "grad") if (fusion & 0xF) in (FUSE_DGELU, FUSE_DSILU) else None
    _want_shape(grad, (M, K), "grad")
    dev = x.device
    need = _mx_need(M, K, axis)
    if fusion & FUSE_DBIAS:
        need["dbias"] = ((K,), F32)
    missing = [k for k in need if (out or {}).get(k) is None]
    if missing:
        raise ValueError(f"mx_quantize_noalloc allocates nothing: out must hold {missing}")
    o = _outputs(out, need, dev)
    _on_device(dev, grad, *o.values())
    st = lib().mx_quantize_noalloc(_ptr(x), _ptr(grad), M, K, axis, fusion,
                                   _ptr(o.get("q_row")), _ptr(o.get("s_row")),
                                   _ptr(o.get("q_col")), _ptr(o.get("s_col")),
                                   _ptr(o.get("dbias")), _stream(dev, stream))
    _check(st, "mx_quantize_noalloc")
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


def _grouped_need(M, W, group_rows, axis):
    """Outputs of a grouped MXFP8 cast of quantised [rows][W] groups."""
    need = {}
    if axis & ROWWISE:
        need["q_row"] = ((M, W), U8)
        need["s_row"] = ((max(1, mx_grouped_scale_size(W, group_rows, axis, False)),), U8)
    if axis & COLWISE:
        need["q_col"] = ((M * W,), U8)
        need["s_col"] = ((max(1, mx_grouped_scale_size(W, group_rows, axis, True)),), U8)
    return need


def mx_quantize_grouped(x, group_rows, grad=None, axis=ROWWISE | COLWISE, fusion=FUSE_NONE,
                        out=None, workspace=None, stream=None):
    """Grouped MXFP8 cast of x[M][K] = len(group_rows) tensors stacked along
    rows.  Returns q_row [M][K], flat s_row / q_col / s_col holding the groups'
    outputs one after the other, and dbias [G][K] (None where not requested)."""
    x = _2d(x, "x")
    M, K = x.shape
    _group_total(group_rows, M)
    grad = _2d(grad, "grad") if (fusion & 0xF) in (FUSE_DGELU, FUSE_DSILU) else None
    _want_shape(grad, (M, K), "grad")
    G = len(group_rows)
    dev = x.device
    need = _grouped_need(M, K, group_rows, axis)
    if fusion & FUSE_DBIAS:
        need["dbias"] = ((G, K), F32)
    o = _outputs(out, need, dev)
    ws_bytes = 0
    if fusion & FUSE_DBIAS:
        workspace = _workspace(workspace,
                               mx_quantize_grouped_workspace_size(K, group_rows, axis, fusion), dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    _on_device(dev, grad, *o.values(), workspace if fusion & FUSE_DBIAS else None)
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
    x = _2d(x, "x")
    M, N2 = x.shape
    N = _half_width(N2, "mx_quantize_gated")
    dev = x.device
    o = _outputs(out, _mx_need(M, N, axis), dev)
    _on_device(dev, *o.values())
    st = lib().mx_quantize_gated(_ptr(x), M, N, axis, act, _ptr(o.get("q_row")),
                                 _ptr(o.get("s_row")), _ptr(o.get("q_col")),
                                 _ptr(o.get("s_col")), _stream(dev, stream))
    _check(st, "mx_quantize_gated")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col")}


def mx_quantize_dgated(grad, x, act, axis=ROWWISE | COLWISE, out=None, stream=None):
    """Gated backward MXFP8 cast: grad[M][N], x[M][2N] = [gate | linear] ->
    quantised dx[M][2N] = [d_gate | d_linear]."""
    grad = _2d(grad, "grad")
    x = _2d(x, "x")
    M, N2 = x.shape
    N = _half_width(N2, "mx_quantize_dgated")
    _want_shape(grad, (M, N), "grad")
    dev = x.device
    o = _outputs(out, _mx_need(M, N2, axis), dev)
    _on_device(dev, grad, *o.values())
    st = lib().mx_quantize_dgated(_ptr(grad), _ptr(x), M, N, axis, act, _ptr(o.get("q_row")),
                                  _ptr(o.get("s_row")), _ptr(o.get("q_col")),
                                  _ptr(o.get("s_col")), _stream(dev, stream))
    _check(st, "mx_quantize_dgated")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col")}


def mx_fused_values(x, grad=None, op=FUSE_GELU, out=None, stream=None):
    """The bf16 values the fused casts quantise (returned as int16 bits).
    Gated ops (OP_GATED | act) take x[M][2K] and give [M][K]; gated backward
    ops (OP_DGATED | act) take x[M][2K] and grad[M][K] and give [M][2K]."""
    x = _2d(x, "x")
    gated = bool(op & (OP_GATED | OP_DGATED))
    M, W = x.shape
    K = _half_width(W, "mx_fused_values") if gated else W
    dev = x.device
    shape = (M, 2 * K) if op & OP_DGATED else (M, K)
    g = _2d(grad, "grad") if (op in (FUSE_DGELU, FUSE_DSILU) or op & OP_DGATED) else None
    _want_shape(g, (M, K), "grad")
    y = _outputs({"y": out}, {"y": (shape, I16)}, dev)["y"]
    _on_device(dev, g, y)
    st = lib().mx_fused_values(_ptr(x), _ptr(g), M, K, op, _ptr(y), _stream(dev, stream))
    _check(st, "mx_fused_values")
    return y


def mx_absmax_bf16(x, out=None, stream=None):
    """Tensor absmax as a one-element float32 device tensor."""
    x = _bf16_bits(x)
    dev = x.device
    amax = _outputs({"amax": out}, {"amax": ((1,), F32)}, dev)["amax"]
    _on_device(dev, amax)
    st = lib().mx_absmax_bf16(_ptr(x), x.numel(), _ptr(amax), _stream(dev, stream))
    _check(st, "mx_absmax_bf16")
    return amax


def _nv_need(M, K, axis, n_sg):
    """NVFP4 outputs: codes [rows][ceil(cols/2)], scales [rows][ceil(cols/16)]."""
    need = {}
    if axis & ROWWISE:
        need["q_row"] = ((M, -(-K // 2)), U8)
        need["s_row"] = ((M, -(-K // 16)), U8)
    if axis & COLWISE:
        need["q_col"] = ((K, -(-M // 2)), U8)
        need["s_col"] = ((K, -(-M // 16)), U8)
    need["sg"] = ((n_sg,), F32)
    return need


def nvfp4_quantize_transpose(x, amax=None, axis=ROWWISE | COLWISE, out=None, stream=None,
                             two_d=False):
    """NVFP4 of x[M][K] and its transpose.  amax: one-element float32 device
    tensor (computed with mx_absmax_bf16 when None).  two_d: one scale per
    16 x 16 block.  Returns {q_row, s_row, q_col, s_col, sg}."""
    x = _2d(x, "x")
    M, K = x.shape
    dev = x.device
    o = _outputs(out, _nv_need(M, K, axis, 1), dev)
    if amax is not None:
        _f32_vec(amax, 1, "amax", dev)
    _on_device(dev, *o.values())
    if amax is None:
        amax = mx_absmax_bf16(x, stream=stream)
    fn = lib().nvfp4_quantize_transpose_2d if two_d else lib().nvfp4_quantize_transpose
    st = fn(_ptr(x), M, K, _ptr(amax), axis, _ptr(o.get("q_row")), _ptr(o.get("s_row")),
            _ptr(o.get("q_col")), _ptr(o.get("s_col")), _ptr(o["sg"]), _stream(dev, stream))
    _check(st, "nvfp4_quantize_transpose_2d" if two_d else "nvfp4_quantize_transpose")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col", "sg")}


def mx_absmax_bf16_grouped(x, group_rows, out=None, stream=None):
    """Per-group max |x| (fp32 [G]) of x[M][K] = len(group_rows) stacked tensors."""
    x = _2d(x, "x")
    M, K = x.shape
    _group_total(group_rows, M)
    G = len(group_rows)
    dev = x.device
    amax = _outputs({"amax": out}, {"amax": ((G,), F32)}, dev)["amax"]
    _on_device(dev, amax)
    rows = _rows_arg(group_rows)
    st = lib().mx_absmax_bf16_grouped(_ptr(x), K, ctypes.cast(rows, _vp), G, _ptr(amax),
                                      _stream(dev, stream))
    _check(st, "mx_absmax_bf16_grouped")
    return amax


def nvfp4_quantize_transpose_grouped(x, group_rows, amax, axis=ROWWISE | COLWISE, two_d=False,
                                     out=None, stream=None):
    """Grouped NVFP4 of x[M][K] = len(group_rows) stacked tensors, each with its
    own tensor amax (device fp32 [G]).  Returns q_row [M][ceil(K/2)], s_row
    [M][ceil(K/16)], flat q_col / s_col (the groups' transposes one after the
    other) and the groups' global scales sg [G]."""
    x = _2d(x, "x")
    M, K = x.shape
    _group_total(group_rows, M)
    G = len(group_rows)
    dev = x.device
    need = _nv_need(M, K, axis, G)
    if "q_col" in need:   # group g's [K][ceil(rows/2)] and [K][ceil(rows/16)], one after the other
        need["q_col"] = ((K * sum(-(-int(m) // 2) for m in group_rows),), U8)
        need["s_col"] = ((K * sum(-(-int(m) // 16) for m in group_rows),), U8)
    o = _outputs(out, need, dev)
    _f32_vec(amax, G, "amax", dev)
    _on_device(dev, *o.values())
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
    x = _2d(x, "x")
    M, N2 = x.shape
    N = _half_width(N2, "mx_quantize_gated_grouped")
    _group_total(group_rows, M)
    if grad is not None:
        grad = _2d(grad, "grad")
        _want_shape(grad, (M, N), "grad")
    W = N2 if grad is not None else N
    G = len(group_rows)
    dev = x.device
    o = _outputs(out, _grouped_need(M, W, group_rows, axis), dev)
    _on_device(dev, grad, *o.values())
    rows = _rows_arg(group_rows)
    ptrs = (_ptr(o.get("q_row")), _ptr(o.get("s_row")), _ptr(o.get("q_col")), _ptr(o.get("s_col")))
    if grad is None:
        st = lib().mx_quantize_gated_grouped(_ptr(x), N, ctypes.cast(rows, _vp), G, axis, act,
                                             *ptrs, _stream(dev, stream))
    else:
        st = lib().mx_quantize_dgated_grouped(_ptr(grad), _ptr(x), N, ctypes.cast(rows, _vp), G,
                                              axis, act, *ptrs, _stream(dev, stream))
    _check(st, "mx_quantize_gated_grouped")
    return {k: o.get(k) for k in ("q_row", "s_row", "q_col", "s_col")}
