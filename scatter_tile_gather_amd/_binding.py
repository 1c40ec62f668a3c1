"""ctypes binding of libstg.so: argument marshalling only.

Each function here has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU (PyTorch supplies device memory and the stream);
nothing is computed in Python and there is no fallback: if the HIP library is
missing or a tensor is not on the GPU the call raises.
"""
from __future__ import annotations

import ctypes
import os
import struct
import threading

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstg.so")

STG_F32, STG_BF16, STG_F16, STG_I32, STG_U8, STG_F64, STG_I64 = range(7)


class StgError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[stg status {code}] {message}")
        self.code = code


class StgTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
# const stg_tensor* and const int64_t[4] arguments: passed as the bytes of
# the structure or array (ctypes hands the C side a pointer to them), which
# converts faster than a typed pointer; byref() of a StgTensor is accepted too
_TP = ctypes.c_void_p
_C64 = ctypes.c_void_p
_I64P = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "stg_version": (ctypes.c_int, []),
    "stg_last_error": (ctypes.c_char_p, []),
    "stg_tile_grid": (_I64, [_I64, _I64, _I64]),
    "tile_gather": (ctypes.c_int, [_TP, _P, _I64, _C64, _C64, _I32, _TP, _P]),
    "tile_gather_masked": (ctypes.c_int, [_TP, _P, _P, _I64, _C64, _C64, _I32, ctypes.c_double, _TP, _P]),
    "tile_scatter_masked": (ctypes.c_int, [_TP, _P, _P, _I64, _C64, _C64, _I32, _TP, _P]),
    "tile_gather_backward": (ctypes.c_int, [_TP, _P, _I64, _C64, _C64, _I32, _TP, _P, _I64, _P]),
    "tile_gather_backward_workspace": (_I64, [_TP, _I64, _C64, _I32]),
    "tile_gather_backward_static": (ctypes.c_int, [_TP, _P, _I64, _C64, _C64, _I32, _TP, _P]),
    "tile_copy_bounded": (ctypes.c_int, [_TP, _I64, _I64, _I64, _I64, _P, _P]),
    "tile_store_clipped": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _TP, _P]),
    "tile_copy_windows": (ctypes.c_int, [_TP, _I64, _I64, _I64, _I64, _I64, _I64, _I32, _P, _P]),
    "tile_store_windows": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _I64, _I64, _I32, _TP, _P]),
    "ragged_tile_schedule": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _I64P]),
    "ragged_tile_load": (ctypes.c_int, [_P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _P, _P]),
    "ragged_tile_store": (ctypes.c_int, [_P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _P, _P]),
    "gemm_bounded": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I32, _P]),
    "gemm_scaled": (ctypes.c_int, [_P, _I32, _I64, _P, _I64, _P, _I32, _I64, _P, _I64, _I32, _I64, _P, _I64, _P, _I64,
                                   _I64, _I64, _I64, _P]),
    "gemm_scaled_ws": (ctypes.c_int, [_P, _I32, _I64, _P, _I64, _P, _I32, _I64, _P, _I64, _I32, _I64, _P, _I64, _P,
                                      _I64, _I64, _I64, _I64, _P, _I64, _P]),
    "gemm_scaled_workspace": (_I64, [_I32, _I32, _I32, _I64, _I64, _I64, _I64]),
    "stg_trace_enable": (ctypes.c_int, [ctypes.c_int]),
    "stg_trace_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]),
}

_lib = None


def load_library() -> ctypes.CDLL:
    """Load the in-tree libstg.so (built by scatter_tile_gather_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libstg.so is not built ({LIB_PATH}); run scatter_tile_gather_amd.build.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_names():
    return list(_SIGNATURES)


_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch

        _TORCH = torch
    return _TORCH


_DTYPES = None  # torch dtype -> stg_dtype, built on first use


def _dtype_code(t) -> int:
    global _DTYPES
    if _DTYPES is None:
        torch = _torch()
        _DTYPES = {
            torch.float32: STG_F32,
            torch.bfloat16: STG_BF16,
            torch.float16: STG_F16,
            torch.int32: STG_I32,
            torch.uint8: STG_U8,
            torch.float64: STG_F64,
            torch.int64: STG_I64,
        }
    code = _DTYPES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def _on_gpu(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")


# stg_tensor's bytes: data, dtype, rank, shape[4], stride[4] (no padding);
# packing them in one call is several times faster than building the
# structure field by field, which small latency-bound calls feel
_DESC = struct.Struct("<Qii4q4q")
assert _DESC.size == ctypes.sizeof(StgTensor)
_ONES = ((), (1,), (1, 1), (1, 1, 1))
_ZEROS = ((), (0,), (0, 0), (0, 0, 0))


def _desc(t, name: str) -> bytes:
    """The stg_tensor of GPU tensor `t`, as the structure's bytes."""
    _on_gpu(t, name)
    shape = t.shape
    r = len(shape)
    if r < 1 or r > 4:
        raise ValueError(f"{name}: rank must be 1..4")
    pad = 4 - r
    return _DESC.pack(t.data_ptr(), _dtype_code(t), r, *shape, *_ONES[pad], *t.stride(), *_ZEROS[pad])


_I64x4 = struct.Struct("<4q")
_I64_CACHE = {}


def _i64arr(vals) -> bytes:
    """A tile shape or offset as the bytes of an int64_t[4] (zero-padded).
    The C side only reads these arrays, so one immutable copy per distinct
    value is kept and reused: a repeated call skips the packing."""
    key = vals if type(vals) is tuple else tuple(vals)
    b = _I64_CACHE.get(key)
    if b is None:
        if len(key) > 4:
            raise ValueError("a tile shape or offset has at most 4 entries")
        b = _I64x4.pack(*(int(v) for v in key), *(0,) * (4 - len(key)))
        if len(_I64_CACHE) >= 4096:
            _I64_CACHE.clear()
        _I64_CACHE[key] = b
    return b


_RAW_STREAM = None


def _stream(stream, like=None, device=None) -> int:
    """The HIP stream to enqueue on: `stream`'s, else the current stream of the
    device `like` lives on (or of `device`, or of the current device)."""
    global _RAW_STREAM
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    if _RAW_STREAM is None:
        # torch's raw-stream accessor skips building a Stream object per call
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    dev = like.get_device() if like is not None else device if device is not None else torch.cuda.current_device()
    if _RAW_STREAM:
        return _RAW_STREAM(dev)
    return torch.cuda.current_stream(dev).cuda_stream


# per host thread: the list of recorded (name, C function, arguments) while
# prepare() runs on that thread, else None; calls from other threads meanwhile
# run as usual.  _TLS.keep: tensors an entry point allocated for itself while
# being prepared (an "auto" workspace), held by the Prepared object.
_TLS = threading.local()


def _capturing():
    return getattr(_TLS, "capture", None)


def _workspace(nbytes: int, device, stream):
    """An "auto" workspace of nbytes: allocated on the stream the kernels run
    on, so that once the caller drops it the caching allocator hands the
    block out again only to work queued on that stream after them; while
    prepare() records the call, kept for the prepared call's lifetime."""
    torch = _torch()
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(device)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if _capturing() is not None:
        _TLS.keep.append(ws)
    return ws


def _call(name: str, *args):
    """Invoke the C entry point `name` (its last argument is the stream) and
    raise on failure -- or, while prepare() runs on this thread, record the
    call instead."""
    fn = getattr(load_library(), name)
    cap = _capturing()
    if cap is not None:
        cap.append((name, fn, args))
        return
    _check(fn(*args))


class Prepared:
    """An entry-point call whose argument marshalling (tensor descriptors,
    shape and offset arrays, checks, output allocation) was done once by
    prepare(); calling it enqueues the same operation again, on the stream
    given at preparation or else on the current stream of the device the
    operands live on.  It holds references to every tensor involved, so they
    stay allocated.  The tensors' contents may change between calls; their
    storage, shapes and strides must not."""

    __slots__ = ("calls", "result", "keep", "stream", "device")

    def __init__(self, calls, result, keep, stream, device):
        self.calls = calls
        self.result = result
        self.keep = keep
        self.stream = stream
        self.device = device

    def __call__(self):
        s = self.stream.cuda_stream if self.stream is not None else _stream(None, None, self.device)
        for name, fn, args in self.calls:
            rc = fn(*args[:-1], s)
            if rc != 0:
                raise StgError(rc, load_library().stg_last_error().decode())
        return self.result


def prepare(op, *args, **kwargs):
    """Prepare `op(*args, **kwargs)` (one of this module's entry points, with
    the same arguments) for repeated calls: marshalling and checks run now and
    the C call is recorded, not made; the returned Prepared object enqueues it
    each time it is called and returns what `op` returns.  For latency-bound
    callers (small gathers) this removes the per-call argument marshalling."""
    torch = _torch()
    if _capturing() is not None:
        raise RuntimeError("prepare() does not nest")
    _TLS.capture, _TLS.keep = [], []
    try:
        result = op(*args, **kwargs)
        calls, kept = _TLS.capture, _TLS.keep
    finally:
        _TLS.capture, _TLS.keep = None, None
    if not calls:
        raise ValueError(f"{getattr(op, '__name__', op)} makes no device call with these arguments")
    tensors = [x for x in list(args) + list(kwargs.values()) if isinstance(x, torch.Tensor)]
    device = next((t.get_device() for t in tensors if t.is_cuda), torch.cuda.current_device())
    return Prepared(calls, result, (args, kwargs, result, kept), kwargs.get("stream"), device)


def _check(rc: int):
    if rc != 0:
        raise StgError(rc, load_library().stg_last_error().decode())


def _dev_array(x, dtype, name: str):
    _on_gpu(x, name)
    if x.dtype != dtype or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor")
    return x.data_ptr()


# ---- entry points -----------------------------------------------------------

def stg_trace_enable(on: bool = True) -> bool:
    """Per-launch kernel timing on this thread; returns the previous setting."""
    return bool(load_library().stg_trace_enable(1 if on else 0))


def stg_trace_read(cap: int = 4096):
    """[(kernel name, milliseconds)] recorded since the last read; synchronise first."""
    lib = load_library()
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = lib.stg_trace_read(cap, names, ms)
    if n < 0:
        raise StgError(-n, lib.stg_last_error().decode())
    return [(names[i].decode(), float(ms[i])) for i in range(n)]


def stg_version() -> int:
    return int(load_library().stg_version())


def stg_tile_grid(extent: int, origin: int, tile: int) -> int:
    return int(load_library().stg_tile_grid(extent, origin, tile))


def _gather_out_shape(tile_shape, n, axis):
    shape = list(tile_shape)
    shape[axis] = n
    return shape


_FAST = None  # the C++ marshalling module (_stg_fast), loaded on first use


def _fast():
    global _FAST
    if _FAST is None:
        from . import _stg_fast

        _FAST = (_stg_fast.tile_gather, ctypes.cast(load_library().tile_gather, ctypes.c_void_p).value)
    return _FAST


def tile_gather(a, indices, tile_shape, offset=None, axis: int = 0, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty(_gather_out_shape(tile_shape, indices.numel(), axis), dtype=a.dtype, device=a.device)
    if _capturing() is None:
        # eager: the same checks and call, marshalled in C++ (this call is
        # latency-bound; see csrc/fastcall.cpp)
        fn, addr = _FAST or _fast()
        rc = fn(addr, a, indices, out, tile_shape, offset, axis, None if stream is None else stream.cuda_stream)
        if rc:
            raise StgError(rc, load_library().stg_last_error().decode())
        return out
    n = indices.numel()
    ad, od = _desc(a, "a"), _desc(out, "out")
    _call("tile_gather", ad, _dev_array(indices, torch.int32, "indices"), n, _i64arr(tile_shape),
                           None if offset is None else _i64arr(offset), axis, od, _stream(stream, a))
    return out


def tile_gather_masked(a, indices, mask, tile_shape, offset=None, axis: int = 0, padding_value: float = 0.0,
                       out=None, stream=None):
    torch = _torch()
    lib = load_library()
    n = indices.numel()
    if out is None:
        out = torch.empty(_gather_out_shape(tile_shape, n, axis), dtype=a.dtype, device=a.device)
    ad, od = _desc(a, "a"), _desc(out, "out")
    if mask is not None and mask.numel() != n:
        raise ValueError("mask must hold one entry per index")
    mp = None if mask is None else _dev_array(mask, torch.uint8, "mask")
    _call("tile_gather_masked", ad, _dev_array(indices, torch.int32, "indices"), mp, n,
                                  _i64arr(tile_shape), None if offset is None else _i64arr(offset), axis,
                                  float(padding_value), od, _stream(stream, a))
    return out


def tile_gather_backward_workspace(a_grad, n_indices: int, tile_shape, axis: int = 0) -> int:
    """Bytes of workspace the grouped execution needs; 0 when the layout always
    runs on atomics."""
    lib = load_library()
    ad = _desc(a_grad, "a_grad")
    n = int(lib.tile_gather_backward_workspace(ad, n_indices, _i64arr(tile_shape), axis))
    if n < 0:
        raise StgError(-n, lib.stg_last_error().decode())
    return n


def tile_gather_backward(a_grad, indices, tile_shape, grad_out, offset=None, axis: int = 0, workspace=None,
                         stream=None):
    """a_grad += adjoint of tile_gather(a, indices, tile_shape, offset, axis) for
    the output gradient grad_out (fp32 or fp64).  workspace: None (hardware
    float atomics), a device uint8 tensor of at least
    tile_gather_backward_workspace(...) bytes, or "auto" to allocate one here
    (grouped execution: each row summed and stored once; float atomics only
    for the pieces of rows with more than 64 terms)."""
    torch = _torch()
    lib = load_library()
    n = indices.numel()
    ad, gd = _desc(a_grad, "a_grad"), _desc(grad_out, "grad_out")
    if isinstance(workspace, str) and workspace == "auto":
        nb = tile_gather_backward_workspace(a_grad, n, tile_shape, axis)
        workspace = _workspace(nb, a_grad.device, stream) if nb else None
    ws_ptr, ws_n = None, 0
    if workspace is not None:
        _on_gpu(workspace, "workspace")
        ws_ptr, ws_n = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _call("tile_gather_backward", ad, _dev_array(indices, torch.int32, "indices"), n,
                                    _i64arr(tile_shape), None if offset is None else _i64arr(offset), axis,
                                    gd, ws_ptr, ws_n, _stream(stream, a_grad))
    return a_grad


# bytes of the library's static scratch array (STG_STATIC_SCRATCH_BYTES in stg.h)
STATIC_SCRATCH_BYTES = 64 << 20


def tile_gather_backward_static(a_grad, indices, tile_shape, grad_out, offset=None, axis: int = 0, stream=None):
    """tile_gather_backward's grouped execution with its scratch in the
    library's static device array instead of a workspace: nothing is
    allocated.  Calls needing more than STATIC_SCRATCH_BYTES raise StgError
    (STG_ERR_RANGE); calls that overlap in time on one GPU race."""
    torch = _torch()
    lib = load_library()
    ad, gd = _desc(a_grad, "a_grad"), _desc(grad_out, "grad_out")
    # the library takes the current device's static array: make it a_grad's
    with torch.cuda.device(a_grad.device):
        _call("tile_gather_backward_static", ad, _dev_array(indices, torch.int32, "indices"),
              indices.numel(), _i64arr(tile_shape), None if offset is None else _i64arr(offset), axis,
              gd, _stream(stream, a_grad))
    return a_grad


def tile_scatter_masked(a, indices, mask, tile_shape, tile, offset=None, axis: int = 0, stream=None):
    torch = _torch()
    lib = load_library()
    n = indices.numel()
    ad, td = _desc(a, "a"), _desc(tile, "tile")
    if mask is not None and mask.numel() != n:
        raise ValueError("mask must hold one entry per index")
    mp = None if mask is None else _dev_array(mask, torch.uint8, "mask")
    _call("tile_scatter_masked", ad, _dev_array(indices, torch.int32, "indices"), mp, n,
                                   _i64arr(tile_shape), None if offset is None else _i64arr(offset), axis,
                                   td, _stream(stream, a))
    return a


def tile_copy_bounded(src, tile_rows: int, tile_cols: int, origin_row: int = 0, origin_col: int = 0, out=None,
                      stream=None):
    torch = _torch()
    lib = load_library()
    if src.dim() != 2:
        raise ValueError("src must be 2-D")
    gr = stg_tile_grid(src.shape[0], origin_row, tile_rows)
    gc = stg_tile_grid(src.shape[1], origin_col, tile_cols)
    if out is None:
        out = torch.empty((max(gr, 0), max(gc, 0), tile_rows, tile_cols), dtype=src.dtype, device=src.device)
    _on_gpu(out, "out")
    if out.dtype != src.dtype or not out.is_contiguous() or out.numel() < max(gr, 0) * max(gc, 0) * tile_rows * tile_cols:
        raise ValueError("out must be a contiguous tile buffer of the source dtype and grid size")
    sd = _desc(src, "src")
    _call("tile_copy_bounded", sd, tile_rows, tile_cols, origin_row, origin_col, out.data_ptr(),
                                 _stream(stream, src))
    return out


def tile_copy_windows(src, tile_rows: int, tile_cols: int, step_rows: int, step_cols: int, origin_row: int = 0,
                      origin_col: int = 0, check_bounds: bool = True, out=None, stream=None):
    """Windows of src whose origins step by (step_rows, step_cols); (G_r, G_c, tile_rows, tile_cols)."""
    torch = _torch()
    lib = load_library()
    if src.dim() != 2:
        raise ValueError("src must be 2-D")
    gr = stg_tile_grid(src.shape[0], origin_row, step_rows)
    gc = stg_tile_grid(src.shape[1], origin_col, step_cols)
    if out is None:
        out = torch.empty((max(gr, 0), max(gc, 0), tile_rows, tile_cols), dtype=src.dtype, device=src.device)
    _on_gpu(out, "out")
    if out.dtype != src.dtype or not out.is_contiguous() or out.numel() < max(gr, 0) * max(gc, 0) * tile_rows * tile_cols:
        raise ValueError("out must be a contiguous tile buffer of the source dtype and grid size")
    sd = _desc(src, "src")
    _call("tile_copy_windows", sd, tile_rows, tile_cols, step_rows, step_cols, origin_row, origin_col,
                                 1 if check_bounds else 0, out.data_ptr(), _stream(stream, src))
    return out


def tile_store_windows(tiles, step_rows: int, step_cols: int, origin_row: int, origin_col: int, dst,
                       check_bounds: bool = True, stream=None):
    lib = load_library()
    _on_gpu(tiles, "tiles")
    if tiles.dim() != 4 or not tiles.is_contiguous() or tiles.dtype != dst.dtype:
        raise ValueError("tiles must be a contiguous (G_r, G_c, tile_rows, tile_cols) buffer of dst's dtype")
    tr, tc = tiles.shape[2], tiles.shape[3]
    if (tiles.shape[0], tiles.shape[1]) != (stg_tile_grid(dst.shape[0], origin_row, step_rows),
                                            stg_tile_grid(dst.shape[1], origin_col, step_cols)):
        raise ValueError("tile buffer grid does not match dst, step and origin")
    dd = _desc(dst, "dst")
    _call("tile_store_windows", tiles.data_ptr(), tr, tc, step_rows, step_cols, origin_row, origin_col,
                                  1 if check_bounds else 0, dd, _stream(stream, dst))
    return dst


def tile_store_clipped(tiles, origin_row: int, origin_col: int, dst, stream=None):
    lib = load_library()
    _on_gpu(tiles, "tiles")
    if tiles.dim() != 4 or not tiles.is_contiguous() or tiles.dtype != dst.dtype:
        raise ValueError("tiles must be a contiguous (G_r, G_c, tile_rows, tile_cols) buffer of dst's dtype")
    tr, tc = tiles.shape[2], tiles.shape[3]
    if (tiles.shape[0], tiles.shape[1]) != (stg_tile_grid(dst.shape[0], origin_row, tr),
                                            stg_tile_grid(dst.shape[1], origin_col, tc)):
        raise ValueError("tile buffer grid does not match dst and origin")
    dd = _desc(dst, "dst")
    _call("tile_store_clipped", tiles.data_ptr(), tr, tc, origin_row, origin_col, dd,
                                  _stream(stream, dst))
    return dst


def ragged_tile_schedule(seq_lens, bm_seq: int, middle_dim: int):
    """Host helper: (ragged_idx, dynamic_dim, middle_idx) uint32 numpy arrays."""
    lib = load_library()
    lens = np.ascontiguousarray(seq_lens, dtype=np.int64)
    n = ctypes.c_int64(0)
    lp = lens.ctypes.data if lens.size else None
    _check(lib.ragged_tile_schedule(lp, lens.size, bm_seq, middle_dim, None, None, None, ctypes.byref(n)))
    ri = np.zeros(n.value, dtype=np.uint32)
    dyn = np.zeros(n.value, dtype=np.uint32)
    mi = np.zeros(n.value, dtype=np.uint32)
    if n.value:
        _check(lib.ragged_tile_schedule(lp, lens.size, bm_seq, middle_dim, ri.ctypes.data, dyn.ctypes.data,
                                        mi.ctypes.data, ctypes.byref(n)))
    return ri, dyn, mi


def ragged_tile_load(src, middle_dim: int, group: int, BM: int, BN: int, ragged_idx, dynamic_dim, middle_idx,
                     col0: int = 0, out=None, stream=None):
    """src: contiguous (total_rows, middle_dim*group, depth); triples: device int32/uint32-valued tensors."""
    torch = _torch()
    lib = load_library()
    _on_gpu(src, "src")
    if src.dim() != 3 or not src.is_contiguous() or src.shape[1] != middle_dim * group:
        raise ValueError("src must be contiguous (total_rows, middle_dim*group, depth)")
    n = ragged_idx.numel()
    if dynamic_dim.numel() != n or middle_idx.numel() != n:
        raise ValueError("ragged triples must have equal lengths")
    if out is None:
        out = torch.empty((n, BM, BN), dtype=src.dtype, device=src.device)
    for t, nm in ((ragged_idx, "ragged_idx"), (dynamic_dim, "dynamic_dim"), (middle_idx, "middle_idx")):
        _on_gpu(t, nm)
        if t.dtype not in (torch.int32, torch.uint32) or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous 32-bit integer tensor")
    _on_gpu(out, "out")
    if out.dtype != src.dtype or not out.is_contiguous() or out.numel() < n * BM * BN:
        raise ValueError("out must be a contiguous (n_tiles, BM, BN) tensor of src's dtype")
    _call("ragged_tile_load", src.data_ptr(), _dtype_code(src), src.shape[0], middle_dim, group, src.shape[2], BM,
                                BN, col0, ragged_idx.data_ptr(), dynamic_dim.data_ptr(), middle_idx.data_ptr(), n,
                                out.data_ptr(), _stream(stream, src))
    return out


def ragged_tile_store(tiles, dst, middle_dim: int, group: int, ragged_idx, dynamic_dim, middle_idx, col0: int = 0,
                      stream=None):
    """tiles: (n_tiles, BM, BN) on the device; dst: contiguous (total_rows,
    middle_dim*group, depth) of the same dtype, written in place; triples:
    device int32/uint32-valued tensors.  Returns dst."""
    torch = _torch()
    lib = load_library()
    _on_gpu(tiles, "tiles")
    _on_gpu(dst, "dst")
    if dst.dim() != 3 or not dst.is_contiguous() or dst.shape[1] != middle_dim * group:
        raise ValueError("dst must be contiguous (total_rows, middle_dim*group, depth)")
    if tiles.dim() != 3 or not tiles.is_contiguous() or tiles.dtype != dst.dtype:
        raise ValueError("tiles must be a contiguous (n_tiles, BM, BN) tensor of dst's dtype")
    n, BM, BN = tiles.shape
    for t, nm in ((ragged_idx, "ragged_idx"), (dynamic_dim, "dynamic_dim"), (middle_idx, "middle_idx")):
        _on_gpu(t, nm)
        if t.dtype not in (torch.int32, torch.uint32) or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{nm} must be a contiguous 32-bit integer tensor with one entry per tile")
    _call("ragged_tile_store", tiles.data_ptr(), _dtype_code(dst), dst.shape[0], middle_dim, group, dst.shape[2], BM,
                                 BN, col0, ragged_idx.data_ptr(), dynamic_dim.data_ptr(), middle_idx.data_ptr(), n,
                                 dst.data_ptr(), _stream(stream, dst))
    return dst


def gemm_bounded(A, B, out=None, out_dtype=None, stream=None):
    """C = A @ B for bf16 A (M, K) and B (K, N) views with unit column stride."""
    torch = _torch()
    lib = load_library()
    _on_gpu(A, "A")
    _on_gpu(B, "B")
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16 or A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D bf16 tensors")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if (A.stride(1) != 1 and K > 1) or (B.stride(1) != 1 and N > 1):
        raise ValueError("A and B need unit column stride")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=A.device)
    _on_gpu(out, "out")
    if out.dim() != 2 or tuple(out.shape) != (M, N) or (out.stride(1) != 1 and N > 1):
        raise ValueError("out must be (M, N) with unit column stride")
    code = _dtype_code(out)
    _call("gemm_bounded", A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0), out.data_ptr(), out.stride(0), M,
                            N, K, code, _stream(stream, A))
    return out


LOWP_FORMATS = {"e4m3": 0, "e5m2": 1, "e2m1": 2}
SCALE_FORMATS = {"e8m0": 0, "e4m3": 1}


def gemm_scaled_workspace(a_fmt: str, b_fmt: str, scale_fmt: str, block: int, M: int, N: int, K: int) -> int:
    n = int(load_library().gemm_scaled_workspace(LOWP_FORMATS[a_fmt], LOWP_FORMATS[b_fmt], SCALE_FORMATS[scale_fmt],
                                                 block, M, N, K))
    if n < 0:
        raise StgError(-n, load_library().stg_last_error().decode())
    return n


def gemm_scaled(A, a_fmt: str, a_scale, Bt, b_fmt: str, b_scale, K: int, block: int, scale_fmt: str = "e8m0",
                acc=None, out=None, workspace="auto", stream=None):
    """C = (A . a_scale)(B . b_scale) + acc, fp32.  A: uint8 (M, >= K*bits/8)
    operand codes (e2m1: two per byte, even element low); Bt: uint8 (N, ...)
    = B K-major; scales uint8 (M, >= K/block) and (N, >= K/block); acc / out
    float32 (M, N).  workspace: "auto" (allocated here where
    gemm_scaled_workspace asks for one: the general path then decodes each
    operand once to bf16 before the bf16 GEMM), a device uint8 tensor of at
    least that many bytes, or None (no workspace: values decoded inside the
    GEMM kernel)."""
    torch = _torch()
    lib = load_library()
    for t, nm in ((A, "A"), (Bt, "Bt"), (a_scale, "a_scale"), (b_scale, "b_scale")):
        _on_gpu(t, nm)
        if t.dtype != torch.uint8 or t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
            raise ValueError(f"{nm} must be a 2-D uint8 tensor with unit column stride")
    M, N = A.shape[0], Bt.shape[0]
    if block < 1 or K < 0 or K % block:
        raise ValueError("K must be a non-negative multiple of block")
    bits_a, bits_b = (4 if a_fmt == "e2m1" else 8), (4 if b_fmt == "e2m1" else 8)
    if A.shape[1] * 8 < K * bits_a or Bt.shape[1] * 8 < K * bits_b:
        raise ValueError("A and Bt rows must hold K values")
    if tuple(a_scale.shape[:1]) != (M,) or tuple(b_scale.shape[:1]) != (N,) or \
            a_scale.shape[1] < K // block or b_scale.shape[1] < K // block:
        raise ValueError("a_scale must be (M, >= K/block) and b_scale (N, >= K/block)")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _on_gpu(out, "out")
    if out.dtype != torch.float32 or tuple(out.shape) != (M, N) or (out.stride(1) != 1 and N > 1):
        raise ValueError("out must be float32 (M, N) with unit column stride")
    accp, ldacc = None, 0
    if acc is not None:
        _on_gpu(acc, "acc")
        if acc.dtype != torch.float32 or tuple(acc.shape) != (M, N) or (acc.stride(1) != 1 and N > 1):
            raise ValueError("acc must be float32 (M, N) with unit column stride")
        accp, ldacc = acc.data_ptr(), acc.stride(0)
    if isinstance(workspace, str) and workspace == "auto":
        nb = gemm_scaled_workspace(a_fmt, b_fmt, scale_fmt, block, M, N, K)
        workspace = _workspace(nb, A.device, stream) if nb else None
    ws_ptr, ws_n = None, 0
    if workspace is not None:
        _on_gpu(workspace, "workspace")
        ws_ptr, ws_n = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _call("gemm_scaled_ws", A.data_ptr(), LOWP_FORMATS[a_fmt], A.stride(0), a_scale.data_ptr(), a_scale.stride(0),
                              Bt.data_ptr(), LOWP_FORMATS[b_fmt], Bt.stride(0), b_scale.data_ptr(), b_scale.stride(0),
                              SCALE_FORMATS[scale_fmt], block, accp, ldacc, out.data_ptr(), out.stride(0), M, N, K,
                              ws_ptr, ws_n, _stream(stream, A))
    return out
