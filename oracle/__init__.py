"""CPU oracle for bounds-checked tile movement -- TEST INFRASTRUCTURE ONLY.

Plain single-threaded C (``stg_oracle.c``) behind a numpy-facing ctypes
wrapper.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product library never does, and the two
share no code.  The definitions each function follows are documented in
``stg_oracle.h`` with their citations (page title and section).

Arrays are numpy arrays on the host.  bf16 and f16 data are carried as
``numpy.uint16`` bit patterns; the ``dtype`` names used here are
"f32", "bf16", "f16", "i32", "u8", "f64", "i64".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "stg_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libstg_oracle.so")

DTYPE_CODES = {"f32": 0, "bf16": 1, "f16": 2, "i32": 3, "u8": 4, "f64": 5, "i64": 6}
DTYPE_SIZES = {"f32": 4, "bf16": 2, "f16": 2, "i32": 4, "u8": 1, "f64": 8, "i64": 8}


def _stale() -> bool:
    if not os.path.exists(_LIB_PATH):
        return True
    built = os.path.getmtime(_LIB_PATH)
    return any(os.path.getmtime(os.path.join(_HERE, f)) > built for f in ("stg_oracle.c", "stg_oracle.h"))


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libstg_oracle.so`` (when
    forced, or when the library is missing or older than its source)."""
    if force or _stale():
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Array(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("esize", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_tile_grid": (_I64, [_I64, _I64, _I64]),
        "orc_round_to_format": (ctypes.c_uint64, [ctypes.c_double, ctypes.c_int, ctypes.c_int]),
        "orc_padding_bits": (ctypes.c_int, [ctypes.c_double, ctypes.c_int, _P]),
        "orc_tile_gather": (None, [_P, _P, _I64, _P, _P, _I32, _P]),
        "orc_tile_gather_masked": (None, [_P, _P, _P, _I64, _P, _P, _I32, _P, _P]),
        "orc_tile_scatter_masked": (None, [_P, _P, _P, _I64, _P, _P, _I32, _P]),
        "orc_tile_copy_bounded": (None, [_P, _I64, _I64, _I64, _I64, _P]),
        "orc_tile_store_clipped": (None, [_P, _I32, _I64, _I64, _I64, _I64, _P]),
        "orc_ragged_schedule": (_I64, [_P, _I64, _I32, _I32, _P, _P, _P]),
        "orc_ragged_tile_load": (None, [_P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _P]),
        "orc_tile_gather_backward": (None, [_P, _P, _I64, _P, _P, _I32, _P, _P, _P, _P]),
        "orc_tile_copy_windows": (None, [_P, _I64, _I64, _I64, _I64, _I64, _I64, _P]),
        "orc_tile_store_windows": (None, [_P, _I32, _I64, _I64, _I64, _I64, _I64, _I64, _P]),
        "orc_decode_lowp": (ctypes.c_double, [ctypes.c_uint8, _I32]),
        "orc_decode_scale": (ctypes.c_double, [ctypes.c_uint8, _I32]),
        "orc_gemm_scaled": (None, [_P, _I32, _I64, _P, _I64, _P, _I32, _I64, _P, _I64, _I32, _P, _I64, _I64, _I64,
                                   _I64, _I64, _P]),
        "orc_ragged_tile_store": (None, [_P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _P]),
        "orc_bf16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_gemm_f64": (None, [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64]),
        "orc_gemm_sample_f64": (None, [_P, _I64, _P, _I64, _I64, _P, _P, _I64, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(x: np.ndarray) -> int:
    return x.__array_interface__["data"][0]


def _arr(x: np.ndarray) -> _Array:
    """Describe a numpy array (any non-negative strides) to the oracle."""
    if x.ndim < 1 or x.ndim > 4:
        raise ValueError("rank must be 1..4")
    es = x.itemsize
    st = [s // es for s in x.strides]
    if any(s % es for s in x.strides) or any(s < 0 for s in st):
        raise ValueError("strides must be non-negative multiples of the element size")
    d = _Array()
    d.data = _ptr(x)
    d.esize = es
    d.rank = x.ndim
    for i in range(4):
        d.shape[i] = x.shape[i] if i < x.ndim else 1
        d.stride[i] = st[i] if i < x.ndim else 0
    return d


def _i64v(vals, n) -> np.ndarray:
    v = np.zeros(4, dtype=np.int64)
    v[:n] = np.asarray(vals, dtype=np.int64)
    return v


# ---- grid and rounding ------------------------------------------------------

def tile_grid(extent: int, origin: int, tile: int) -> int:
    return int(_load().orc_tile_grid(extent, origin, tile))


def round_to_format(v: float, ebits: int, mbits: int) -> int:
    return int(_load().orc_round_to_format(float(v), ebits, mbits))


def padding_bits(v: float, dtype: str) -> np.ndarray:
    """Padding value as one element of ``dtype`` (raw bytes, uint8 array)."""
    out = np.zeros(8, dtype=np.uint8)
    rc = _load().orc_padding_bits(float(v), DTYPE_CODES[dtype], _ptr(out))
    if rc != 0:
        raise ValueError(f"padding value {v!r} is not representable as {dtype}")
    return out[: DTYPE_SIZES[dtype]].copy()


# ---- gather / scatter -------------------------------------------------------

def _gather_out(a: np.ndarray, n_indices: int, tile_shape, axis: int) -> np.ndarray:
    shape = list(tile_shape)
    shape[axis] = n_indices
    return np.empty(shape, dtype=a.dtype)


def tile_gather(a, indices, tile_shape, offset=None, axis=0) -> np.ndarray:
    a = np.asarray(a)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    offset = [0] * a.ndim if offset is None else offset
    out = _gather_out(a, idx.size, tile_shape, axis)
    ad, od = _arr(a), _arr(out)
    ts, of = _i64v(tile_shape, a.ndim), _i64v(offset, a.ndim)
    _load().orc_tile_gather(ctypes.byref(ad), _ptr(idx), idx.size, _ptr(ts), _ptr(of), axis, ctypes.byref(od))
    return out


def tile_gather_masked(a, indices, mask, tile_shape, offset=None, axis=0, padding_value=0.0,
                       dtype="f32") -> np.ndarray:
    a = np.asarray(a)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    msk = np.ascontiguousarray(mask, dtype=np.uint8)
    assert msk.size == idx.size
    offset = [0] * a.ndim if offset is None else offset
    pad = padding_bits(padding_value, dtype)
    assert pad.size == a.itemsize
    out = _gather_out(a, idx.size, tile_shape, axis)
    ad, od = _arr(a), _arr(out)
    ts, of = _i64v(tile_shape, a.ndim), _i64v(offset, a.ndim)
    _load().orc_tile_gather_masked(ctypes.byref(ad), _ptr(idx), _ptr(msk), idx.size, _ptr(ts), _ptr(of),
                                   axis, _ptr(pad), ctypes.byref(od))
    return out


def tile_scatter_masked(a, indices, mask, tile_shape, tile, offset=None, axis=0) -> None:
    """Writes into ``a`` in place (``a`` may be a strided view)."""
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    msk = np.ascontiguousarray(mask, dtype=np.uint8)
    tile = np.asarray(tile)
    assert msk.size == idx.size and tile.dtype == a.dtype
    offset = [0] * a.ndim if offset is None else offset
    ad, td = _arr(a), _arr(tile)
    ts, of = _i64v(tile_shape, a.ndim), _i64v(offset, a.ndim)
    _load().orc_tile_scatter_masked(ctypes.byref(ad), _ptr(idx), _ptr(msk), idx.size, _ptr(ts), _ptr(of),
                                    axis, ctypes.byref(td))


# ---- bounded copy / clipped store -------------------------------------------

def tile_copy_bounded(src, tm: int, tn: int, origin_row: int, origin_col: int) -> np.ndarray:
    """Dense (G_r, G_c, tm, tn) tile buffer of ``src`` (a 2-D, possibly strided, view)."""
    assert src.ndim == 2
    gr = tile_grid(src.shape[0], origin_row, tm)
    gc = tile_grid(src.shape[1], origin_col, tn)
    out = np.empty((gr, gc, tm, tn), dtype=src.dtype)
    sd = _arr(src)
    _load().orc_tile_copy_bounded(ctypes.byref(sd), tm, tn, origin_row, origin_col, _ptr(out))
    return out


def tile_store_clipped(tiles, origin_row: int, origin_col: int, dst) -> None:
    """Clipped store of a dense (G_r, G_c, tm, tn) buffer into ``dst`` in place."""
    tiles = np.ascontiguousarray(tiles)
    assert tiles.ndim == 4 and dst.ndim == 2 and tiles.dtype == dst.dtype
    tm, tn = tiles.shape[2], tiles.shape[3]
    assert tiles.shape[0] == tile_grid(dst.shape[0], origin_row, tm)
    assert tiles.shape[1] == tile_grid(dst.shape[1], origin_col, tn)
    dd = _arr(dst)
    _load().orc_tile_store_clipped(_ptr(tiles), tiles.itemsize, tm, tn, origin_row, origin_col, ctypes.byref(dd))


def tile_gather_backward(a_grad, indices, tile_shape, grad_out, offset=None, axis=0):
    """Adjoint of tile_gather accumulated into a copy of ``a_grad`` (float32 or
    float64): returns (acc, abs_sum, count) -- the fp64 sums, the fp64 sum of
    magnitudes (initial |a_grad| plus every |term|) and the number of terms
    per element, all of a_grad's shape."""
    a_grad = np.asarray(a_grad)
    grad_out = np.asarray(grad_out)
    assert a_grad.dtype in (np.float32, np.float64) and grad_out.dtype == a_grad.dtype
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    offset = [0] * a_grad.ndim if offset is None else offset
    assert grad_out.shape == tuple(_gather_out(a_grad, idx.size, tile_shape, axis).shape)
    acc = np.ascontiguousarray(a_grad, dtype=np.float64).copy()
    abs_sum = np.abs(acc)
    count = np.zeros(a_grad.shape, dtype=np.int64)
    gd = _arr(grad_out)
    ts, of, sh = _i64v(tile_shape, a_grad.ndim), _i64v(offset, a_grad.ndim), _i64v(a_grad.shape, a_grad.ndim)
    _load().orc_tile_gather_backward(ctypes.byref(gd), _ptr(idx), idx.size, _ptr(ts), _ptr(of), axis, _ptr(sh),
                                     _ptr(acc), _ptr(abs_sum), _ptr(count))
    return acc, abs_sum, count


def tile_copy_windows(src, tm: int, tn: int, step_rows: int, step_cols: int, origin_row: int,
                      origin_col: int) -> np.ndarray:
    """Dense (G_r, G_c, tm, tn) buffer of the windows of ``src`` whose origins
    step by (step_rows, step_cols)."""
    assert src.ndim == 2
    gr = tile_grid(src.shape[0], origin_row, step_rows)
    gc = tile_grid(src.shape[1], origin_col, step_cols)
    out = np.empty((gr, gc, tm, tn), dtype=src.dtype)
    sd = _arr(src)
    _load().orc_tile_copy_windows(ctypes.byref(sd), tm, tn, step_rows, step_cols, origin_row, origin_col, _ptr(out))
    return out


def tile_store_windows(tiles, step_rows: int, step_cols: int, origin_row: int, origin_col: int, dst) -> None:
    """Clipped store of every window of a dense (G_r, G_c, tm, tn) buffer into ``dst`` in place."""
    tiles = np.ascontiguousarray(tiles)
    assert tiles.ndim == 4 and dst.ndim == 2 and tiles.dtype == dst.dtype
    tm, tn = tiles.shape[2], tiles.shape[3]
    assert tiles.shape[0] == tile_grid(dst.shape[0], origin_row, step_rows)
    assert tiles.shape[1] == tile_grid(dst.shape[1], origin_col, step_cols)
    dd = _arr(dst)
    _load().orc_tile_store_windows(_ptr(tiles), tiles.itemsize, tm, tn, step_rows, step_cols, origin_row, origin_col,
                                   ctypes.byref(dd))


# ---- ragged ----------------------------------------------------------------

def ragged_schedule(seq_lens, bm_seq: int, middle_dim: int):
    lens = np.ascontiguousarray(seq_lens, dtype=np.int64)
    lib = _load()
    n = int(lib.orc_ragged_schedule(_ptr(lens), lens.size, bm_seq, middle_dim, None, None, None))
    ri = np.zeros(n, dtype=np.uint32)
    dyn = np.zeros(n, dtype=np.uint32)
    mi = np.zeros(n, dtype=np.uint32)
    if n:
        lib.orc_ragged_schedule(_ptr(lens), lens.size, bm_seq, middle_dim, _ptr(ri), _ptr(dyn), _ptr(mi))
    return ri, dyn, mi


def ragged_tile_load(X, middle_dim: int, group: int, BM: int, BN: int, col0: int, ri, dyn, mi) -> np.ndarray:
    """X is contiguous (total_rows, middle_dim*group, depth); returns (n_tiles, BM, BN)."""
    X = np.ascontiguousarray(X)
    assert X.ndim == 3 and X.shape[1] == middle_dim * group
    ri = np.ascontiguousarray(ri, dtype=np.uint32)
    dyn = np.ascontiguousarray(dyn, dtype=np.uint32)
    mi = np.ascontiguousarray(mi, dtype=np.uint32)
    n = ri.size
    out = np.empty((n, BM, BN), dtype=X.dtype)
    _load().orc_ragged_tile_load(_ptr(X), X.itemsize, X.shape[0], middle_dim, group, X.shape[2], BM, BN, col0,
                                 _ptr(ri), _ptr(dyn), _ptr(mi), n, _ptr(out))
    return out


def ragged_tile_store(tiles, X, middle_dim: int, group: int, col0: int, ri, dyn, mi) -> np.ndarray:
    """tiles (n_tiles, BM, BN) into a copy of X (total_rows, middle_dim*group,
    depth); returns the updated copy (elements no tile writes keep X's bits)."""
    tiles = np.ascontiguousarray(tiles)
    out = np.array(X, copy=True, order="C")
    assert out.ndim == 3 and out.shape[1] == middle_dim * group and tiles.ndim == 3
    assert tiles.dtype == out.dtype
    ri = np.ascontiguousarray(ri, dtype=np.uint32)
    dyn = np.ascontiguousarray(dyn, dtype=np.uint32)
    mi = np.ascontiguousarray(mi, dtype=np.uint32)
    n, BM, BN = tiles.shape
    assert ri.size == n and dyn.size == n and mi.size == n
    _load().orc_ragged_tile_store(_ptr(tiles), out.itemsize, out.shape[0], middle_dim, group, out.shape[2], BM, BN,
                                  col0, _ptr(ri), _ptr(dyn), _ptr(mi), n, _ptr(out))
    return out


# ---- block-scaled GEMM -------------------------------------------------------

LOWP = {"e4m3": 0, "e5m2": 1, "e2m1": 2}
SCALES = {"e8m0": 0, "e4m3": 1}


def decode_lowp(codes, fmt: str) -> np.ndarray:
    """Exact fp64 values of e4m3 / e5m2 / e2m1 codes (e2m1: low 4 bits of each code)."""
    codes = np.asarray(codes, dtype=np.uint8)
    lib = _load()
    return np.array([lib.orc_decode_lowp(int(c), LOWP[fmt]) for c in codes.ravel()]).reshape(codes.shape)


def decode_scale(codes, fmt: str) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    lib = _load()
    return np.array([lib.orc_decode_scale(int(c), SCALES[fmt]) for c in codes.ravel()]).reshape(codes.shape)


def gemm_scaled_f64(A, a_fmt, a_scale, Bt, b_fmt, b_scale, K: int, block: int, s_fmt="e8m0", acc=None) -> np.ndarray:
    """fp64 (A . a_scale)(B . b_scale) + acc.  A: uint8 (M, bytes per row), Bt:
    uint8 (N, bytes per row) = B transposed, K-major; e2m1 packs two values per
    byte (low nibble first); scales uint8 (M, K/block) and (N, K/block)."""
    A, Bt = np.ascontiguousarray(A, dtype=np.uint8), np.ascontiguousarray(Bt, dtype=np.uint8)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.uint8)
    b_scale = np.ascontiguousarray(b_scale, dtype=np.uint8)
    M, N = A.shape[0], Bt.shape[0]
    assert K % block == 0 and a_scale.shape == (M, K // block) and b_scale.shape == (N, K // block)
    C = np.empty((M, N), dtype=np.float64)
    accp, ldacc = None, 0
    if acc is not None:
        acc = np.ascontiguousarray(acc, dtype=np.float32)
        accp, ldacc = _ptr(acc), acc.shape[1]
    _load().orc_gemm_scaled(_ptr(A), LOWP[a_fmt], A.shape[1], _ptr(a_scale), a_scale.shape[1], _ptr(Bt), LOWP[b_fmt],
                            Bt.shape[1], _ptr(b_scale), b_scale.shape[1], SCALES[s_fmt], accp, ldacc, M, N, K, block,
                            _ptr(C))
    return C


# ---- GEMM ------------------------------------------------------------------

def bf16_to_f64(h: int) -> float:
    return float(_load().orc_bf16_to_f64(int(h)))


def gemm_f64(A, B) -> np.ndarray:
    """fp64 C = A.B for bf16 bit arrays A (M,K) and B (K,N) (row views, unit column stride)."""
    assert A.dtype == np.uint16 and B.dtype == np.uint16
    assert A.strides[1] == 2 and B.strides[1] == 2
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    C = np.empty((M, N), dtype=np.float64)
    _load().orc_gemm_f64(_ptr(A), A.strides[0] // 2, _ptr(B), B.strides[0] // 2, _ptr(C), N, M, N, K)
    return C


def gemm_sample_f64(A, B, rows, cols) -> np.ndarray:
    assert A.dtype == np.uint16 and B.dtype == np.uint16
    assert A.strides[1] == 2 and B.strides[1] == 2
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(r.size, dtype=np.float64)
    _load().orc_gemm_sample_f64(_ptr(A), A.strides[0] // 2, _ptr(B), B.strides[0] // 2, A.shape[1],
                                _ptr(r), _ptr(c), r.size, _ptr(out))
    return out


def f64_to_bf16_bits(c64: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 bit patterns, to nearest even (element by element)."""
    flat = np.asarray(c64, dtype=np.float64).ravel()
    lib = _load()
    out = np.fromiter((lib.orc_round_to_format(float(v), 8, 7) for v in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(np.shape(c64))
