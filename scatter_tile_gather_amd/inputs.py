"""Seeded synthetic inputs for the tile-movement workloads.

This module is shared by the tests, the benchmark and the oracle-side checks,
so it holds none of the method's arithmetic: it only draws numbers and encodes
them.  Everything is host numpy, drawn from ``numpy.random.default_rng``
(PCG64) with per-workload seeds and ``SeedSequence.spawn`` sub-streams, so the
same bytes go to the GPU path and to the oracle.

bf16 and f16 values are carried as ``numpy.uint16`` bit patterns; bf16 values
are fp32 draws rounded to nearest-even on their top 16 bits.

The workloads (shapes, value distributions, index and mask statistics):

* row gather        fp32 (1024, 256) ~ N(0,1); 4096 int32 row indices uniform
                    in [-64, 1087]; (64, 256) tiles along axis 0.
* warp example      arange(1..16) as 4x4 fp32; indices [0, 2]; (2, 4) tile.
* bounded copy      bf16 logical (8191, 4097) ~ N(0,1) stored with row stride
                    4103; (64, 32) tiles over ceil-div grids based at (0, 0)
                    and (-16, -16); destination pre-filled with a sentinel.
* masked gather / scatter
                    fp32 table (1048576, 128) ~ U(-1,1); 4194304 int32 indices
                    uniform over rows with a Bernoulli(0.9) mask, padding -1.0;
                    scatter of (1048576, 128) U(-1,1) rows to a permutation
                    of destination rows under a Bernoulli(0.5) mask.
* ragged load       bf16 (total_rows, 8, 128) ~ N(0,1); 64 sequences with
                    lengths uniform in [1, 8192].
* bounded GEMM      bf16 A (M, K) ~ N(0,1), B (K, N) ~ N(0,1)/sqrt(K);
                    (65, 97, 73) and (8191, 8193, 4097).
* block-scaled GEMM operand codes uniform over every finite code of the
                    format (e4m3, e5m2; e2m1 packed two per byte, even element
                    in the low nibble), B given K-major as (N, K); e8m0 scale
                    bytes uniform in [120, 133] (2^-7 .. 2^6), one per 32-value
                    block; (8191, 8193, 4096).
"""
from __future__ import annotations

import numpy as np

SEED_ROW_GATHER = 1001
SEED_BOUNDED_COPY = 1002
SEED_MASKED = 1003
SEED_RAGGED = 1004
SEED_GEMM = 1005
SEED_SCALED_GEMM = 1006
SEED_ZIPF = 1007

# A bf16 bit pattern that a N(0,1) draw never produces (a signalling-NaN-like
# payload); it marks padding columns and untouched destination elements.
BF16_SENTINEL = np.uint16(0x7FA5)
F32_SENTINEL_BITS = np.uint32(0x7FA5A5A5)


def _rngs(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode fp32 draws as bf16 bit patterns, rounding to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- indexed row gather -----------------------------------------------------

def warp_example():
    """The 4x4 arange(1..16) source with indices [0, 2] and a (2, 4) tile."""
    x = np.arange(1, 17, dtype=np.float32).reshape(4, 4)
    return {"a": x, "indices": np.array([0, 2], dtype=np.int32), "tile_shape": (2, 4), "offset": (0, 0), "axis": 0}


def row_gather(seed: int = SEED_ROW_GATHER, rows: int = 1024, cols: int = 256, n_indices: int = 4096,
               lo: int = -64, hi: int = 1087, tile_rows: int = 64):
    ra, ri = _rngs(seed, 2)
    a = ra.standard_normal((rows, cols), dtype=np.float32)
    idx = ri.integers(lo, hi, size=n_indices, endpoint=True, dtype=np.int64).astype(np.int32)
    return {"a": a, "indices": idx, "tile_shape": (tile_rows, cols), "offset": (0, 0), "axis": 0}


# ---- bounded 2-D tile copy --------------------------------------------------

def bounded_copy(seed: int = SEED_BOUNDED_COPY, M: int = 8191, N: int = 4097, ld: int = 4103,
                 tile=(64, 32), origins=((0, 0), (-16, -16))):
    """src / dst storage arrays (M, ld) of bf16 bits; the logical views are [:, :N]."""
    (rs,) = _rngs(seed, 1)
    vals = f32_to_bf16_bits(rs.standard_normal((M, N), dtype=np.float32))
    src = np.full((M, ld), BF16_SENTINEL, dtype=np.uint16)
    src[:, :N] = vals
    dst = np.full((M, ld), BF16_SENTINEL, dtype=np.uint16)
    return {"src": src, "dst": dst, "M": M, "N": N, "ld": ld, "tile": tuple(tile), "origins": tuple(origins)}


# ---- masked gather / scatter ------------------------------------------------

def masked(seed: int = SEED_MASKED, rows: int = 1048576, cols: int = 128, n_gather: int = 4194304,
           p_gather: float = 0.9, n_scatter: int = 1048576, p_scatter: float = 0.5,
           padding_value: float = -1.0):
    rt, ri, rm, rv, rp, rs = _rngs(seed, 6)
    table = rt.uniform(-1.0, 1.0, size=(rows, cols)).astype(np.float32)
    idx = ri.integers(0, rows, size=n_gather, dtype=np.int64).astype(np.int32)
    gmask = (rm.random(n_gather) < p_gather).astype(np.uint8)
    vals = rv.uniform(-1.0, 1.0, size=(n_scatter, cols)).astype(np.float32)
    perm = rp.permutation(rows)[:n_scatter].astype(np.int32)
    smask = (rs.random(n_scatter) < p_scatter).astype(np.uint8)
    return {"table": table, "indices": idx, "gmask": gmask, "padding_value": padding_value,
            "vals": vals, "perm": perm, "smask": smask}


def zipf_indices(seed: int = SEED_ZIPF, rows: int = 1048576, n: int = 4194304, a: float = 1.1) -> np.ndarray:
    """Skewed gather indices, int32: a Zipf law truncated to the table, row k
    drawn with probability proportional to (k + 1)^-a, k < rows (inverse CDF
    of uniform draws).  At a = 1.1 over 1,048,576 rows, row 0 takes about 12%
    of the terms and about 3,600 rows take more than 64 each."""
    (rz,) = _rngs(seed, 1)
    w = np.arange(1, rows + 1, dtype=np.float64) ** -a
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    return np.minimum(np.searchsorted(cdf, rz.random(n), side="right"), rows - 1).astype(np.int32)


# ---- ragged varlen 3-D tiles ------------------------------------------------

def ragged(seed: int = SEED_RAGGED, n_seqs: int = 64, max_len: int = 8192, heads: int = 8,
           depth: int = 128):
    rl, rx = _rngs(seed, 2)
    lens = rl.integers(1, max_len, size=n_seqs, endpoint=True, dtype=np.int64)
    total = int(lens.sum())
    X = f32_to_bf16_bits(rx.standard_normal((total, heads, depth), dtype=np.float32))
    return {"seq_lens": lens, "X": X, "heads": heads, "depth": depth}


# ---- bounded GEMM -----------------------------------------------------------

def gemm(M: int, N: int, K: int, seed: int = SEED_GEMM, scale_a: bool = False):
    """A ~ N(0,1), B ~ N(0,1)/sqrt(K) so that C ~ N(0,1); scale_a also divides A by sqrt(K)."""
    ra, rb = _rngs(seed, 2)
    a = ra.standard_normal((M, K), dtype=np.float32)
    if scale_a:
        a = a / np.float32(np.sqrt(K))
    b = rb.standard_normal((K, N), dtype=np.float32) / np.float32(np.sqrt(K))
    return {"A": f32_to_bf16_bits(a), "B": f32_to_bf16_bits(b), "M": M, "N": N, "K": K}


def lowp_codes(rng, shape, fmt: str) -> np.ndarray:
    """Uniform finite codes of an 8-bit (e4m3, e5m2) or 4-bit (e2m1) format,
    one code per uint8; NaN and infinity codes are redrawn as +1.5."""
    if fmt == "e2m1":
        return rng.integers(0, 16, shape, dtype=np.uint8)
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    if fmt == "e4m3":
        c[(c & 0x7F) == 0x7F] = 0x3C  # e4m3fn NaN
    elif fmt == "e5m2":
        c[(c & 0x7C) == 0x7C] = 0x3E  # e5m2 infinities and NaNs
    else:
        raise ValueError(fmt)
    return c


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis, the even element low."""
    return ((codes[..., 0::2] & 0xF) | ((codes[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def scaled_gemm(M: int, N: int, K: int, fmt: str = "e4m3", block: int = 32, seed: int = SEED_SCALED_GEMM):
    """Operand codes A (M, K) and Bt (N, K) (packed for e2m1) and e8m0 scale
    bytes (M, K/block), (N, K/block)."""
    ra, rb, rs, rt = _rngs(seed, 4)
    A, Bt = lowp_codes(ra, (M, K), fmt), lowp_codes(rb, (N, K), fmt)
    if fmt == "e2m1":
        A, Bt = pack_e2m1(A), pack_e2m1(Bt)
    sa = rs.integers(120, 134, (M, K // block), dtype=np.uint8)
    sb = rt.integers(120, 134, (N, K // block), dtype=np.uint8)
    return {"A": A, "Bt": Bt, "sa": sa, "sb": sb, "fmt": fmt, "block": block, "M": M, "N": N, "K": K}
