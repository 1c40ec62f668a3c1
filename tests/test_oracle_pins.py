"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code: values the pages
print (fixtures under tests/golden/, each with its citation), closed forms,
special cases that reduce to a numpy routine, and brute force on tiny inputs
written as a second formulation (zero-bordered fancy indexing and slicing
instead of the oracle's per-element loops).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

from scatter_tile_gather_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# second formulations (numpy, vectorised) used as brute force
# ---------------------------------------------------------------------------

def np_gather(a, indices, tile_shape, offset, axis, mask=None, fill=None):
    """Zero-bordered fancy-index formulation of the indexed gather."""
    a = np.asarray(a)
    n = len(indices)
    out_shape = list(tile_shape)
    out_shape[axis] = n
    grids = np.meshgrid(*[np.arange(s) for s in out_shape], indexing="ij")
    coords, ok = [], np.ones(out_shape, dtype=bool)
    for d in range(a.ndim):
        if d == axis:
            s = offset[d] + np.asarray(indices, dtype=np.int64)[grids[d]]
        else:
            s = offset[d] + grids[d]
        ok &= (s >= 0) & (s < a.shape[d])
        coords.append(s)
    if mask is not None:
        ok &= np.asarray(mask).astype(bool)[grids[axis]]
    # one zero (or fill) cell in front of every dimension; invalid -> cell 0
    padded = np.zeros([s + 1 for s in a.shape], dtype=a.dtype)
    padded[tuple(slice(1, None) for _ in a.shape)] = a
    if fill is not None:
        padded[tuple(0 for _ in a.shape)] = fill
    sel = tuple(np.where(ok, c + 1, 0) for c in coords)
    return padded[sel]


def np_copy_tiles(src, tm, tn, r0, c0):
    M, N = src.shape
    gr = max(0, math.ceil((M - r0) / tm)) if M - r0 > 0 else 0
    gc = max(0, math.ceil((N - c0) / tn)) if N - c0 > 0 else 0
    B = max(tm, tn, abs(r0), abs(c0)) + 1
    P = np.zeros((M + 2 * B + gr * tm, N + 2 * B + gc * tn), dtype=src.dtype)
    P[B:B + M, B:B + N] = src
    out = np.zeros((gr, gc, tm, tn), dtype=src.dtype)
    for g in range(gr):
        for h in range(gc):
            R, C = r0 + g * tm + B, c0 + h * tn + B
            out[g, h] = P[R:R + tm, C:C + tn]
    return out


# ---------------------------------------------------------------------------
# grid sizing (ceil-div)
# ---------------------------------------------------------------------------

def test_grid_ceil_div_and_workload_counts(orc):
    # cuTile.jl Memory, "Tile windows": host count is cld(size, step)
    for size in range(0, 70):
        for step in (1, 3, 8, 16):
            assert orc.tile_grid(size, 0, step) == -(-size // step)
    # bounded-copy workload: 8191 x 4097 with (64, 32) tiles
    assert orc.tile_grid(8191, 0, 64) == 128
    assert orc.tile_grid(4097, 0, 32) == 129
    assert orc.tile_grid(8191, -16, 64) == 129
    assert orc.tile_grid(4097, -16, 32) == 129
    assert orc.tile_grid(8191, 0, 64) * orc.tile_grid(4097, 0, 32) == 16512
    assert orc.tile_grid(8191, -16, 64) * orc.tile_grid(4097, -16, 32) == 16641
    # GEMM K loop with BK = 64: 65 steps, the last holding one K value
    assert orc.tile_grid(4097, 0, 64) == 65
    # origin at or past the end: no tiles
    assert orc.tile_grid(10, 10, 4) == 0 and orc.tile_grid(10, 12, 4) == 0
    # every element covered exactly once, no tile starts past the end
    for extent in range(1, 40):
        for origin in range(-9, extent):
            for t in (1, 2, 5, 8):
                g = orc.tile_grid(extent, origin, t)
                assert origin + g * t >= extent and origin + (g - 1) * t < extent


# ---------------------------------------------------------------------------
# rounding of the padding value
# ---------------------------------------------------------------------------

def test_round_f32_matches_correctly_rounded_cast(orc):
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(2000) * 10.0 ** rng.integers(-45, 39, 2000),
        [0.0, -0.0, 1.0, -1.0, 3.4028235677973366e38, 3.5e38, -3.5e38, 1e-46, 7e-46, 1.401298464324817e-45,
         1.1754942e-38, np.inf, -np.inf],
        # exact ties between adjacent floats
        [(1.0 + (2 * k + 1) * 2.0 ** -24) for k in range(16)],
    ])
    for v in vals:
        with np.errstate(over="ignore"):
            want = int(np.float64(v).astype(np.float32).view(np.uint32))
        assert orc.round_to_format(v, 8, 23) == want, v


def test_round_f16_matches_numpy_half(orc):
    rng = np.random.default_rng(8)
    vals = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000),
                           [65504.0, 65520.0, 65519.99, 6.0e-8, 2.9e-8, 3.0e-8, -0.0]])
    for v in vals:
        with np.errstate(over="ignore"):
            want = int(np.float64(v).astype(np.float16).view(np.uint16))
        assert orc.round_to_format(v, 5, 10) == want, v


def test_round_bf16_ties_to_even_exhaustive(orc):
    """Every pair of adjacent positive finite bf16 values: the values map to
    themselves, the midpoint goes to the even neighbour, and points just off
    the midpoint go to the nearer neighbour."""
    dec = lambda h: float(np.uint32(h << 16).view(np.float32))
    for h in range(0, 0x7F7F):
        x, y = dec(h), dec(h + 1)
        assert orc.round_to_format(x, 8, 7) == h
        m = 0.5 * (x + y)
        assert orc.round_to_format(m, 8, 7) == (h if h % 2 == 0 else h + 1)
        eps = (y - x) * 2.0 ** -10
        assert orc.round_to_format(m - eps, 8, 7) == h
        assert orc.round_to_format(m + eps, 8, 7) == h + 1
        assert orc.round_to_format(-x, 8, 7) == h | 0x8000
    assert orc.round_to_format(float("inf"), 8, 7) == 0x7F80
    assert orc.round_to_format(3.4e38, 8, 7) == 0x7F80  # past the largest finite bf16 midpoint
    assert orc.round_to_format(float("nan"), 8, 7) & 0x7FC0 == 0x7FC0


def test_padding_bits(orc):
    # -1.0 in IEEE binary32 / bf16 / binary16 / binary64
    assert orc.padding_bits(-1.0, "f32").view(np.uint32)[0] == 0xBF800000
    assert orc.padding_bits(-1.0, "bf16").view(np.uint16)[0] == 0xBF80
    assert orc.padding_bits(-1.0, "f16").view(np.uint16)[0] == 0xBC00
    assert orc.padding_bits(-1.0, "f64").view(np.float64)[0] == -1.0
    assert orc.padding_bits(-7.9, "i32").view(np.int32)[0] == -7
    assert orc.padding_bits(255.0, "u8")[0] == 255
    assert orc.padding_bits(-0.0, "f32").view(np.uint32)[0] == 0x80000000
    with pytest.raises(ValueError):
        orc.padding_bits(256.0, "u8")
    with pytest.raises(ValueError):
        orc.padding_bits(3e9, "i32")


# ---------------------------------------------------------------------------
# indexed gather
# ---------------------------------------------------------------------------

def test_gather_warp_worked_example(orc):
    g = _golden("warp_gather_even_rows.json")
    x = np.arange(1, 17, dtype=np.float32).reshape(g["source_shape"])
    out = orc.tile_gather(x, g["indices"], g["tile_shape"], (0, 0), g["axis"])
    np.testing.assert_array_equal(out, np.array(g["expected"], dtype=np.float32))
    # the same example through the shared input generator
    ex = inputs.warp_example()
    out2 = orc.tile_gather(ex["a"], ex["indices"], ex["tile_shape"], ex["offset"], ex["axis"])
    np.testing.assert_array_equal(out2, np.array(g["expected"], dtype=np.float32))


def test_gather_negative_and_past_end_read_zero(orc):
    # Warp tile_load_indexed: a negative or past-the-end source index reads zero
    x = np.arange(1, 17, dtype=np.float32).reshape(4, 4)
    out = orc.tile_gather(x, [-1, 2, 4, 3], (4, 4), (0, 0), 0)
    np.testing.assert_array_equal(out[0], 0)
    np.testing.assert_array_equal(out[1], x[2])
    np.testing.assert_array_equal(out[2], 0)
    np.testing.assert_array_equal(out[3], x[3])
    # offset on the axis is added to each index; off-axis offset shifts columns
    out = orc.tile_gather(x, [0, 1], (2, 3), (1, 2), 0)
    np.testing.assert_array_equal(out, np.array([[7, 8, 0], [11, 12, 0]], dtype=np.float32))


def test_gather_identity_indices_reproduce_source(orc):
    a = np.random.default_rng(1).standard_normal((32, 24)).astype(np.float32)
    out = orc.tile_gather(a, np.arange(32), (8, 24), (0, 0), 0)
    np.testing.assert_array_equal(out, a)
    out = orc.tile_gather(a, np.arange(24), (32, 6), (0, 0), 1)
    np.testing.assert_array_equal(out, a)


@pytest.mark.parametrize("seed", range(12))
def test_gather_bruteforce(orc, seed):
    rng = np.random.default_rng(100 + seed)
    rank = int(rng.integers(1, 5))
    shape = tuple(int(s) for s in rng.integers(1, 6, rank))
    dt = [np.float32, np.uint16, np.uint8, np.int64][seed % 4]
    a = (rng.integers(1, 200, shape)).astype(dt)
    axis = int(rng.integers(0, rank))
    tile = [int(rng.integers(1, 5)) for _ in range(rank)]
    n_tiles = int(rng.integers(1, 4))
    idx = rng.integers(-3, shape[axis] + 3, tile[axis] * n_tiles).astype(np.int32)
    offset = [int(o) for o in rng.integers(-2, 3, rank)]
    want = np_gather(a, idx, tile, offset, axis)
    got = orc.tile_gather(a, idx, tile, offset, axis)
    np.testing.assert_array_equal(got, want)


def test_gather_strided_source(orc):
    rng = np.random.default_rng(3)
    base = rng.standard_normal((10, 13)).astype(np.float32)
    view = base[:, 2:11]  # row stride 13, logical (10, 9)
    idx = rng.integers(-2, 12, 6).astype(np.int32)
    np.testing.assert_array_equal(orc.tile_gather(view, idx, (3, 9), (0, 0), 0),
                                  np_gather(view, idx, (3, 9), (0, 0), 0))


# ---------------------------------------------------------------------------
# masked gather / scatter
# ---------------------------------------------------------------------------

def test_masked_gather_special_cases(orc):
    rng = np.random.default_rng(11)
    a = rng.uniform(-1, 1, (50, 8)).astype(np.float32)
    idx = rng.integers(0, 50, 40).astype(np.int32)
    ones = np.ones(40, np.uint8)
    # mask all true with in-range indices == the plain gather
    np.testing.assert_array_equal(orc.tile_gather_masked(a, idx, ones, (8, 8), (0, 0), 0, -1.0, "f32"),
                                  orc.tile_gather(a, idx, (8, 8), (0, 0), 0))
    # mask all false: every element is the padding bit pattern
    out = orc.tile_gather_masked(a, idx, np.zeros(40, np.uint8), (8, 8), (0, 0), 0, -1.0, "f32")
    assert np.all(out.view(np.uint32) == 0xBF800000)
    # mixed: padding rows == mask zeros; mask-true rows equal the source rows
    m = (rng.random(40) < 0.6).astype(np.uint8)
    out = orc.tile_gather_masked(a, idx, m, (8, 8), (0, 0), 0, -1.0, "f32")
    pad_rows = np.all(out.view(np.uint32) == 0xBF800000, axis=1)
    assert pad_rows.sum() == (m == 0).sum()
    np.testing.assert_array_equal(out[m == 1], a[idx[m == 1]])
    # an out-of-range index under a true mask also takes the padding value
    idx2 = idx.copy()
    idx2[0] = 50
    out = orc.tile_gather_masked(a, idx2, ones, (8, 8), (0, 0), 0, -1.0, "f32")
    assert np.all(out[0].view(np.uint32) == 0xBF800000)


@pytest.mark.parametrize("seed", range(8))
def test_masked_gather_bruteforce(orc, seed):
    rng = np.random.default_rng(200 + seed)
    rank = int(rng.integers(2, 5))
    shape = tuple(int(s) for s in rng.integers(1, 6, rank))
    a = rng.standard_normal(shape).astype(np.float32)
    axis = int(rng.integers(0, rank))
    tile = [int(rng.integers(1, 5)) for _ in range(rank)]
    idx = rng.integers(-2, shape[axis] + 2, tile[axis] * 3).astype(np.int32)
    mask = (rng.random(idx.size) < 0.7).astype(np.uint8)
    offset = [int(o) for o in rng.integers(-1, 2, rank)]
    want = np_gather(a, idx, tile, offset, axis, mask=mask, fill=np.float32(2.5))
    got = orc.tile_gather_masked(a, idx, mask, tile, offset, axis, 2.5, "f32")
    np.testing.assert_array_equal(got, want)


def test_scatter_roundtrip_and_untouched_rows(orc):
    rng = np.random.default_rng(21)
    rows, cols = 64, 16
    dst0 = rng.uniform(-1, 1, (rows, cols)).astype(np.float32)
    vals = rng.uniform(-1, 1, (48, cols)).astype(np.float32)
    perm = rng.permutation(rows)[:48].astype(np.int32)
    m = (rng.random(48) < 0.5).astype(np.uint8)
    dst = dst0.copy()
    orc.tile_scatter_masked(dst, perm, m, (16, cols), vals, (0, 0), 0)
    # numpy formulation with unique destinations
    want = dst0.copy()
    want[perm[m == 1]] = vals[m == 1]
    np.testing.assert_array_equal(dst, want)
    # gather back through the same permutation returns the written rows
    back = orc.tile_gather(dst, perm, (16, cols), (0, 0), 0)
    np.testing.assert_array_equal(back[m == 1], vals[m == 1])
    # rows never written keep their bits
    untouched = np.setdiff1d(np.arange(rows), perm[m == 1])
    np.testing.assert_array_equal(dst[untouched], dst0[untouched])
    # mask all false: nothing written
    dst = dst0.copy()
    orc.tile_scatter_masked(dst, perm, np.zeros(48, np.uint8), (16, cols), vals, (0, 0), 0)
    np.testing.assert_array_equal(dst, dst0)


def test_scatter_out_of_range_is_clipped(orc):
    dst0 = np.zeros((4, 3), dtype=np.float32)
    vals = np.arange(1, 13, dtype=np.float32).reshape(4, 3)
    dst = dst0.copy()
    orc.tile_scatter_masked(dst, [-1, 0, 7, 3], np.ones(4, np.uint8), (4, 4), np.pad(vals, ((0, 0), (0, 1))),
                            (0, 0), 0)
    # tile is (4, 4) but dst has 3 columns: column 3 is clipped; rows -1 and 7 skipped
    want = dst0.copy()
    want[0] = vals[1]
    want[3] = vals[3]
    np.testing.assert_array_equal(dst, want)


@pytest.mark.parametrize("seed", range(6))
def test_scatter_bruteforce_rank3(orc, seed):
    rng = np.random.default_rng(300 + seed)
    shape = (5, 6, 4)
    axis = seed % 3
    dst0 = rng.integers(1, 1000, shape).astype(np.int32)
    tile_shape = [3, 3, 3]
    n = shape[axis]
    idx = rng.permutation(n + 2)[: n].astype(np.int32) - 1  # unique, some out of range
    tile_shape[axis] = n
    offset = [0, 1, 0]
    offset[axis] = 0
    out_shape = list(tile_shape)
    tile = rng.integers(1000, 2000, out_shape).astype(np.int32)
    mask = (rng.random(n) < 0.6).astype(np.uint8)
    dst = dst0.copy()
    orc.tile_scatter_masked(dst, idx, mask, tile_shape, tile, offset, axis)
    want = dst0.copy()
    for o in np.ndindex(*out_shape):
        if not mask[o[axis]]:
            continue
        s = [offset[d] + (idx[o[d]] if d == axis else o[d]) for d in range(3)]
        if all(0 <= s[d] < shape[d] for d in range(3)):
            want[tuple(s)] = tile[o]
    np.testing.assert_array_equal(dst, want)


# ---------------------------------------------------------------------------
# bounded copy / clipped store
# ---------------------------------------------------------------------------

def test_copy_tylo_concrete_edge(orc):
    g = _golden("tylo_concrete_edge.json")
    M, N = g["matrix_shape"]
    tm, tn = g["tile_shape"]
    r0, c0 = g["origin"]
    A = (np.arange(M * N, dtype=np.uint32) % 60000 + 1).astype(np.uint16).reshape(M, N)  # no zero bits
    tiles = orc.tile_copy_bounded(A, tm, tn, r0, c0)
    assert tiles.shape == (1, 1, tm, tn)
    t = tiles[0, 0]
    nz = np.argwhere(t != 0)
    assert len(nz) == g["valid_rows"] * g["valid_cols"] == g["tile_slots"] - g["zero_slots"]
    assert set(nz[:, 0]) == {0} and list(nz[:, 1]) == list(range(g["valid_cols"]))
    v = g["vector_elements"]
    np.testing.assert_array_equal(t[0, :v], A[64, 64:64 + v])  # vector 0: full
    assert (t[0, v:2 * v] != 0).sum() == g["vector1_valid"] and t[0, v] == A[64, 72]
    assert (t != 0).sum() == g["tile_slots"] - g["zero_slots"]
    # the first vector's source byte offset is 16-byte aligned when the base is
    assert ((r0 * N + c0) * g["element_bytes"]) % 16 == 0


@pytest.mark.parametrize("seed", range(10))
def test_copy_bruteforce(orc, seed):
    rng = np.random.default_rng(400 + seed)
    M, N = int(rng.integers(1, 40)), int(rng.integers(1, 40))
    ld = N + int(rng.integers(0, 5))
    tm, tn = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    r0, c0 = int(rng.integers(-tm - 2, 3)), int(rng.integers(-tn - 2, 3))
    store = rng.integers(1, 60000, (M, ld)).astype(np.uint16)
    src = store[:, :N]
    np.testing.assert_array_equal(orc.tile_copy_bounded(src, tm, tn, r0, c0), np_copy_tiles(src, tm, tn, r0, c0))


def test_copy_column_strided_source(orc):
    rng = np.random.default_rng(5)
    store = rng.integers(1, 60000, (20, 30)).astype(np.uint16)
    src = store[:, ::3]  # non-unit column stride
    np.testing.assert_array_equal(orc.tile_copy_bounded(src, 4, 3, -1, -2), np_copy_tiles(src, 4, 3, -1, -2))


@pytest.mark.parametrize("origin", [(0, 0), (-16, -16)])
def test_copy_workload_closed_form_counts(orc, origin):
    """Bounded-copy workload: valid slots = M*N; zero slots = tiles*2048 - M*N."""
    M, N, ld, tm, tn = 8191, 4097, 4103, 64, 32
    store = np.full((M, ld), 0x7FA5, dtype=np.uint16)
    store[:, :N] = np.random.default_rng(9).integers(1, 0x7F00, (M, N), dtype=np.uint16)
    tiles = orc.tile_copy_bounded(store[:, :N], tm, tn, *origin)
    n_tiles = tiles.shape[0] * tiles.shape[1]
    assert n_tiles == {(0, 0): 16512, (-16, -16): 16641}[origin]
    zeros = int((tiles == 0).sum())
    assert zeros == n_tiles * tm * tn - M * N == {(0, 0): 258049, (-16, -16): 522241}[origin]
    assert not np.any(tiles == 0x7FA5)  # ld padding never read into a tile


@pytest.mark.parametrize("seed", range(8))
def test_store_inverts_copy_and_leaves_padding(orc, seed):
    rng = np.random.default_rng(500 + seed)
    M, N = int(rng.integers(1, 50)), int(rng.integers(1, 50))
    ld = N + int(rng.integers(0, 6))
    tm, tn = int(rng.integers(1, 10)), int(rng.integers(1, 10))
    r0, c0 = int(rng.integers(-tm - 1, 2)), int(rng.integers(-tn - 1, 2))
    src = rng.integers(1, 60000, (M, ld)).astype(np.uint16)
    tiles = orc.tile_copy_bounded(src[:, :N], tm, tn, r0, c0)
    dst = np.full((M, ld), 0x7FA5, dtype=np.uint16)
    orc.tile_store_clipped(tiles, r0, c0, dst[:, :N])
    # rows/cols the grid covers are restored; nothing else is written
    rr, cc = max(0, r0), max(0, c0)
    want = np.full((M, ld), 0x7FA5, dtype=np.uint16)
    want[rr:, cc:N] = src[rr:, cc:N]
    np.testing.assert_array_equal(dst, want)
    # a tile buffer of a different source stores exactly its valid slots
    other = rng.integers(1, 60000, tiles.shape).astype(np.uint16)
    dst2 = np.full((M, ld), 0x7FA5, dtype=np.uint16)
    orc.tile_store_clipped(other, r0, c0, dst2[:, :N])
    canvas = other.transpose(0, 2, 1, 3).reshape(tiles.shape[0] * tm, tiles.shape[1] * tn)
    want2 = np.full((M, ld), 0x7FA5, dtype=np.uint16)
    want2[rr:M, cc:N] = canvas[rr - r0:M - r0, cc - c0:N - c0]
    np.testing.assert_array_equal(dst2, want2)


# ---------------------------------------------------------------------------
# ragged varlen 3-D tiles
# ---------------------------------------------------------------------------

def np_ragged(X, middle_dim, group, BM, BN, col0, ri, dyn, mi):
    bm_seq = BM // group
    out = np.zeros((len(ri), BM, BN), dtype=X.dtype)
    for k in range(len(ri)):
        block = X[ri[k]:ri[k] + dyn[k], mi[k] * group:(mi[k] + 1) * group, col0:col0 + BN]
        pad = np.zeros((bm_seq, group, BN), dtype=X.dtype)
        pad[:block.shape[0], :block.shape[1], :block.shape[2]] = block
        out[k] = pad.reshape(BM, BN)
    return out


def test_ragged_schedule_closed_forms(orc):
    lens = np.array([5, 1, 8, 13, 16], dtype=np.int64)
    ri, dyn, mi = orc.ragged_schedule(lens, 4, 3)
    assert len(ri) == sum(-(-L // 4) for L in lens) * 3
    # lexicographic (sequence, block, head)
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = 0
    for s, L in enumerate(lens):
        for u in range(-(-L // 4)):
            for m in range(3):
                assert (ri[k], dyn[k], mi[k]) == (cu[s] + 4 * u, min(4, L - 4 * u), m)
                k += 1
    # every row of every sequence is covered exactly once per head
    cover = np.zeros(int(lens.sum()), dtype=int)
    for r, d, m in zip(ri, dyn, mi):
        if m == 0:
            cover[r:r + d] += 1
    assert np.all(cover == 1)


@pytest.mark.parametrize("group", [1, 4])
def test_ragged_multiple_of_bm_is_reshape(orc, group):
    rng = np.random.default_rng(31)
    bm, heads, depth = 8, 8, 16
    bm_seq = bm // group
    lens = np.array([bm_seq * 3, bm_seq, bm_seq * 2], dtype=np.int64)
    X = rng.integers(1, 60000, (int(lens.sum()), heads, depth)).astype(np.uint16)
    md = heads // group
    ri, dyn, mi = orc.ragged_schedule(lens, bm_seq, md)
    out = orc.ragged_tile_load(X, md, group, bm, depth, 0, ri, dyn, mi)
    # (blocks, bm_seq, md, group, depth) -> (blocks, md, bm_seq, group, depth)
    want = X.reshape(-1, bm_seq, md, group, depth).transpose(0, 2, 1, 3, 4).reshape(-1, bm, depth)
    np.testing.assert_array_equal(out, want)
    assert not np.any(out == 0)


@pytest.mark.parametrize("group", [1, 2, 4])
def test_ragged_zero_rows_and_bruteforce(orc, group):
    rng = np.random.default_rng(40 + group)
    heads, depth, BM = 8, 24, 16
    bm_seq, md = BM // group, heads // group
    lens = rng.integers(1, 40, 7).astype(np.int64)
    X = rng.integers(1, 60000, (int(lens.sum()), heads, depth)).astype(np.uint16)
    ri, dyn, mi = orc.ragged_schedule(lens, bm_seq, md)
    for BN, col0 in [(depth, 0), (16, 0), (16, 16)]:
        out = orc.ragged_tile_load(X, md, group, BM, BN, col0, ri, dyn, mi)
        np.testing.assert_array_equal(out, np_ragged(X, md, group, BM, BN, col0, ri, dyn, mi))
    out = orc.ragged_tile_load(X, md, group, BM, depth, 0, ri, dyn, mi)
    zero_rows = int(np.all(out == 0, axis=2).sum())
    assert zero_rows == md * group * int(sum(-(-L // bm_seq) * bm_seq - L for L in lens))


def test_ragged_rows_past_total_are_zero(orc):
    X = np.arange(1, 1 + 3 * 2 * 4, dtype=np.uint16).reshape(3, 2, 4)
    out = orc.ragged_tile_load(X, 2, 1, 4, 4, 0, [1], [4], [1])
    np.testing.assert_array_equal(out[0, :2], X[1:3, 1])
    np.testing.assert_array_equal(out[0, 2:], 0)
    # a head index past middle_dim selects nothing: the tile is all zero
    out = orc.ragged_tile_load(X, 2, 1, 4, 4, 0, [0], [3], [2])
    np.testing.assert_array_equal(out, 0)
    np.testing.assert_array_equal(np_ragged(X, 2, 1, 4, 4, 0, [0], [3], [2]), 0)


@pytest.mark.parametrize("group", [1, 4])
def test_ragged_store_multiple_of_bm_is_inverse_reshape(orc, group):
    """Every sequence a multiple of BM_seq: the tiles of the schedule, stored,
    are X rearranged from (blocks, head block, position, group, depth) back to
    (rows, heads, depth) -- the inverse of the load's reshape."""
    rng = np.random.default_rng(61)
    bm, heads, depth = 8, 8, 16
    bm_seq, md = bm // group, heads // group
    lens = np.array([bm_seq * 2, bm_seq, bm_seq * 3], dtype=np.int64)
    rows = int(lens.sum())
    tiles = rng.integers(1, 60000, (rows // bm_seq * md, bm, depth)).astype(np.uint16)
    ri, dyn, mi = orc.ragged_schedule(lens, bm_seq, md)
    got = orc.ragged_tile_store(tiles, np.zeros((rows, heads, depth), np.uint16), md, group, 0, ri, dyn, mi)
    want = tiles.reshape(-1, md, bm_seq, group, depth).transpose(0, 2, 1, 3, 4).reshape(rows, heads, depth)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("group", [1, 2, 4])
def test_ragged_store_load_round_trips(orc, group):
    """Over a schedule that covers every row once: store(load(X)) rebuilds X
    from a sentinel-filled array, and load(store(T)) keeps exactly the tile
    elements that have a place in X (rows below dynamic_dim, columns inside
    depth) and reads zero for the others."""
    rng = np.random.default_rng(70 + group)
    heads, depth, BM = 8, 24, 16
    bm_seq, md = BM // group, heads // group
    lens = rng.integers(1, 40, 7).astype(np.int64)
    rows = int(lens.sum())
    X = rng.integers(1, 60000, (rows, heads, depth)).astype(np.uint16)
    ri, dyn, mi = orc.ragged_schedule(lens, bm_seq, md)
    sentinel = np.full_like(X, 0xFFFF)
    tiles = orc.ragged_tile_load(X, md, group, BM, depth, 0, ri, dyn, mi)
    np.testing.assert_array_equal(orc.ragged_tile_store(tiles, sentinel, md, group, 0, ri, dyn, mi), X)
    # two column windows, the second overhanging depth by 8 columns
    parts = sentinel
    for col0 in (0, 16):
        t = orc.ragged_tile_load(X, md, group, BM, 16, col0, ri, dyn, mi)
        parts = orc.ragged_tile_store(t, parts, md, group, col0, ri, dyn, mi)
    np.testing.assert_array_equal(parts, X)
    T = rng.integers(1, 60000, (len(ri), BM, 16)).astype(np.uint16)
    back = orc.ragged_tile_load(orc.ragged_tile_store(T, sentinel, md, group, 16, ri, dyn, mi), md, group, BM, 16, 16,
                                ri, dyn, mi)
    s_of_row = np.arange(BM) // group
    keep = (s_of_row[None, :, None] < dyn[:, None, None].astype(np.int64)) & (np.arange(16)[None, None, :] < 8)
    np.testing.assert_array_equal(back, np.where(keep, T, 0))


def test_ragged_store_writes_nothing_outside(orc):
    """Hand-worked case: X (5 rows, 2 heads, 4 columns), one tile of BM 4 at
    ragged_idx 1 with dynamic_dim 2 for head 1 writes X[1:3, 1, :] only; rows
    past total_rows, a head index past middle_dim and columns past depth are
    never written."""
    X = np.arange(40, dtype=np.int32).reshape(5, 2, 4)
    t = -np.arange(1, 17, dtype=np.int32).reshape(1, 4, 4)
    got = orc.ragged_tile_store(t, X, 2, 1, 0, [1], [2], [1])
    want = X.copy()
    want[1, 1] = [-1, -2, -3, -4]
    want[2, 1] = [-5, -6, -7, -8]
    np.testing.assert_array_equal(got, want)
    # dynamic_dim 4 at ragged_idx 3: rows 3, 4 exist, rows 5, 6 do not
    got = orc.ragged_tile_store(t, X, 2, 1, 0, [3], [4], [0])
    want = X.copy()
    want[3, 0] = [-1, -2, -3, -4]
    want[4, 0] = [-5, -6, -7, -8]
    np.testing.assert_array_equal(got, want)
    # head 2 of middle_dim 2: nothing; col0 2 with BN 4: only columns 2, 3
    np.testing.assert_array_equal(orc.ragged_tile_store(t, X, 2, 1, 0, [0], [4], [2]), X)
    got = orc.ragged_tile_store(t, X, 2, 1, 2, [0], [1], [0])
    want = X.copy()
    want[0, 0, 2:] = [-1, -2]
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------------------
# backward of the indexed gather (adjoint accumulated into a.grad)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", [
    ((40, 24), (8, 24), (0, 0), 0, 64),     # rows, full width
    ((40, 24), (8, 16), (0, 5), 0, 48),     # column window partly past the edge
    ((30, 50), (12, 7), (-3, 0), 1, 35),    # gather along the last axis, negative row offset
    ((6, 20, 9), (4, 5, 9), (1, 0, 0), 1, 40),  # rank 3, middle axis
    ((5, 7, 4, 6), (2, 3, 4, 6), (0, 2, 0, 0), 2, 12),  # rank 4
])
def test_gather_backward_is_the_adjoint_of_the_gather(orc, case):
    """<gather(a), g> = <a, backward(g)> for every a and g: the backward is the
    transpose of the gather's linear map (indices out of range included)."""
    shape, tile, off, axis, n_idx = case
    rng = np.random.default_rng(sum(shape) + n_idx)
    idx = rng.integers(-4, shape[axis] + 4, n_idx).astype(np.int32)
    a = rng.standard_normal(shape)
    g_shape = list(tile)
    g_shape[axis] = n_idx
    g = rng.standard_normal(g_shape)
    fwd = orc.tile_gather(a, idx, tile, off, axis)
    back, _, _ = orc.tile_gather_backward(np.zeros(shape), idx, tile, g, off, axis)
    lhs = float(np.sum(fwd * g))
    rhs = float(np.sum(a * back))
    assert abs(lhs - rhs) <= 1e-11 * (np.sum(np.abs(fwd * g)) + 1.0)


def test_gather_backward_with_unique_indices_is_a_scatter(orc):
    rng = np.random.default_rng(404)
    idx = rng.permutation(64)[:48].astype(np.int32)
    g = rng.standard_normal((48, 16)).astype(np.float32)
    back, _, count = orc.tile_gather_backward(np.zeros((64, 16), np.float32), idx, (16, 16), g)
    want = np.zeros((64, 16), np.float32)
    orc.tile_scatter_masked(want, idx, np.ones(48, np.uint8), (16, 16), g)
    np.testing.assert_array_equal(back, want.astype(np.float64))
    assert set(np.unique(count)) <= {0, 1}


def test_gather_backward_counts_repeated_indices(orc):
    """With a gradient of ones every element of a.grad receives one term per
    occurrence of its row among the in-range indices (bincount)."""
    rng = np.random.default_rng(405)
    idx = rng.integers(-10, 40, 200).astype(np.int32)
    a0 = rng.standard_normal((32, 8))
    back, abs_sum, count = orc.tile_gather_backward(a0, idx, (20, 8), np.ones((200, 8)))
    occ = np.bincount(idx[(idx >= 0) & (idx < 32)], minlength=32)
    np.testing.assert_array_equal(count, np.repeat(occ[:, None], 8, axis=1))
    np.testing.assert_allclose(back, a0 + count, rtol=0, atol=1e-12)  # accumulates onto a.grad's values
    np.testing.assert_allclose(abs_sum, np.abs(a0) + count, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# tile windows with a step (eachtile with step != shape)
# ---------------------------------------------------------------------------

def np_windows(X, tm, tn, sr, sc, r0, c0):
    """Windows as slices of a zero-padded copy of X (numpy slicing only)."""
    M, N = X.shape
    gr = -(-(M - r0) // sr) if M > r0 else 0
    gc = -(-(N - c0) // sc) if N > c0 else 0
    pad_r = max(tm + sr, abs(r0)) + 1
    pad_c = max(tn + sc, abs(c0)) + 1
    P = np.zeros((M + 2 * pad_r + gr * sr, N + 2 * pad_c + gc * sc), dtype=X.dtype)
    P[pad_r:pad_r + M, pad_c:pad_c + N] = X
    out = np.zeros((gr, gc, tm, tn), dtype=X.dtype)
    for a in range(gr):
        for b in range(gc):
            R, C = r0 + a * sr + pad_r, c0 + b * sc + pad_c
            out[a, b] = P[R:R + tm, C:C + tn]
    return out


def test_windows_with_step_equal_to_shape_are_the_bounded_copy(orc):
    rng = np.random.default_rng(81)
    X = rng.integers(1, 1000, (37, 29)).astype(np.int32)
    for (tm, tn, r0, c0) in [(8, 8, 0, 0), (5, 7, -3, -2), (16, 4, 2, 5)]:
        np.testing.assert_array_equal(orc.tile_copy_windows(X, tm, tn, tm, tn, r0, c0),
                                      orc.tile_copy_bounded(X, tm, tn, r0, c0))
        t = orc.tile_copy_bounded(X, tm, tn, r0, c0)
        a = np.full_like(X, -1)
        b = np.full_like(X, -1)
        orc.tile_store_windows(t, tm, tn, r0, c0, a)
        orc.tile_store_clipped(t, r0, c0, b)
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("case", [(8, 8, 4, 8, 0, 0), (8, 8, 16, 8, 0, 0), (6, 5, 3, 7, -4, 2), (4, 9, 5, 2, 3, -6),
                                  (1, 1, 3, 3, 0, 0), (7, 7, 1, 1, -2, -2)])
def test_windows_copy_matches_padded_slices(orc, case):
    tm, tn, sr, sc, r0, c0 = case
    rng = np.random.default_rng(sum(case) + 90)
    X = rng.integers(1, 60000, (23, 19)).astype(np.uint16)
    got = orc.tile_copy_windows(X, tm, tn, sr, sc, r0, c0)
    np.testing.assert_array_equal(got, np_windows(X, tm, tn, sr, sc, r0, c0))
    # the page's window count: cld(extent, step) from a zero origin
    if r0 == 0 and c0 == 0:
        assert got.shape[:2] == (-(-23 // sr), -(-19 // sc))


@pytest.mark.parametrize("case", [(8, 8, 16, 8, 0, 0), (4, 3, 4, 5, -1, -2), (5, 5, 7, 6, 2, 1)])
def test_windows_store_without_overlap_is_slice_assignment(orc, case):
    tm, tn, sr, sc, r0, c0 = case
    assert sr >= tm and sc >= tn
    rng = np.random.default_rng(sum(case) + 120)
    dst = rng.integers(1, 1000, (21, 17)).astype(np.int32)
    M, N = dst.shape
    gr, gc = orc.tile_grid(M, r0, sr), orc.tile_grid(N, c0, sc)
    tiles = rng.integers(-1000, -1, (gr, gc, tm, tn)).astype(np.int32)
    want = dst.copy()
    for a in range(gr):
        for b in range(gc):
            R, C = r0 + a * sr, c0 + b * sc
            rs, cs = max(R, 0), max(C, 0)
            re, ce = min(R + tm, M), min(C + tn, N)
            if re > rs and ce > cs:
                want[rs:re, cs:ce] = tiles[a, b, rs - R:re - R, cs - C:ce - C]
    got = dst.copy()
    orc.tile_store_windows(tiles, sr, sc, r0, c0, got)
    np.testing.assert_array_equal(got, want)


def test_windows_overlapping_store_of_consistent_tiles_rebuilds_the_covered_region(orc):
    X = np.arange(1, 1 + 30 * 26, dtype=np.int32).reshape(30, 26)
    for (tm, tn, sr, sc, r0, c0) in [(8, 8, 4, 8, 0, 0), (6, 5, 3, 2, -2, -1), (5, 5, 8, 3, 1, 0)]:
        t = orc.tile_copy_windows(X, tm, tn, sr, sc, r0, c0)
        got = np.full_like(X, -1)
        orc.tile_store_windows(t, sr, sc, r0, c0, got)
        covered = np.zeros(X.shape, bool)
        for a in range(t.shape[0]):
            for b in range(t.shape[1]):
                R, C = r0 + a * sr, c0 + b * sc
                covered[max(R, 0):max(R + tm, 0), max(C, 0):max(C + tn, 0)] = True
        np.testing.assert_array_equal(got, np.where(covered, X, -1))


# ---------------------------------------------------------------------------
# block-scaled GEMM: low-precision formats and the scaled product
# ---------------------------------------------------------------------------

def test_e2m1_decodes_to_its_value_set(orc):
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    np.testing.assert_array_equal(orc.decode_lowp(np.arange(16), "e2m1"), mags + [-m for m in mags])


def test_e5m2_is_the_top_byte_of_an_ieee_half(orc):
    codes = np.arange(256, dtype=np.uint16)
    want = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(orc.decode_lowp(codes.astype(np.uint8), "e5m2"), want)


def test_e4m3fn_structure(orc):
    v = orc.decode_lowp(np.arange(256, dtype=np.uint8), "e4m3")
    pos = v[:128]
    assert np.isnan(pos[0x7F]) and np.isnan(v[0xFF]) and not np.isinf(v).any()
    fin = pos[:0x7F]
    assert np.all(np.diff(fin) > 0) and fin[0] == 0 and fin.size == 127  # monotone, 127 non-negative finite values
    assert fin[-1] == 448 and pos[0x38] == 1.0 and pos[0x08] == 2.0 ** -6 and pos[0x01] == 2.0 ** -9
    np.testing.assert_array_equal(v[128:255], -fin)  # the sign bit mirrors
    # at most 4 significant bits: every value is an integer multiple of its
    # leading power of two divided by 8, and subnormals are multiples of 2^-9
    for x in fin[1:]:
        e = np.floor(np.log2(x))
        q = x / 2.0 ** max(e - 3, -9)
        assert q == int(q)


def test_e8m0_is_a_power_of_two(orc):
    codes = np.arange(255, dtype=np.uint8)
    np.testing.assert_array_equal(orc.decode_scale(codes, "e8m0"), np.ldexp(1.0, codes.astype(int) - 127))
    assert np.isnan(orc.decode_scale([255], "e8m0")[0])
    np.testing.assert_array_equal(orc.decode_scale([0x38, 0x7E], "e4m3"), [1.0, 448.0])


def _pack_e2m1(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] & 0xF) | ((codes[..., 1::2] & 0xF) << 4)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e2m1", "e2m1")])
def test_scaled_gemm_with_unit_scales_is_the_plain_product(orc, fa, fb):
    rng = np.random.default_rng(500)
    M, N, K, block = 9, 7, 96, 32

    def codes(shape, fmt):
        c = rng.integers(0, 256 if fmt != "e2m1" else 16, shape).astype(np.uint8)
        if fmt == "e4m3":
            c[(c & 0x7F) == 0x7F] = 0x38  # no NaN
        if fmt == "e5m2":
            c[(c & 0x7C) == 0x7C] = 0x3C  # no infinity or NaN
        return c

    ca, cb = codes((M, K), fa), codes((N, K), fb)
    A = _pack_e2m1(ca) if fa == "e2m1" else ca
    Bt = _pack_e2m1(cb) if fb == "e2m1" else cb
    one = lambda r: np.full((r, K // block), 127, np.uint8)
    got = orc.gemm_scaled_f64(A, fa, one(M), Bt, fb, one(N), K, block)
    want = orc.decode_lowp(ca, fa) @ orc.decode_lowp(cb, fb).T
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)


def test_scaled_gemm_scale_blocks_act_linearly(orc):
    """Raising one a_scale element from 2^e to 2^(e+3) adds 7 times that
    block's contribution to its row, and changes nothing else."""
    rng = np.random.default_rng(501)
    M, N, K, block = 4, 5, 128, 64
    ca = rng.integers(0, 0x70, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 0x70, (N, K)).astype(np.uint8)
    sa = rng.integers(120, 134, (M, K // block)).astype(np.uint8)
    sb = rng.integers(120, 134, (N, K // block)).astype(np.uint8)
    base = orc.gemm_scaled_f64(ca, "e4m3", sa, cb, "e4m3", sb, K, block)
    sa2 = sa.copy()
    sa2[2, 1] += 3
    bumped = orc.gemm_scaled_f64(ca, "e4m3", sa2, cb, "e4m3", sb, K, block)
    a = orc.decode_lowp(ca, "e4m3") * np.repeat(orc.decode_scale(sa, "e8m0"), block, axis=1)
    b = orc.decode_lowp(cb, "e4m3") * np.repeat(orc.decode_scale(sb, "e8m0"), block, axis=1)
    contrib = a[2, 64:] @ b[:, 64:].T
    want = base.copy()
    want[2] += 7 * contrib
    np.testing.assert_allclose(bumped, want, rtol=1e-13, atol=1e-300)


def test_scaled_gemm_fp4_nibble_order_and_accumulator(orc):
    """Hand-worked: byte 0x21 holds the e2m1 values (0.5, 1.0) -- the even
    element in the low nibble -- and 0x11 holds (0.5, 0.5); with block 2,
    scales 2^1 and 2^-1 and acc 0.25: 0.25 + 2 * (0.5*0.5 + 1.0*0.5) / 2."""
    got = orc.gemm_scaled_f64(np.array([[0x21]]), "e2m1", np.array([[128]]), np.array([[0x11]]), "e2m1",
                              np.array([[126]]), 2, 2, acc=np.array([[0.25]], np.float32))
    assert got[0, 0] == 0.25 + 0.75


# ---------------------------------------------------------------------------
# bounded GEMM reference
# ---------------------------------------------------------------------------

def test_gemm_matches_numpy_f64_matmul(orc):
    g = inputs.gemm(65, 97, 73)
    A, B = g["A"], g["B"]
    C = orc.gemm_f64(A, B)
    Af = inputs.bf16_bits_to_f32(A).astype(np.float64)
    Bf = inputs.bf16_bits_to_f32(B).astype(np.float64)
    np.testing.assert_allclose(C, Af @ Bf, rtol=1e-12, atol=1e-12)
    # sampled form agrees with the full form
    rows = np.array([0, 64, 13, 64]); cols = np.array([0, 96, 50, 0])
    np.testing.assert_array_equal(orc.gemm_sample_f64(A, B, rows, cols), C[rows, cols])


def test_gemm_row_selection_is_exact(orc):
    rng = np.random.default_rng(51)
    M, N, K = 65, 97, 73
    B = inputs.f32_to_bf16_bits(rng.standard_normal((K, N)).astype(np.float32))
    sel = rng.integers(0, K, M)
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), sel] = 0x3F80  # bf16 1.0
    C = orc.gemm_f64(A, B)
    np.testing.assert_array_equal(C, inputs.bf16_bits_to_f32(B[sel]).astype(np.float64))
    np.testing.assert_array_equal(orc.f64_to_bf16_bits(C), B[sel])


def test_gemm_strided_operands(orc):
    g = inputs.gemm(9, 7, 5)
    As = np.zeros((9, 8), np.uint16); As[:, :5] = g["A"]
    Bs = np.zeros((5, 11), np.uint16); Bs[:, :7] = g["B"]
    np.testing.assert_array_equal(orc.gemm_f64(As[:, :5], Bs[:, :7]), orc.gemm_f64(g["A"], g["B"]))
    Af = inputs.bf16_bits_to_f32(g["A"]).astype(np.float64)
    Bf = inputs.bf16_bits_to_f32(g["B"]).astype(np.float64)
    np.testing.assert_allclose(orc.gemm_f64(g["A"], g["B"]), Af @ Bf, rtol=1e-13, atol=1e-13)


def test_bf16_decode(orc):
    for h, v in [(0x3F80, 1.0), (0xBF80, -1.0), (0x0000, 0.0), (0x4049, 3.140625), (0x0001, 2.0 ** -133)]:
        assert orc.bf16_to_f64(h) == v
