"""GPU parity of tile_copy_bounded / tile_store_clipped against the CPU
oracle: bit-exact, with sentinel-filled buffers proving that every tile slot
is written and that nothing outside the logical extent is."""
import json
import os

import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import random_bits, say, to_dev, to_host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SENT = 0x7FA5


def test_tylo_concrete_edge(stg, orc):
    g = json.load(open(os.path.join(GOLDEN, "tylo_concrete_edge.json")))
    M, N = g["matrix_shape"]
    A = (np.arange(M * N, dtype=np.uint32) % 60000 + 1).astype(np.uint16).reshape(M, N)
    say("tylo concrete edge (65,73) tile (64,32) at (64,64)")
    tiles = stg.tile_copy_bounded(to_dev(A), 64, 32, 64, 64)
    torch.cuda.synchronize()
    t = to_host(tiles)
    np.testing.assert_array_equal(t, orc.tile_copy_bounded(A, 64, 32, 64, 64))
    assert (t != 0).sum() == g["valid_rows"] * g["valid_cols"]


def _copy_store_case(stg, orc, store, N, tm, tn, r0, c0, dev_store=None):
    M = store.shape[0]
    src_h = store[:, :N]
    dev = to_dev(store) if dev_store is None else dev_store
    src_d = dev[:, :N]
    gr, gc = orc.tile_grid(M, r0, tm), orc.tile_grid(N, c0, tn)
    # pre-fill the tile buffer with a sentinel: every slot must be overwritten
    tiles = torch.full((gr, gc, tm, tn), 0, dtype=src_d.dtype, device="cuda:0")
    tiles.view(torch.uint8).fill_(0xA5)
    stg.tile_copy_bounded(src_d, tm, tn, r0, c0, out=tiles)
    torch.cuda.synchronize()
    want = orc.tile_copy_bounded(src_h, tm, tn, r0, c0)
    np.testing.assert_array_equal(to_host(tiles), want)
    # clipped store into a sentinel-filled destination of the same layout
    dst_h = np.full_like(store, 0)
    dst_h.view(np.uint8)[...] = 0xA5
    dst = to_dev(dst_h)
    stg.tile_store_clipped(tiles, r0, c0, dst[:, :N])
    torch.cuda.synchronize()
    want_dst = dst_h.copy()
    orc.tile_store_clipped(want, r0, c0, want_dst[:, :N])
    np.testing.assert_array_equal(to_host(dst), want_dst)


@pytest.mark.parametrize("seed", range(40))
def test_copy_store_random(stg, orc, seed):
    rng = np.random.default_rng(3000 + seed)
    dt = [np.uint16, np.float32, np.uint8, np.float64][seed % 4]
    M, N = int(rng.integers(1, 70)), int(rng.integers(1, 90))
    ld = N + int(rng.integers(0, 9))
    es = np.dtype(dt).itemsize
    # tile widths: whole 16-byte vectors (vector path) and odd widths (element path)
    tn = int(rng.choice([16 // es, 32 // es, 64 // es, 3, 5, 7])) if seed % 5 else int(rng.integers(1, 12))
    tn = max(tn, 1)
    tm = int(rng.integers(1, 40))
    r0 = int(rng.integers(-tm - 3, 4))
    c0 = int(rng.integers(-tn - 3, 4))
    store = random_bits(rng, (M, ld), dt)
    say("copy/store random", seed, dt.__name__, (M, N, ld), "tile", (tm, tn), "origin", (r0, c0))
    _copy_store_case(stg, orc, store, N, tm, tn, r0, c0)


@pytest.mark.parametrize("col_shift", range(8))
def test_copy_every_column_alignment(stg, orc, col_shift):
    """Row starts at every 2-byte phase mod 16, partial right-edge vectors."""
    rng = np.random.default_rng(40 + col_shift)
    M, N, ld = 37, 61 + col_shift, 67 + col_shift
    store = random_bits(rng, (M, ld), np.uint16)
    for (r0, c0) in [(0, 0), (-16, -16), (-3, -5), (2, 7)]:
        say("copy alignment", col_shift, "origin", (r0, c0))
        _copy_store_case(stg, orc, store, N, 16, 32, r0, c0)


def test_copy_degenerate_grids(stg, orc):
    rng = np.random.default_rng(3)
    store = random_bits(rng, (5, 9), np.uint16)
    # a tile much larger than the matrix, origin far negative: mostly zeros
    say("copy degenerate: tile larger than matrix")
    _copy_store_case(stg, orc, store, 9, 64, 32, -40, -20)
    # 1x1 tiles
    say("copy degenerate: 1x1 tiles")
    _copy_store_case(stg, orc, store, 9, 1, 1, 0, 0)
    # origin past the end: empty grid, nothing written
    say("copy degenerate: empty grid")
    tiles = stg.tile_copy_bounded(to_dev(store), 4, 8, 5, 0)
    torch.cuda.synchronize()
    assert tiles.numel() == 0


def test_copy_column_strided_source(stg, orc):
    rng = np.random.default_rng(4)
    a = random_bits(rng, (30, 40), np.float32)
    say("copy with column stride 3 (element path)")
    tiles = stg.tile_copy_bounded(to_dev(a)[:, ::3], 8, 4, -2, -1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(tiles), orc.tile_copy_bounded(a[:, ::3], 8, 4, -2, -1))


@pytest.mark.parametrize("origin", [(0, 0), (-16, -16)])
def test_bounded_copy_workload_full(stg, orc, origin):
    w = inputs.bounded_copy()
    M, N = w["M"], w["N"]
    tm, tn = w["tile"]
    say("bounded copy workload (8191,4097) ld 4103 bf16, tiles (64,32), origin", origin)
    _copy_store_case(stg, orc, w["src"], N, tm, tn, *origin)


# ---- tile windows with a step, unchecked full-tile path ----------------------

def _windows_case(stg, orc, store, N, tm, tn, sr, sc, r0, c0, check=True):
    """Copy the windows, then store them back into a sentinel-filled copy of
    the layout; overlapping windows carry equal values (they were copied from
    the same source), so the overlapped stores agree."""
    M = store.shape[0]
    src_h = store[:, :N]
    src_d = to_dev(store)[:, :N]
    gr, gc = orc.tile_grid(M, r0, sr), orc.tile_grid(N, c0, sc)
    tiles = torch.zeros((gr, gc, tm, tn), dtype=src_d.dtype, device="cuda:0")
    tiles.view(torch.uint8).fill_(0xA5)
    stg.tile_copy_windows(src_d, tm, tn, sr, sc, r0, c0, check_bounds=check, out=tiles)
    torch.cuda.synchronize()
    want = orc.tile_copy_windows(src_h, tm, tn, sr, sc, r0, c0)
    np.testing.assert_array_equal(to_host(tiles), want)
    dst_h = np.full_like(store, 0)
    dst_h.view(np.uint8)[...] = 0xA5
    dst = to_dev(dst_h)
    stg.tile_store_windows(tiles, sr, sc, r0, c0, dst[:, :N], check_bounds=check)
    torch.cuda.synchronize()
    want_dst = dst_h.copy()
    orc.tile_store_windows(want, sr, sc, r0, c0, want_dst[:, :N])
    np.testing.assert_array_equal(to_host(dst), want_dst)


@pytest.mark.parametrize("seed", range(32))
def test_windows_random(stg, orc, seed):
    rng = np.random.default_rng(7000 + seed)
    dt = [np.uint16, np.float32, np.uint8, np.float64][seed % 4]
    M, N = int(rng.integers(1, 70)), int(rng.integers(1, 90))
    ld = N + int(rng.integers(0, 9))
    es = np.dtype(dt).itemsize
    tn = int(rng.choice([16 // es, 32 // es, 64 // es, 3, 5])) if seed % 3 else int(rng.integers(1, 12))
    tn = max(tn, 1)
    tm = int(rng.integers(1, 24))
    sr = int(rng.integers(1, 2 * tm + 3))  # overlapping, adjacent or gapped row windows
    sc = int(rng.integers(1, 2 * tn + 3))
    r0 = int(rng.integers(-tm - 3, 4))
    c0 = int(rng.integers(-tn - 3, 4))
    store = random_bits(rng, (M, ld), dt)
    say("windows random", seed, dt.__name__, (M, N, ld), "tile", (tm, tn), "step", (sr, sc), "origin", (r0, c0))
    _windows_case(stg, orc, store, N, tm, tn, sr, sc, r0, c0)


@pytest.mark.parametrize("case", [(16, 32, 16, 32, 0, 0), (8, 16, 12, 16, 0, 8), (4, 8, 4, 40, 3, 0),
                                  (1, 8, 3, 8, 0, 0)])
@pytest.mark.parametrize("check", [False, True])
def test_windows_inside_unchecked(stg, orc, case, check):
    """Grids whose windows all lie inside the array: the unchecked instance,
    requested (check_bounds = 0) or chosen by the host."""
    tm, tn, sr, sc, r0, c0 = case
    rng = np.random.default_rng(sum(case))
    G_r, G_c = 5, 6
    M, N = r0 + (G_r - 1) * sr + tm, c0 + (G_c - 1) * sc + tn
    M, N = max(M, r0 + (G_r - 1) * sr + 1), max(N, c0 + (G_c - 1) * sc + 1)
    store = random_bits(rng, (M, N + 5), np.uint16)
    say("windows inside", case, "check_bounds", check, "matrix", (M, N))
    _windows_case(stg, orc, store, N, tm, tn, sr, sc, r0, c0, check=check)


def test_full_tile_workload_unchecked(stg, orc):
    """(8192, 4096) bf16 with unit-aligned row stride and (64, 32) tiles from
    (0, 0): every tile is full, so tile_copy_bounded takes the unchecked
    instance by itself; the result is the bounded copy's."""
    rng = np.random.default_rng(4242)
    src = random_bits(rng, (8192, 4096), np.uint16)
    say("full-tile workload (8192,4096) bf16 tiles (64,32), automatic unchecked dispatch")
    _copy_store_case(stg, orc, src, 4096, 64, 32, 0, 0)
