"""GPU parity of tile_gather / tile_gather_masked / tile_scatter_masked
against the CPU oracle: bit-exact, element by element."""
import json
import os

import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import random_bits, say, to_dev, to_host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

DTYPES = [np.float32, np.uint16, np.uint8, np.int64, np.float64, np.int32]
PAD_NAME = {np.float32: "f32", np.uint16: "bf16", np.uint8: "u8", np.int64: "i64", np.float64: "f64", np.int32: "i32"}


def test_warp_worked_example(stg):
    g = json.load(open(os.path.join(GOLDEN, "warp_gather_even_rows.json")))
    say("warp worked example")
    x = to_dev(np.arange(1, 17, dtype=np.float32).reshape(4, 4))
    out = stg.tile_gather(x, to_dev(np.array(g["indices"], dtype=np.int32)), g["tile_shape"], axis=0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), np.array(g["expected"], dtype=np.float32))


def test_row_gather_workload_full(stg, orc):
    w = inputs.row_gather()
    say("row gather workload (1024,256) fp32, 4096 indices")
    out = stg.tile_gather(to_dev(w["a"]), to_dev(w["indices"]), w["tile_shape"], w["offset"], w["axis"])
    torch.cuda.synchronize()
    want = orc.tile_gather(w["a"], w["indices"], w["tile_shape"], w["offset"], w["axis"])
    got = to_host(out)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    n_oob = int(((w["indices"] < 0) | (w["indices"] >= 1024)).sum())
    assert n_oob > 0 and int(np.all(got == 0, axis=1).sum()) >= n_oob


def _random_case(seed):
    rng = np.random.default_rng(seed)
    rank = int(rng.integers(1, 5))
    shape = tuple(int(s) for s in rng.integers(1, 7, rank))
    if rank >= 2:
        shape = shape[:-1] + (int(rng.integers(1, 40)),)  # varied row lengths, ragged tails
    dt = DTYPES[seed % len(DTYPES)]
    a = random_bits(rng, shape, dt)
    axis = int(rng.integers(0, rank))
    tile = [int(rng.integers(1, 5)) for _ in range(rank)]
    if rank >= 2:
        tile[-1] = int(rng.integers(1, shape[-1] + 6))
    n_tiles = int(rng.integers(1, 5))
    idx = rng.integers(-3, shape[axis] + 3, tile[axis] * n_tiles).astype(np.int32)
    offset = [int(o) for o in rng.integers(-3, 4, rank)]
    return rng, a, dt, axis, tile, idx, offset


@pytest.mark.parametrize("seed", range(40))
def test_gather_random(stg, orc, seed):
    rng, a, dt, axis, tile, idx, offset = _random_case(seed)
    say("gather random", seed, a.shape, a.dtype, "axis", axis, "tile", tile, "offset", offset)
    out = stg.tile_gather(to_dev(a), to_dev(idx), tile, offset, axis)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), orc.tile_gather(a, idx, tile, offset, axis))


@pytest.mark.parametrize("seed", range(30))
def test_gather_masked_random(stg, orc, seed):
    rng, a, dt, axis, tile, idx, offset = _random_case(1000 + seed)
    mask = (rng.random(idx.size) < 0.6).astype(np.uint8)
    pad = {np.uint8: 7.0, np.int32: -5.0, np.int64: -9.0}.get(dt, -1.0 if seed % 2 else 0.3)
    say("gather masked random", seed, a.shape, a.dtype, "axis", axis, "tile", tile, "pad", pad)
    out = stg.tile_gather_masked(to_dev(a), to_dev(idx), to_dev(mask), tile, offset, axis, pad)
    torch.cuda.synchronize()
    want = orc.tile_gather_masked(a, idx, mask, tile, offset, axis, pad, PAD_NAME[dt])
    np.testing.assert_array_equal(to_host(out), want)


def test_gather_masked_f16_padding(stg, orc):
    rng = np.random.default_rng(5)
    a = rng.integers(1, 0x7B00, (20, 9)).astype(np.uint16)
    idx = rng.integers(-2, 22, 12).astype(np.int32)
    mask = (rng.random(12) < 0.5).astype(np.uint8)
    for pad in (-1.0, 0.1, 65520.0, -1e-7):
        say("gather masked f16 padding", pad)
        out = stg.tile_gather_masked(to_dev(a, f16=True), to_dev(idx), to_dev(mask), (4, 9), None, 0, pad)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out), orc.tile_gather_masked(a, idx, mask, (4, 9), None, 0, pad, "f16"))
    for pad in (0.1, 3.0e38, -2.0 ** -130):
        say("gather masked bf16 padding", pad)
        out = stg.tile_gather_masked(to_dev(a), to_dev(idx), to_dev(mask), (4, 9), None, 0, pad)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out), orc.tile_gather_masked(a, idx, mask, (4, 9), None, 0, pad, "bf16"))


def test_gather_strided_views(stg, orc):
    rng = np.random.default_rng(9)
    store = rng.integers(1, 0x7F00, (40, 4103)).astype(np.uint16)
    src_h = store[:, :4097]
    idx = rng.integers(-4, 44, 24).astype(np.int32)
    dev = to_dev(store)[:, :4097]  # row stride 4103: rows start 2-byte aligned only
    for off in [(0, 0), (0, -5), (2, 3), (0, 4090)]:
        say("gather unaligned rows, offset", off)
        out = stg.tile_gather(dev, to_dev(idx), (8, 37), off, 0)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out), orc.tile_gather(src_h, idx, (8, 37), off, 0))
    # innermost stride 2 (element path), axis 1 (element path)
    a = rng.standard_normal((12, 10)).astype(np.float32)
    dev = to_dev(a)
    say("gather non-unit inner stride")
    got = stg.tile_gather(dev[:, ::2], to_dev(idx[:8]), (12, 4), (0, 0), 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(got), orc.tile_gather(a[:, ::2], idx[:8], (12, 4), (0, 0), 1))
    # strided output view
    out_store = torch.zeros((24, 50), dtype=torch.float32, device="cuda:0")
    say("gather into a strided output")
    stg.tile_gather(dev, to_dev(idx), (8, 7), (0, 1), 0, out=out_store[:, 3:10])
    torch.cuda.synchronize()
    full = to_host(out_store)
    np.testing.assert_array_equal(full[:, 3:10], orc.tile_gather(a, idx, (8, 7), (0, 1), 0))
    assert not full[:, :3].any() and not full[:, 10:].any()


def test_gather_edge_cases(stg, orc):
    a = np.arange(1, 31, dtype=np.float32).reshape(6, 5)
    dev = to_dev(a)
    say("gather: empty index list")
    out = stg.tile_gather(dev, to_dev(np.zeros(0, np.int32)), (2, 5), None, 0)
    torch.cuda.synchronize()
    assert out.shape == (0, 5)
    say("gather: all indices out of range")
    idx = np.array([-1, 6, 100, -100], dtype=np.int32)
    out = stg.tile_gather(dev, to_dev(idx), (2, 5), None, 0)
    torch.cuda.synchronize()
    assert not to_host(out).any()
    say("gather: mask all false / mask absent")
    idx = np.array([0, 1, 2, 3], dtype=np.int32)
    out = stg.tile_gather_masked(dev, to_dev(idx), to_dev(np.zeros(4, np.uint8)), (2, 5), None, 0, -1.0)
    torch.cuda.synchronize()
    assert np.all(to_host(out).view(np.uint32) == 0xBF800000)
    out = stg.tile_gather_masked(dev, to_dev(idx), None, (2, 5), None, 0, -1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), a[:4])
    say("gather: -0.0 and NaN payloads survive")
    b = np.array([[-0.0, np.nan], [1.0, -np.inf]], dtype=np.float32)
    b.view(np.uint32)[0, 1] = 0x7FA0_0001
    out = stg.tile_gather(to_dev(b), to_dev(np.array([1, 0], np.int32)), (2, 2), None, 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out).view(np.uint32), b[[1, 0]].view(np.uint32))


def test_masked_gather_workload_full(stg, orc):
    """The whole masked-gather workload output (4,194,304 x 128 fp32, 2 GiB),
    compared bit for bit with the oracle in slices of 262,144 indices (whole
    (64, 128) tiles, so each slice is the same gather restricted to its
    indices)."""
    w = inputs.masked()
    table, idx, gmask = w["table"], w["indices"], w["gmask"]
    say("masked gather workload (1048576,128) fp32, 4194304 indices")
    out = stg.tile_gather_masked(to_dev(table), to_dev(idx), to_dev(gmask), (64, 128), None, 0, w["padding_value"])
    torch.cuda.synchronize()
    step = 262144
    n_pad = 0
    for s in range(0, idx.size, step):
        e = min(s + step, idx.size)
        got = to_host(out[s:e])
        want = orc.tile_gather_masked(table, idx[s:e], gmask[s:e], (64, 128), None, 0, w["padding_value"], "f32")
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32), err_msg=f"rows {s}..{e}")
        n_pad += int((want.view(np.uint32) == 0xBF800000).all(axis=1).sum())
    assert n_pad == int((gmask == 0).sum())


@pytest.mark.parametrize("seed", range(30))
def test_scatter_random(stg, orc, seed):
    rng = np.random.default_rng(2000 + seed)
    rank = int(rng.integers(2, 5))
    shape = [int(s) for s in rng.integers(1, 6, rank)]
    shape[-1] = int(rng.integers(1, 30))
    dt = DTYPES[seed % len(DTYPES)]
    axis = int(rng.integers(0, rank - 1)) if seed % 3 else int(rng.integers(0, rank))
    dst0 = random_bits(rng, shape, dt)
    n = shape[axis] + 2
    idx = (rng.permutation(n) - 1).astype(np.int32)  # unique, -1 and shape[axis] out of range
    tile = [int(rng.integers(1, 4)) for _ in range(rank)]
    tile[axis] = n
    tile[-1] = tile[-1] if axis == rank - 1 else int(rng.integers(1, shape[-1] + 4))
    tshape = list(tile)
    vals = random_bits(rng, tshape, dt)
    mask = (rng.random(n) < 0.6).astype(np.uint8)
    offset = [int(o) for o in rng.integers(-2, 3, rank)]
    offset[axis] = 0
    say("scatter random", seed, shape, dt.__name__, "axis", axis, "tile", tile, "offset", offset)
    dev = to_dev(dst0)
    stg.tile_scatter_masked(dev, to_dev(idx), to_dev(mask), tile, to_dev(vals), offset, axis)
    torch.cuda.synchronize()
    want = dst0.copy()
    orc.tile_scatter_masked(want, idx, mask, tile, vals, offset, axis)
    np.testing.assert_array_equal(to_host(dev), want)


def test_scatter_strided_destination(stg, orc):
    rng = np.random.default_rng(12)
    store = rng.integers(1, 0x7F00, (64, 4103)).astype(np.uint16)
    vals = rng.integers(1, 0x7F00, (48, 4097)).astype(np.uint16)
    idx = rng.permutation(64)[:48].astype(np.int32)
    mask = (rng.random(48) < 0.5).astype(np.uint8)
    dev = to_dev(store)
    say("scatter into unaligned-stride rows")
    stg.tile_scatter_masked(dev[:, :4097], to_dev(idx), to_dev(mask), (16, 4097), to_dev(vals), None, 0)
    torch.cuda.synchronize()
    want = store.copy()
    orc.tile_scatter_masked(want[:, :4097], idx, mask, (16, 4097), vals, None, 0)
    np.testing.assert_array_equal(to_host(dev), want)  # includes the ld padding columns


def test_scatter_workload_full(stg, orc):
    w = inputs.masked()
    say("masked scatter workload: 1048576 rows x 128 fp32 to a permutation, Bernoulli(0.5) mask")
    dst = to_dev(w["table"])
    stg.tile_scatter_masked(dst, to_dev(w["perm"]), to_dev(w["smask"]), (64, 128), to_dev(w["vals"]), None, 0)
    torch.cuda.synchronize()
    want = w["table"].copy()
    orc.tile_scatter_masked(want, w["perm"], w["smask"], (64, 128), w["vals"], None, 0)
    np.testing.assert_array_equal(to_host(dst).view(np.uint32), want.view(np.uint32))


def test_scatter_debug_mode_rejects_duplicate_destinations(stg, monkeypatch):
    """STG_DEBUG=1: two active indices with one destination row fail before
    anything is written; duplicates among inactive or out-of-range indices
    are fine; without STG_DEBUG the call is not checked."""
    a = torch.zeros((16, 8), dtype=torch.float32, device="cuda:0")
    vals = torch.ones((4, 8), dtype=torch.float32, device="cuda:0")
    idx = to_dev(np.array([3, 5, 3, 20], dtype=np.int32))
    say("scatter STG_DEBUG duplicate destinations")
    monkeypatch.setenv("STG_DEBUG", "1")
    with pytest.raises(stg.StgError, match="STG_DEBUG"):
        stg.tile_scatter_masked(a, idx, to_dev(np.array([1, 1, 1, 1], np.uint8)), (4, 8), vals, None, 0)
    torch.cuda.synchronize()
    assert not a.any()  # nothing written
    stg.tile_scatter_masked(a, idx, to_dev(np.array([1, 1, 0, 1], np.uint8)), (4, 8), vals, None, 0)
    torch.cuda.synchronize()
    assert a[3].eq(1).all() and a[5].eq(1).all() and a.sum().item() == 16
    dup_out = to_dev(np.array([3, 5, 20, 20], dtype=np.int32))  # row 20 is out of range: nothing written there
    stg.tile_scatter_masked(a, dup_out, to_dev(np.array([1, 1, 1, 1], np.uint8)), (4, 8), vals, None, 0)
    monkeypatch.setenv("STG_DEBUG", "0")
    stg.tile_scatter_masked(a, idx, to_dev(np.array([1, 1, 1, 1], np.uint8)), (4, 8), vals, None, 0)
    torch.cuda.synchronize()


def test_binding_rejects_short_masks(stg):
    a = torch.zeros((16, 8), dtype=torch.float32, device="cuda:0")
    idx = to_dev(np.array([1, 2, 3, 4], dtype=np.int32))
    short = to_dev(np.array([1, 1, 1], np.uint8))
    with pytest.raises(ValueError, match="one entry per index"):
        stg.tile_gather_masked(a, idx, short, (4, 8), None, 0, -1.0)
    with pytest.raises(ValueError, match="one entry per index"):
        stg.tile_scatter_masked(a, idx, short, (4, 8), torch.ones((4, 8), device="cuda:0"), None, 0)


def test_eager_marshalling_matches_the_ctypes_path(stg, orc):
    """Eager tile_gather calls marshal their arguments in C++; prepare()
    records the ctypes form.  Both give the oracle's result bit for bit (with
    and without an offset, on the current and on a given stream), and the
    eager form rejects what the ctypes form rejects."""
    rng = np.random.default_rng(41)
    a = rng.standard_normal((300, 7, 40)).astype(np.float32)
    idx = rng.integers(-8, 310, 96).astype(np.int32)
    ad, idd = to_dev(a), to_dev(idx)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for off, stream in [(None, None), ((0, 2, -5), None), ((3, -1, 9), side)]:
        say("eager vs prepared gather, offset", off, "stream", stream is not None)
        want = orc.tile_gather(a, idx, (32, 4, 16), off, 0)
        eager = stg.tile_gather(ad, idd, (32, 4, 16), off, 0, stream=stream)
        prepared = stg.prepare(stg.tile_gather, ad, idd, (32, 4, 16), off, 0, stream=stream)()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(eager), want)
        np.testing.assert_array_equal(to_host(prepared), want)
    with pytest.raises(ValueError, match="int32"):
        stg.tile_gather(ad, idd.to(torch.int64), (32, 4, 16))
    with pytest.raises(stg.StgError, match="shape"):
        stg.tile_gather(ad, idd, (32, 4, 16), out=torch.empty((96, 4, 15), device="cuda:0"))
    with pytest.raises(ValueError, match="rank"):
        stg.tile_gather(ad.view(300, 7, 40, 1, 1), idd, (32, 4, 16, 1, 1))
    with pytest.raises(TypeError):
        stg.tile_gather(ad, idd, (32, 4, 16), out=np.zeros((96, 4, 16), np.float32))
