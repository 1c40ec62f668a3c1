"""GPU parity of ragged_tile_load against the CPU oracle (bit-exact)."""
import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import random_bits, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(stg, orc, X, md, group, BM, BN, col0, ri, dyn, mi):
    out = stg.ragged_tile_load(to_dev(X), md, group, BM, BN, to_dev(ri.astype(np.int32)), to_dev(dyn.astype(np.int32)),
                               to_dev(mi.astype(np.int32)), col0=col0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), orc.ragged_tile_load(X, md, group, BM, BN, col0, ri, dyn, mi))


@pytest.mark.parametrize("group", [1, 4])
def test_ragged_workload_full(stg, orc, group):
    w = inputs.ragged()
    md = w["heads"] // group
    bm_seq = 128 // group
    ri, dyn, mi = stg.ragged_tile_schedule(w["seq_lens"], bm_seq, md)
    say("ragged workload group", group, "tiles", len(ri), "rows", w["X"].shape[0])
    _run(stg, orc, w["X"], md, group, 128, 128, 0, ri, dyn, mi)


@pytest.mark.parametrize("seed", range(24))
def test_ragged_random(stg, orc, seed):
    rng = np.random.default_rng(5000 + seed)
    dt = [np.uint16, np.float32, np.uint8, np.float64][seed % 4]
    group = int(rng.choice([1, 2, 4]))
    md = int(rng.integers(1, 4))
    depth = int(rng.integers(1, 80))
    bm_seq = int(rng.integers(1, 12))
    BM = bm_seq * group
    BN = int(rng.integers(1, depth + 10))
    col0 = int(rng.integers(0, depth))
    lens = rng.integers(1, 30, int(rng.integers(1, 6)))
    total = int(lens.sum())
    X = random_bits(rng, (total, md * group, depth), dt)
    ri, dyn, mi = stg.ragged_tile_schedule(lens, bm_seq, md)
    # guarded triples: dynamic_dim past BM_seq, rows past the end, head past middle_dim
    extra = np.array([[total - 1, bm_seq + 5, 0], [total + 3, 2, 0], [0, 1, md], [0, 0, 0]], dtype=np.uint32)
    ri = np.concatenate([ri, extra[:, 0]])
    dyn = np.concatenate([dyn, extra[:, 1]])
    mi = np.concatenate([mi, extra[:, 2]])
    say("ragged random", seed, dt.__name__, "group", group, "md", md, "depth", depth, "BM", BM, "BN", BN, "col0", col0)
    _run(stg, orc, X, md, group, BM, BN, col0, ri, dyn, mi)


# ---- store direction ---------------------------------------------------------

def _store(stg, orc, tiles, X0, md, group, col0, ri, dyn, mi):
    """Store `tiles` into a device copy of X0 and compare every element of the
    result (written and untouched alike) with the oracle."""
    dst = to_dev(X0)
    stg.ragged_tile_store(to_dev(tiles), dst, md, group, to_dev(ri.astype(np.int32)), to_dev(dyn.astype(np.int32)),
                          to_dev(mi.astype(np.int32)), col0=col0)
    torch.cuda.synchronize()
    want = orc.ragged_tile_store(tiles, X0, md, group, col0, ri, dyn, mi)
    np.testing.assert_array_equal(to_host(dst), want)
    return want


@pytest.mark.parametrize("group", [1, 4])
def test_ragged_store_workload_full(stg, orc, group):
    w = inputs.ragged()
    md = w["heads"] // group
    bm_seq = 128 // group
    ri, dyn, mi = stg.ragged_tile_schedule(w["seq_lens"], bm_seq, md)
    rng = np.random.default_rng(777 + group)
    tiles = random_bits(rng, (len(ri), 128, 128), np.uint16)
    say("ragged store workload group", group, "tiles", len(ri), "rows", w["X"].shape[0])
    _store(stg, orc, tiles, w["X"], md, group, 0, ri, dyn, mi)


@pytest.mark.parametrize("group", [1, 4])
def test_ragged_store_load_round_trip(stg, group):
    """load then store over the covering schedule rebuilds X in a
    sentinel-filled array, on the device alone."""
    w = inputs.ragged(n_seqs=9, max_len=700)
    md = w["heads"] // group
    ri, dyn, mi = stg.ragged_tile_schedule(w["seq_lens"], 128 // group, md)
    trip = [to_dev(a.astype(np.int32)) for a in (ri, dyn, mi)]
    X = to_dev(w["X"])
    say("ragged store round trip group", group, "tiles", len(ri))
    tiles = stg.ragged_tile_load(X, md, group, 128, 128, *trip)
    dst = torch.full_like(X, -7.0)
    stg.ragged_tile_store(tiles, dst, md, group, *trip)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(dst), w["X"])


@pytest.mark.parametrize("seed", range(24))
def test_ragged_store_random(stg, orc, seed):
    rng = np.random.default_rng(9000 + seed)
    dt = [np.uint16, np.float32, np.uint8, np.float64][seed % 4]
    group = int(rng.choice([1, 2, 4]))
    md = int(rng.integers(1, 4))
    depth = int(rng.integers(1, 80))
    bm_seq = int(rng.integers(1, 12))
    BM = bm_seq * group
    BN = int(rng.integers(1, depth + 10))
    col0 = int(rng.integers(0, depth))
    lens = rng.integers(1, 30, int(rng.integers(1, 6)))
    total = int(lens.sum())
    X0 = random_bits(rng, (total, md * group, depth), dt)
    ri, dyn, mi = stg.ragged_tile_schedule(lens, bm_seq, md)
    # guarded triples that write nothing: rows past the end, head past middle_dim, no rows
    extra = np.array([[total + 3, 2, 0], [0, 1, md], [0, 0, 0]], dtype=np.uint32)
    ri = np.concatenate([ri, extra[:, 0]])
    dyn = np.concatenate([dyn, extra[:, 1]])
    mi = np.concatenate([mi, extra[:, 2]])
    tiles = random_bits(rng, (len(ri), BM, BN), dt)
    say("ragged store random", seed, dt.__name__, "group", group, "md", md, "depth", depth, "BM", BM, "BN", BN,
        "col0", col0)
    X1 = _store(stg, orc, tiles, X0, md, group, col0, ri, dyn, mi)
    # a dynamic_dim past BM_seq and past the end of the array, applied afterwards on its own
    one = random_bits(rng, (1, BM, BN), dt)
    _store(stg, orc, one, X1, md, group, col0, np.array([total - 1], np.uint32), np.array([bm_seq + 5], np.uint32),
           np.array([0], np.uint32))


def test_ragged_load_rejects_a_small_out(stg):
    X = torch.zeros((40, 8, 128), dtype=torch.bfloat16, device="cuda:0")
    ri, dyn, mi = stg.ragged_tile_schedule([40], 128, 8)
    trip = [to_dev(t.astype(np.int32)) for t in (ri, dyn, mi)]
    small = torch.empty((len(ri), 64, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError, match="out must be"):
        stg.ragged_tile_load(X, 8, 1, 128, 128, *trip, out=small)


# ---- tiles spanning many workgroup slices --------------------------------------

@pytest.mark.parametrize("case", [
    # dtype, group, md, depth, BM, BN, col0: 4800 vectors = 18 whole slices of 256 and a tail of 192
    (np.float32, 1, 3, 210, 96, 200, 7),
    # 16-byte rows of a 1-byte type: one vector per row, 4 whole slices and a tail of 8
    (np.uint8, 4, 2, 40, 1032, 16, 24),
    # exactly 2 slices, every row whole vectors (the unchecked-interior instance)
    (np.uint16, 2, 2, 64, 64, 64, 0),
])
def test_ragged_many_slices(stg, orc, case):
    dt, group, md, depth, BM, BN, col0 = case
    rng = np.random.default_rng(4242 + BM)
    bm_seq = BM // group
    lens = np.array([bm_seq * 2 + 5, 3, bm_seq, 1, bm_seq + 1], dtype=np.int64)
    total = int(lens.sum())
    X0 = random_bits(rng, (total, md * group, depth), dt)
    ri, dyn, mi = stg.ragged_tile_schedule(lens, bm_seq, md)
    say("ragged many slices", dt.__name__, "group", group, "md", md, "depth", depth, "BM", BM, "BN", BN, "tiles",
        len(ri))
    _run(stg, orc, X0, md, group, BM, BN, col0, ri, dyn, mi)
    tiles = random_bits(rng, (len(ri), BM, BN), dt)
    _store(stg, orc, tiles, X0, md, group, col0, ri, dyn, mi)
