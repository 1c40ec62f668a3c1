"""GPU parity of tile_gather_backward against the fp64 CPU oracle.

The accumulation is atomic, so the order of the terms that land on one
element is unspecified.  Tolerance (derived from the arithmetic): an element
that receives k terms, summed in any order in the gradient's precision with
unit roundoff u (2^-24 for fp32, 2^-53 for fp64), differs from the exact sum
by at most gamma_k * S, gamma_k = k u / (1 - k u), where S is the sum of the
magnitudes of the initial value and of every term; the fp64 oracle's own
rounding adds at most gamma_k(2^-53) * S.  Elements with no term keep their
initial bits exactly, and a single term onto zero is exact.
"""
import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gamma(k, u):
    ku = k * u
    return ku / (1.0 - ku)


def check_backward(got, a0, acc, abs_sum, count):
    u = 2.0 ** -24 if got.dtype == np.float32 else 2.0 ** -53
    tol = (_gamma(count, u) + _gamma(count, 2.0 ** -53)) * abs_sum
    err = np.abs(got.astype(np.float64) - acc)
    assert np.all(err <= tol), float((err - tol).max())
    untouched = count == 0
    np.testing.assert_array_equal(got[untouched], a0[untouched])


def run_case(stg, orc, a0, idx, tile, g, off=None, axis=0, ws=None):
    a_dev = to_dev(a0.copy())
    stg.tile_gather_backward(a_dev, to_dev(idx.astype(np.int32)), tile, to_dev(g), off, axis, workspace=ws)
    torch.cuda.synchronize()
    got = to_host(a_dev)
    acc, abs_sum, count = orc.tile_gather_backward(a0, idx, tile, g, off, axis)
    check_backward(got, a0, acc, abs_sum, count)
    return got, count


@pytest.mark.parametrize("ws", [None, "auto"])
def test_backward_row_gather_workload(stg, orc, ws):
    w = inputs.row_gather()
    rng = np.random.default_rng(2024)
    a0 = np.zeros(w["a"].shape, np.float32)
    g = rng.standard_normal((w["indices"].size, w["a"].shape[1])).astype(np.float32)
    say("gather backward: row gather workload (1024,256) fp32, 4096 indices with repeats and out-of-range, ws", ws)
    _, count = run_case(stg, orc, a0, w["indices"], w["tile_shape"], g, w["offset"], w["axis"], ws)
    assert count.max() >= 3  # repeated rows really accumulate


@pytest.mark.parametrize("ws", [None, "auto"])
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_backward_permutation_is_exact(stg, orc, dtype, ws):
    rng = np.random.default_rng(11)
    idx = rng.permutation(512).astype(np.int32)
    g = rng.standard_normal((512, 96)).astype(dtype)
    say("gather backward: permutation (512,96)", np.dtype(dtype).name, "ws", ws)
    got, _ = run_case(stg, orc, np.zeros((512, 96), dtype), idx, (64, 96), g, ws=ws)
    want = np.zeros((512, 96), dtype)
    want[idx] = g
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("ws", [None, "auto"])
@pytest.mark.parametrize("seed", range(20))
def test_backward_random(stg, orc, seed, ws):
    rng = np.random.default_rng(6100 + seed)
    dtype = [np.float32, np.float64][seed % 2]
    rank = int(rng.integers(2, 5))
    shape = [int(rng.integers(1, 12)) for _ in range(rank)]
    shape[-1] = int(rng.integers(1, 70))
    axis = int(rng.integers(0, rank))
    tile = [int(rng.integers(1, s + 3)) for s in shape]
    T = tile[axis]
    n_idx = T * int(rng.integers(1, 6))
    idx = rng.integers(-3, shape[axis] + 3, n_idx).astype(np.int32)  # repeats and out-of-range
    off = [int(rng.integers(-2, 3)) for _ in range(rank)]
    off[axis] = int(rng.integers(-1, 2))
    g_shape = list(tile)
    g_shape[axis] = n_idx
    a0 = rng.standard_normal(shape).astype(dtype)
    g = rng.standard_normal(g_shape).astype(dtype)
    say("gather backward random", seed, np.dtype(dtype).name, "shape", shape, "tile", tile, "axis", axis, "off", off,
        "n_idx", n_idx, "ws", ws)
    run_case(stg, orc, a0, idx, tile, g, off, axis, ws)


@pytest.mark.parametrize("ws", [None, "auto"])
def test_backward_embedding_scale(stg, orc, ws):
    """(262144, 128) fp32 gradient table, 1,048,576 indices drawn uniformly
    (about four terms per row), (64, 128) tiles."""
    rng = np.random.default_rng(77)
    rows = 262144
    idx = rng.integers(0, rows, 1048576).astype(np.int32)
    g = rng.standard_normal((idx.size, 128)).astype(np.float32)
    a0 = rng.standard_normal((rows, 128)).astype(np.float32)
    say("gather backward: embedding scale (262144,128) fp32, 1048576 indices, ws", ws)
    run_case(stg, orc, a0, idx, (64, 128), g, ws=ws)


@pytest.mark.parametrize("dist", ["uniform", "zipf"])
def test_backward_grouped_workload_full(stg, orc, dist):
    """The timed gather-backward workloads at full size, in the grouped
    execution the benchmark runs: a (1048576, 128) fp32 gradient, 4,194,304
    indices in (64, 128) tiles, drawn uniformly or from Zipf(1.1) truncated to
    the table (the hottest row takes 519,112 terms: its pieces, the
    many-workgroup build of the hot buckets and the one-launch sums at the
    sizes they run at), every element against the fp64 oracle."""
    rows, n = 1 << 20, 1 << 22
    rng = np.random.default_rng(4242 + (dist == "zipf"))
    idx = inputs.zipf_indices(rows=rows, n=n) if dist == "zipf" else rng.integers(0, rows, n).astype(np.int32)
    g = rng.standard_normal((n, 128), dtype=np.float32)
    a0 = rng.standard_normal((rows, 128), dtype=np.float32)
    say("gather backward grouped: full workload", dist)
    _, count = run_case(stg, orc, a0, idx, (64, 128), g, ws="auto")
    if dist == "zipf":
        assert int(count.max()) == 519112  # terms onto each element of the hottest row


def test_backward_grouped_long_segments(stg, orc):
    """Grouped execution with a skewed index list: one row takes 5000 terms,
    a few others hundreds, most none."""
    rng = np.random.default_rng(91)
    idx = np.concatenate([np.full(5000, 7), rng.integers(0, 40, 3000), rng.integers(0, 4096, 192)]).astype(np.int32)
    rng.shuffle(idx)
    g = rng.standard_normal((idx.size, 40)).astype(np.float32)
    a0 = rng.standard_normal((4096, 40)).astype(np.float32)
    say("gather backward grouped: skewed segments")
    run_case(stg, orc, a0, idx, (8, 40), g, ws="auto")


@pytest.mark.parametrize("rows,cols,n_tiles", [
    (3 * 2 ** 20 + 5, 2, 5000),  # more than 2^20 destination rows: 769 buckets of 4096 rows
    (2 ** 24 + 4099, 1, 4000),   # more than 2^24 rows: buckets of two 4096-row windows
])
def test_backward_grouped_large_tables(stg, orc, rows, cols, n_tiles):
    """Grouped execution on tables past the single-window bucket sizes, with
    out-of-range indices and one heavy row in the last bucket."""
    rng = np.random.default_rng(rows % 1000)
    n = 64 * n_tiles
    idx = rng.integers(-2, rows + 2, n).astype(np.int32)
    idx[: n // 8] = rows - 1
    rng.shuffle(idx)
    g = rng.standard_normal((n, cols)).astype(np.float32)
    a0 = rng.standard_normal((rows, cols)).astype(np.float32)
    say("gather backward grouped: large table", rows, "x", cols, "terms", n)
    run_case(stg, orc, a0, idx, (64, cols), g, ws="auto")


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_backward_grouped_segment_pieces(stg, orc, dtype):
    """Rows whose segments are just under, at and past multiples of the
    64-term piece a reduce group sums (63, 64, 65, 127, 128, 129, 1000 and
    7000 terms): longer segments are split over several groups that add
    their partial sums atomically."""
    rng = np.random.default_rng(64 + (dtype == np.float64))
    counts = {3: 63, 10: 64, 17: 65, 40: 127, 41: 128, 42: 129, 77: 1000, 90: 7000}
    fill = 500 + (-(sum(counts.values()) + 500)) % 8  # other rows' terms, to a whole number of tiles
    idx = np.concatenate([np.full(c, r) for r, c in counts.items()] + [rng.integers(100, 200, fill)]).astype(np.int32)
    rng.shuffle(idx)
    n = idx.size
    assert n % 8 == 0 and all(int((idx == r).sum()) == c for r, c in counts.items())
    g = rng.standard_normal((n, 24)).astype(dtype)
    a0 = rng.standard_normal((200, 24)).astype(dtype)
    say("gather backward grouped: segment pieces", np.dtype(dtype).name, "terms", n)
    run_case(stg, orc, a0, idx, (8, 24), g, ws="auto")


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("cols,col_off", [(24, 0), (37, 3), (40, -5), (600, 0), (601, 3)])
def test_backward_grouped_row_groups(stg, orc, dtype, cols, col_off):
    """The reduce sums four consecutive destination rows per group as one run
    of terms.  Terms per row, group by group: runs that cross empty rows,
    groups that mix short segments with long ones (left to the pieces),
    segments of exactly 64 and 65 terms, an empty group, and a last group cut
    short by the table's end (35 rows); column windows that start inside a
    16-byte chunk or are clipped on the left, so element reads at the edges,
    and rows wider than a wavefront's 64 chunks, so several chunks per lane."""
    rng = np.random.default_rng(4000 + cols + (dtype == np.float64))
    pattern = [0, 1, 63, 64, 65, 0, 2, 200, 1, 1, 1, 1, 0, 0, 0, 0, 300, 5, 0, 64, 0, 3, 0, 0, 7, 0, 0, 9,
               64, 65, 64, 65, 2, 0, 4]
    R = len(pattern)
    idx = np.concatenate([np.full(c, r) for r, c in enumerate(pattern) if c]).astype(np.int32)
    rng.shuffle(idx)
    assert R % 4 == 3 and all(int((idx == r).sum()) == c for r, c in enumerate(pattern))
    g = rng.standard_normal((idx.size, cols)).astype(dtype)
    a0 = rng.standard_normal((R, cols + 4)).astype(dtype)
    say("gather backward grouped: row groups", np.dtype(dtype).name, "cols", cols, "col_off", col_off)
    _, count = run_case(stg, orc, a0, idx, (1, cols), g, off=[0, col_off], ws="auto")
    assert count.max() >= 300


def test_backward_grouped_hot_row(stg, orc):
    """One row takes 300,000 terms, more than 4096 pieces of 64: its pieces
    grow (74 terms) so that at most 4096 partial sums meet on the row."""
    rng = np.random.default_rng(300)
    idx = np.concatenate([np.full(300000, 5), rng.integers(0, 1000, 4000)]).astype(np.int32)
    rng.shuffle(idx)
    g = rng.standard_normal((idx.size, 3)).astype(np.float32)
    a0 = rng.standard_normal((1000, 3)).astype(np.float32)
    say("gather backward grouped: hot row of 300000 terms")
    run_case(stg, orc, a0, idx, (8, 3), g, ws="auto")


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_backward_grouped_hot_buckets(stg, orc, dtype):
    """Skewed indices that make buckets of more than 16384 terms, which many
    workgroups build slice by slice: Zipf-distributed rows over a (70000, 20)
    table (row 0 alone takes about a third of the 300,000 terms), plus a block
    of rows hit uniformly."""
    rng = np.random.default_rng(1100 + (dtype == np.float64))
    idx = np.concatenate([np.minimum(rng.zipf(1.3, 240000) - 1, 69999), rng.integers(40000, 70000, 60000)])
    idx = idx.astype(np.int32)
    rng.shuffle(idx)
    g = rng.standard_normal((idx.size, 20)).astype(dtype)
    a0 = rng.standard_normal((70000, 20)).astype(dtype)
    say("gather backward grouped: hot buckets", np.dtype(dtype).name, "max count", int(np.bincount(idx).max()))
    run_case(stg, orc, a0, idx, (8, 20), g, ws="auto")


def test_backward_auto_workspace_on_side_stream(stg, orc):
    """workspace="auto" with the kernels on a side stream: the workspace is
    released when the call returns, while its kernels may still run there.
    Tensors allocated and filled on the default stream right after must not
    receive that block; the gradient still matches the oracle."""
    rng = np.random.default_rng(31)
    rows, cols, n = 1 << 16, 64, 1 << 20
    idx = rng.integers(0, rows, n).astype(np.int32)
    g = rng.standard_normal((n, cols)).astype(np.float32)
    a0 = np.zeros((rows, cols), np.float32)
    a_dev, i_dev, g_dev = to_dev(a0), to_dev(idx), to_dev(g)
    nb = stg.tile_gather_backward_workspace(a_dev, n, (64, cols), 0)
    assert nb > 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("gather backward, auto workspace on a side stream, then default-stream allocations of the same size")
    stg.tile_gather_backward(a_dev, i_dev, (64, cols), g_dev, None, 0, workspace="auto", stream=side)
    fills = [torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda:0") for _ in range(4)]
    torch.cuda.synchronize()
    assert all(int(f.min()) == 0xFF for f in fills)
    acc, abs_sum, count = orc.tile_gather_backward(a0, idx, (64, cols), g, None, 0)
    check_backward(to_host(a_dev), a0, acc, abs_sum, count)


def test_backward_grouped_many_scan_blocks(stg, orc):
    """40,000,000 terms onto 2^20 one-value rows: the bucket-count table has
    512 x 9,766 entries, 4,883 scan blocks, past the 4,096 up to which the
    offsets kernel sums the blocks before its own itself -- so a separate
    scan of the block sums runs (the other form is taken by every other
    grouped case).  Within gamma_k * sum|terms| of the fp64 oracle."""
    rows, n = 1 << 20, 40_000_000
    rng = np.random.default_rng(2024)
    idx = rng.integers(0, rows, n).astype(np.int32)
    g = rng.standard_normal((n, 1)).astype(np.float32)
    a0 = np.zeros((rows, 1), np.float32)
    say("gather backward grouped, 40M terms onto 2^20 rows of one value (many scan blocks)")
    run_case(stg, orc, a0, idx, (64, 1), g, ws="auto")
