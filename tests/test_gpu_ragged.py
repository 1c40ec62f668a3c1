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
