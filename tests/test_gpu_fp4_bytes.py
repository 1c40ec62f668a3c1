"""FP4 (e2m1) values carried two per byte (cuTile.jl Operations, reinterpret:
a UInt8 tile viewed as twice as many Float4_E2M1FN values) move through the
tile kernels as plain bytes and reach the block-scaled GEMM intact.

Movement is compared bit for bit with the oracle; the GEMM on gathered FP4
rows against the fp64 oracle on the oracle's gather, within gamma_K *
sum|terms| (fp4 products and e8m0 scales are exact in fp32)."""
import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_fp4_tiles_copy_and_store_as_bytes(stg, orc):
    rng = np.random.default_rng(41)
    M, K = 257, 190  # 95 bytes per row: the last tile column is partial
    A = inputs.pack_e2m1(inputs.lowp_codes(rng, (M, K), "e2m1"))
    say("fp4 bytes: bounded copy (64, 16) at (-8, -4) of", A.shape)
    tiles = stg.tile_copy_bounded(to_dev(A), 64, 16, -8, -4)
    torch.cuda.synchronize()
    want = orc.tile_copy_bounded(A, 64, 16, -8, -4)
    np.testing.assert_array_equal(to_host(tiles), want)
    # zero bytes are pairs of FP4 zeros: the zero fill is FP4 zero too
    assert orc.decode_lowp(np.zeros(1, np.uint8), "e2m1")[0] == 0.0
    dst = torch.full((M, A.shape[1]), 0xA5, dtype=torch.uint8, device="cuda:0")
    stg.tile_store_clipped(tiles, -8, -4, dst)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(dst), A)


def test_fp4_gathered_rows_feed_the_scaled_gemm(stg, orc):
    rng = np.random.default_rng(42)
    rows, K, N = 300, 256, 96
    table = inputs.pack_e2m1(inputs.lowp_codes(rng, (rows, K), "e2m1"))
    idx = rng.integers(-10, rows + 10, 160).astype(np.int32)  # some rows out of range: zeros
    Bt = inputs.pack_e2m1(inputs.lowp_codes(rng, (N, K), "e2m1"))
    sa = rng.integers(120, 134, (idx.size, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 134, (N, K // 32)).astype(np.uint8)
    say("fp4 bytes: gather", idx.size, "rows of", table.shape, "then gemm_scaled N", N, "K", K)
    g = stg.tile_gather(to_dev(table), to_dev(idx), (32, table.shape[1]), None, 0)
    C = stg.gemm_scaled(g, "e2m1", to_dev(sa), to_dev(Bt), "e2m1", to_dev(sb), K, 32)
    torch.cuda.synchronize()
    g_want = orc.tile_gather(table, idx, (32, table.shape[1]), None, 0)
    np.testing.assert_array_equal(to_host(g), g_want)
    want = orc.gemm_scaled_f64(g_want, "e2m1", sa, Bt, "e2m1", sb, K, 32)
    mag = orc.gemm_scaled_f64(g_want & 0x77, "e2m1", sa, Bt & 0x77, "e2m1", sb, K, 32)
    u = 2.0 ** -24
    tol = K * u / (1 - K * u) * mag + 1e-30
    assert np.all(np.abs(to_host(C).astype(np.float64) - want) <= tol)
