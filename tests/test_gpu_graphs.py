"""The entry points under HIP graph capture (torch.cuda.CUDAGraph): a
sequence of calls captured once and replayed, with eager work and
synchronization between replays, reproduces the eager results bit for bit
on every replay.  No entry point records a memset or a host synchronization,
so nothing in them is replayed differently from how it ran eagerly."""
import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_captured_sequence_replays_like_eager(stg):
    dev = "cuda:0"
    g = torch.Generator(device="cpu").manual_seed(31)
    a = torch.randn((1024, 256), generator=g).to(dev)
    idx = torch.randint(-64, 1088, (4096,), generator=g, dtype=torch.int32).to(dev)
    src = torch.randn((300, 129), generator=g).to(torch.bfloat16).to(dev)
    sg = inputs.scaled_gemm(300, 260, 256, "e4m3")
    A, Bt = torch.from_numpy(sg["A"]).to(dev), torch.from_numpy(sg["Bt"]).to(dev)
    sa, sb = torch.from_numpy(sg["sa"]).to(dev), torch.from_numpy(sg["sb"]).to(dev)
    grad = torch.zeros((1024, 256), device=dev)
    gout = torch.randn((4096, 256), generator=g).to(dev)
    ws = torch.empty(stg.tile_gather_backward_workspace(grad, 4096, (64, 256), 0), dtype=torch.uint8, device=dev)

    gathered = torch.empty((4096, 256), device=dev)
    tiles = torch.empty((stg.stg_tile_grid(300, -16, 64), stg.stg_tile_grid(129, -16, 32), 64, 32),
                        dtype=torch.bfloat16, device=dev)
    dst = torch.full((300, 129), 7.0, dtype=torch.bfloat16, device=dev)
    C = torch.empty((300, 260), device=dev)
    # the general block-scaled path (e4m3 scales per 16 values)
    rng = np.random.default_rng(31)
    sa16 = torch.from_numpy(rng.integers(0x30, 0x48, (300, 16), dtype=np.uint8)).to(dev)
    sb16 = torch.from_numpy(rng.integers(0x30, 0x48, (260, 16), dtype=np.uint8)).to(dev)
    C16 = torch.empty((300, 260), device=dev)
    # the static-scratch backward and a prepared gather
    grad2 = torch.zeros((1024, 256), device=dev)
    gathered2 = torch.empty((4096, 256), device=dev)
    prepared = stg.prepare(stg.tile_gather, a, idx, (64, 256), out=gathered2)

    def seq():
        stg.tile_gather(a, idx, (64, 256), out=gathered)
        stg.tile_copy_bounded(src, 64, 32, -16, -16, out=tiles)
        stg.tile_store_clipped(tiles, -16, -16, dst)
        stg.gemm_scaled(A, "e4m3", sa, Bt, "e4m3", sb, 256, 32, out=C)
        grad.zero_()
        stg.tile_gather_backward(grad, idx, (64, 256), gout, workspace=ws)
        stg.gemm_scaled(A, "e4m3", sa16, Bt, "e4m3", sb16, 256, 16, scale_fmt="e4m3", out=C16)
        grad2.zero_()
        stg.tile_gather_backward_static(grad2, idx, (64, 256), gout)
        prepared()

    say("graph capture: eager reference")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):  # warm up on the capture stream (configures the GEMM's LDS)
            seq()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    want = [t.clone() for t in (gathered, tiles, dst, C, C16, gathered2)]
    grad_eager = grad.clone()
    grad2_eager = grad2.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        seq()
    for r in range(3):
        say("graph replay", r)
        for t in (gathered, tiles, C, C16, gathered2, grad2):
            t.fill_(-3.0)  # eager work between replays: clobber every output
        dst.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((gathered, tiles, dst, C, C16, gathered2), want):
            assert torch.equal(got, ref)
        # the grouped backward's sums are order-independent only up to rounding:
        # compare against the eager run within a few ulps of the magnitudes
        assert torch.allclose(grad, grad_eager, rtol=1e-5, atol=1e-5)
        assert torch.allclose(grad2, grad2_eager, rtol=1e-5, atol=1e-5)
        assert torch.allclose(grad2, grad, rtol=1e-5, atol=1e-5)
