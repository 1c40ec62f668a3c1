"""Prepared calls (binding-level call plans): the marshalling runs once, each
call enqueues the same entry point again.  Results must equal the direct
calls' bit for bit, follow changes to the inputs' contents between calls, and
go to the stream given at preparation or else the current one."""
import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_prepared_row_gather_matches_direct_and_follows_inputs(stg, orc):
    w = inputs.row_gather()
    a, idx = to_dev(w["a"]), to_dev(w["indices"])
    say("prepared row gather (1024,256) fp32, 4096 indices")
    call = stg.prepare(stg.tile_gather, a, idx, w["tile_shape"], w["offset"], w["axis"])
    out = call()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), orc.tile_gather(w["a"], w["indices"], w["tile_shape"], w["offset"],
                                                                  w["axis"]))
    assert call() is out  # the same output tensor every call
    # new contents in the same storage: the next call gathers them
    rng = np.random.default_rng(5)
    a2 = rng.standard_normal(w["a"].shape).astype(np.float32)
    i2 = rng.integers(-64, 1088, w["indices"].size).astype(np.int32)
    a.copy_(torch.from_numpy(a2))
    idx.copy_(torch.from_numpy(i2))
    call()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), orc.tile_gather(a2, i2, w["tile_shape"], w["offset"], w["axis"]))


def test_prepared_masked_gather_and_copy(stg, orc):
    rng = np.random.default_rng(8)
    a = rng.standard_normal((300, 40)).astype(np.float32)
    idx = rng.integers(-5, 305, 128).astype(np.int32)
    mask = (rng.random(128) < 0.7).astype(np.uint8)
    say("prepared masked gather and bounded copy")
    call = stg.prepare(stg.tile_gather_masked, to_dev(a), to_dev(idx), to_dev(mask), (64, 40), None, 0, -2.5)
    out = call()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), orc.tile_gather_masked(a, idx, mask, (64, 40), None, 0, -2.5, "f32"))
    src = rng.integers(1, 0x7F00, (130, 77)).astype(np.uint16)
    cp = stg.prepare(stg.tile_copy_bounded, to_dev(src), 64, 32, -16, -16)
    tiles = cp()
    cp()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(tiles), orc.tile_copy_bounded(src, 64, 32, -16, -16))


def test_prepared_call_uses_the_current_or_given_stream(stg, orc):
    rng = np.random.default_rng(9)
    a = rng.standard_normal((64, 16)).astype(np.float32)
    idx = rng.integers(0, 64, 64).astype(np.int32)
    ad, idd = to_dev(a), to_dev(idx)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("prepared gather on the current stream, then on a given stream")
    call = stg.prepare(stg.tile_gather, ad, idd, (64, 16), None, 0)
    with torch.cuda.stream(side):
        out = call()  # current stream inside the context: side
    side.synchronize()
    np.testing.assert_array_equal(to_host(out), a[idx])
    call2 = stg.prepare(stg.tile_gather, ad, idd, (64, 16), None, 0, stream=side)
    out2 = call2()
    side.synchronize()
    np.testing.assert_array_equal(to_host(out2), a[idx])


def test_prepare_keeps_an_auto_workspace(stg):
    """workspace="auto" under prepare(): allocated once at preparation and
    held by the prepared call, which then matches the unprepared call bit for
    bit, applied once and twice (the grouped backward adds a row's terms in
    one order onto its current value)."""
    gen = torch.Generator(device="cpu").manual_seed(5)
    idx = torch.randint(0, 128, (64,), generator=gen, dtype=torch.int32).to("cuda:0")
    go = torch.randn((64, 8), generator=gen).to("cuda:0")
    ref = torch.zeros((128, 8), dtype=torch.float32, device="cuda:0")
    g = torch.zeros((128, 8), dtype=torch.float32, device="cuda:0")
    say("prepared grouped backward with an auto workspace")
    call = stg.prepare(stg.tile_gather_backward, g, idx, (64, 8), go, workspace="auto")
    for _ in range(2):
        stg.tile_gather_backward(ref, idx, (64, 8), go, workspace="auto")
        call()
        torch.cuda.synchronize()
        assert torch.equal(g, ref)
