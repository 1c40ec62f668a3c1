"""tile_gather_backward_static (grouped gather backward with the library's
static scratch array, allocating nothing) against tile_gather_backward with a
caller workspace and against the fp64 oracle: two calls in a row on one GPU,
the second with a smaller input, so the second runs on scratch the first
left filled.

Bar: the gradient is a float sum in an unspecified order, so each result
lies within gamma_k * S of the oracle's exact sum (k terms on the element,
S = |initial| + sum |terms|, as in the backward parity tests) and the two
entry points within twice that of each other; elements with no term keep
their bits."""
import numpy as np
import pytest
import torch

from gpu_util import say, to_dev, to_host
from test_gpu_gather_backward import _gamma, check_backward

pytestmark = pytest.mark.gpu


def _case(seed, rows, cols, n, dtype):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-3, rows + 3, n).astype(np.int32)  # a few out of range
    idx[: n // 50] = 7  # one hot row: its segment is split into pieces
    g = rng.standard_normal((n, cols)).astype(dtype)
    a0 = rng.standard_normal((rows, cols)).astype(dtype)
    return idx, g, a0


@pytest.mark.parametrize("order", ["large_then_small"])
def test_static_scratch_matches_workspace_entry_point(stg, orc, order):
    cases = [(101, 1 << 16, 128, 1 << 20, np.float32), (102, 5000, 40, 1 << 17, np.float64)]
    for seed, rows, cols, n, dtype in cases:
        idx, g, a0 = _case(seed, rows, cols, n, dtype)
        tile = (64, cols)
        i_dev, g_dev = to_dev(idx), to_dev(g)
        a_ws, a_st = to_dev(a0), to_dev(a0)
        need = stg.tile_gather_backward_workspace(a_ws, n, tile, 0)
        assert 0 < need <= stg.STATIC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        say("static-scratch gather backward", rows, "rows", cols, "cols", n, "terms", np.dtype(dtype).name)
        stg.tile_gather_backward(a_ws, i_dev, tile, g_dev, None, 0, workspace=ws)
        stg.tile_gather_backward_static(a_st, i_dev, tile, g_dev, None, 0)
        torch.cuda.synchronize()
        got_ws, got_st = to_host(a_ws), to_host(a_st)
        acc, abs_sum, count = orc.tile_gather_backward(a0, idx, tile, g, None, 0)
        assert count.max() > 64  # the hot row's pieces ran
        check_backward(got_ws, a0, acc, abs_sum, count)
        check_backward(got_st, a0, acc, abs_sum, count)
        u = 2.0 ** -24 if dtype == np.float32 else 2.0 ** -53
        tol = 2 * (_gamma(count, u) + _gamma(count, 2.0 ** -53)) * abs_sum
        assert np.all(np.abs(got_st.astype(np.float64) - got_ws.astype(np.float64)) <= tol)


def test_static_scratch_rejects_oversized_call(stg):
    """A call whose scratch would exceed the static array fails before any
    launch and leaves the gradient untouched."""
    rows, cols = 1 << 21, 16
    n = 1 << 23
    a = torch.zeros((rows, cols), dtype=torch.float32, device="cuda:0")
    assert stg.tile_gather_backward_workspace(a, n, (64, cols), 0) > stg.STATIC_SCRATCH_BYTES
    idx = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    g = torch.ones((n, cols), dtype=torch.float32, device="cuda:0")
    say("static-scratch gather backward, oversized call")
    with pytest.raises(stg.StgError, match="static array"):
        stg.tile_gather_backward_static(a, idx, (64, cols), g, None, 0)
    torch.cuda.synchronize()
    assert not a.any()
