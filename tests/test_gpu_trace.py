"""Kernel tracing records one kernel-only duration per launch, in order."""
import numpy as np
import pytest
import torch

from scatter_tile_gather_amd import inputs
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def test_trace_records_each_launch(stg):
    w = inputs.bounded_copy(M=300, N=129, ld=135)
    src = to_dev(w["src"])[:, :129]
    g = inputs.gemm(300, 530, 64)  # 512 main columns + an 18-column edge strip
    g2 = inputs.gemm(300, 515, 64)  # 512 main columns + a 3-column skinny strip
    say("trace: copy, store, gemm")
    stg.stg_trace_read()
    stg.stg_trace_enable(True)
    try:
        tiles = stg.tile_copy_bounded(src, 64, 32, -16, -16)
        stg.tile_store_clipped(tiles, -16, -16, to_dev(w["dst"])[:, :129])
        stg.gemm_bounded(to_dev(g["A"]), to_dev(g["B"]))
        stg.gemm_bounded(to_dev(g2["A"]), to_dev(g2["B"]))
        torch.cuda.synchronize()
    finally:
        stg.stg_trace_enable(False)
    rec = stg.stg_trace_read()
    assert [n for n, _ in rec] == ["tile_copy_bounded", "tile_store_clipped", "gemm_bounded/main",
                                   "gemm_bounded/edge", "gemm_bounded/main", "gemm_bounded/skinny"]
    assert all(0.0 < ms < 100.0 for _, ms in rec)
    assert stg.stg_trace_read() == []
