"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/stg.h declares, and its host-only logic (grid sizing, ragged
schedule, argument validation) behaves as documented.  No kernel is launched:
every call here either is host-only or fails validation before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import scatter_tile_gather_amd as stg_pkg
from scatter_tile_gather_amd._binding import StgTensor

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "stg.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s+\**([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(stg):
    lib = stg.load_library()
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(stg_pkg.exported_names()) == names
    assert stg.stg_version() >= 100
    assert lib.stg_last_error() is not None


def test_tile_grid_matches_oracle(stg, orc):
    for extent in range(0, 50):
        for origin in range(-20, 52, 3):
            for t in (1, 2, 7, 16, 64):
                assert stg.stg_tile_grid(extent, origin, t) == orc.tile_grid(extent, origin, t)
    assert stg.stg_tile_grid(10, 0, 0) == -1
    assert stg.stg_tile_grid(8191, -16, 64) == 129
    assert stg.stg_tile_grid(4097, 0, 32) == 129


@pytest.mark.parametrize("seed", range(5))
def test_ragged_schedule_matches_oracle(stg, orc, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 300, rng.integers(1, 20))
    for bm_seq, md in [(128, 8), (32, 2), (7, 3), (1, 1)]:
        got = stg.ragged_tile_schedule(lens, bm_seq, md)
        want = orc.ragged_schedule(lens, bm_seq, md)
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g, w)


def test_ragged_schedule_workload_matches_oracle(stg, orc):
    """The ragged workload's own 64 lengths, at both group settings: the
    product's schedule (which the ragged parity tests take their triples
    from) equals the oracle's, entry by entry."""
    lens = stg_pkg.inputs.ragged()["seq_lens"]
    assert len(lens) == 64
    for bm_seq, md in [(128, 8), (32, 2)]:
        got = stg.ragged_tile_schedule(lens, bm_seq, md)
        want = orc.ragged_schedule(lens, bm_seq, md)
        assert len(got[0]) == len(want[0]) > 0
        for g, w in zip(got, want):
            np.testing.assert_array_equal(np.asarray(g, dtype=np.uint32), w)


def test_ragged_schedule_workload_count(stg):
    lens = stg_pkg.inputs.ragged()["seq_lens"]
    for bm_seq, md in [(128, 8), (32, 2)]:
        ri, dyn, mi = stg.ragged_tile_schedule(lens, bm_seq, md)
        assert len(ri) == md * int(sum(-(-int(L) // bm_seq) for L in lens))
        assert int(dyn.sum()) == md * int(lens.sum())


def _t(shape, dtype=0, data=0x1000, stride=None):
    d = StgTensor()
    d.data = data
    d.dtype = dtype
    d.rank = len(shape)
    st = stride or [int(np.prod(shape[i + 1:])) for i in range(len(shape))]
    for i in range(4):
        d.shape[i] = shape[i] if i < len(shape) else 1
        d.stride[i] = st[i] if i < len(shape) else 0
    return d


def _i64(vals):
    a = (ctypes.c_int64 * 4)()
    for i, v in enumerate(vals):
        a[i] = v
    return a


def test_gather_argument_errors(stg):
    lib = stg.load_library()
    a, out = _t([16, 8]), _t([8, 8])
    ts = _i64([4, 8])
    B = ctypes.byref
    assert lib.tile_gather(None, 0x10, 8, ts, None, 0, B(out), None) == 1
    assert b"null tensor" in lib.stg_last_error()
    assert lib.tile_gather(B(a), None, 8, ts, None, 0, B(out), None) == 1
    assert lib.tile_gather(B(a), 0x10, 7, ts, None, 0, B(out), None) == 1  # not a multiple of 4
    assert b"multiple" in lib.stg_last_error()
    assert lib.tile_gather(B(a), 0x10, 8, ts, None, 2, B(out), None) == 1  # axis out of range
    assert lib.tile_gather(B(a), 0x10, 12, ts, None, 0, B(out), None) == 1  # out shape mismatch
    assert lib.tile_gather(B(a), 0x10, 8, _i64([0, 8]), None, 0, B(out), None) == 1  # empty tile dim
    assert lib.tile_gather(B(_t([16, 8], dtype=9)), 0x10, 8, ts, None, 0, B(out), None) == 2  # dtype
    assert lib.tile_gather(B(_t([16, 8], dtype=1)), 0x10, 8, ts, None, 0, B(out), None) == 1  # dtype mismatch
    bad = _t([16, 8])
    bad.rank = 5
    assert lib.tile_gather(B(bad), 0x10, 8, ts, None, 0, B(out), None) == 1
    assert lib.tile_gather(B(_t([16, 8], data=0)), 0x10, 8, ts, None, 0, B(out), None) == 1  # null data
    neg = _t([16, 8], stride=[-8, 1])
    assert lib.tile_gather(B(neg), 0x10, 8, ts, None, 0, B(out), None) == 1
    assert lib.tile_gather(B(a), 0x10, 8, ts, _i64([1 << 50, 0]), 0, B(out), None) == 3  # offset range
    # extents whose product would overflow int64 (4 x 2^20 extents = 2^80
    # elements), and a single extent past 2^40: range errors, nothing launched
    huge = _t([1 << 20, 1 << 20, 1 << 20, 1 << 20], stride=[0, 0, 0, 1])
    assert lib.tile_gather(B(huge), 0x10, 8, _i64([4, 1, 1, 8]), None, 0, B(_t([8, 1, 1, 8])), None) == 3
    assert b"2^48" in lib.stg_last_error()
    assert lib.tile_gather(B(_t([1 << 41, 8], stride=[8, 1])), 0x10, 8, ts, None, 0, B(out), None) == 3
    # padding value not representable in the element type
    ai, oi = _t([16, 8], dtype=4), _t([8, 8], dtype=4)
    assert lib.tile_gather_masked(B(ai), 0x10, None, 8, ts, None, 0, 300.0, B(oi), None) == 1
    assert b"padding" in lib.stg_last_error()
    assert lib.tile_scatter_masked(B(a), 0x10, None, 8, ts, None, 0, None, None) == 1


def test_copy_argument_errors(stg):
    lib = stg.load_library()
    B = ctypes.byref
    assert lib.tile_copy_bounded(B(_t([4, 4, 4])), 2, 2, 0, 0, 0x10, None) == 1  # rank 3
    assert lib.tile_copy_bounded(B(_t([8, 8])), 0, 2, 0, 0, 0x10, None) == 1
    assert lib.tile_copy_bounded(B(_t([8, 8])), 2, 2, 0, 0, None, None) == 1  # null tile buffer
    assert lib.tile_copy_bounded(B(_t([8, 8])), 2, 2, -(1 << 41), 0, 0x10, None) == 3
    assert lib.tile_store_clipped(None, 2, 2, 0, 0, B(_t([8, 8])), None) == 1
    assert lib.tile_store_clipped(0x10, 2, 2, 0, 0, None, None) == 1
    # grids that are empty are a successful no-op without touching the GPU
    assert lib.tile_copy_bounded(B(_t([8, 8])), 2, 2, 8, 0, None, None) == 0
    # a grid whose tile buffer would exceed 2^48 elements: range error
    # (the array itself is within the descriptor limit of 2^48 elements)
    big = _t([1 << 24, 1 << 24], stride=[1 << 24, 1])
    assert lib.tile_copy_bounded(B(big), 1, 1, -(1 << 20), -(1 << 20), 0x10, None) == 3
    assert b"tile buffer" in lib.stg_last_error()


def test_ragged_argument_errors(stg):
    lib = stg.load_library()
    args = dict(src=0x10, dtype=1, total_rows=100, middle_dim=8, group=1, depth=128, BM=128, BN=128, col0=0,
                ri=0x10, dyn=0x10, mi=0x10, n=4, out=0x10)

    def call(**kw):
        a = dict(args, **kw)
        return lib.ragged_tile_load(a["src"], a["dtype"], a["total_rows"], a["middle_dim"], a["group"], a["depth"],
                                    a["BM"], a["BN"], a["col0"], a["ri"], a["dyn"], a["mi"], a["n"], a["out"], None)

    assert call(group=3) == 1  # BM % group
    assert b"multiple of group" in lib.stg_last_error()
    assert call(col0=128) == 1
    assert call(col0=-1) == 1
    assert call(dtype=11) == 2
    assert call(ri=None) == 1
    assert call(out=None) == 1
    assert call(middle_dim=0) == 1
    assert call(n=0, out=None) == 0  # nothing to do
    # packed rows too large for 32-bit tile offsets, factor products that
    # would overflow, and more than 2^40 rows: range errors
    assert call(middle_dim=1 << 20, group=1 << 10, BM=1 << 10) == 3
    assert call(middle_dim=(1 << 31) - 1, group=(1 << 14), depth=(1 << 31) - 1, BM=1 << 14) == 3
    assert call(total_rows=(1 << 41)) == 3
    n = ctypes.c_int64()
    assert lib.ragged_tile_schedule(None, 3, 4, 1, None, None, None, ctypes.byref(n)) == 1
    lens = np.array([3, -1], dtype=np.int64)
    assert lib.ragged_tile_schedule(lens.ctypes.data, 2, 4, 1, None, None, None, ctypes.byref(n)) == 1
    big = np.array([1 << 33, 5], dtype=np.int64)
    assert lib.ragged_tile_schedule(big.ctypes.data, 2, 1 << 30, 1, None, None, None, ctypes.byref(n)) == 3


def test_gemm_argument_errors(stg):
    lib = stg.load_library()
    # bad output dtype, strides below the row length, negative sizes
    assert lib.gemm_bounded(0x10, 8, 0x10, 8, 0x10, 8, 8, 8, 8, 3, None) in (1, 2)
    assert lib.gemm_bounded(0x10, 4, 0x10, 8, 0x10, 8, 8, 8, 8, 1, None) in (1, 2)
    assert lib.gemm_bounded(0x10, 8, 0x10, 8, 0x10, 8, -1, 8, 8, 1, None) in (1, 2)
    assert lib.gemm_bounded(None, 8, 0x10, 8, 0x10, 8, 8, 8, 8, 1, None) in (1, 2)


def test_binding_rejects_host_tensors(stg):
    import torch

    a = torch.zeros(4, 4)
    idx = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        stg.tile_gather(a, idx, (4, 4))


def test_trace_host_paths(stg):
    lib = stg.load_library()
    prev = stg.stg_trace_enable(False)
    assert stg.stg_trace_enable(False) is False
    assert stg.stg_trace_read() == []  # nothing launched: an empty log
    assert lib.stg_trace_read(3, None, None) < 0  # bad output arrays
    stg.stg_trace_enable(prev)


def test_ragged_store_argument_errors(stg):
    lib = stg.load_library()

    def call(**kw):
        a = dict(tiles=0x10, dtype=1, total_rows=100, middle_dim=8, group=1, depth=128, BM=128, BN=128, col0=0,
                 ri=0x10, dyn=0x10, mi=0x10, n=4, dst=0x10)
        a.update(kw)
        return lib.ragged_tile_store(a["tiles"], a["dtype"], a["total_rows"], a["middle_dim"], a["group"], a["depth"],
                                     a["BM"], a["BN"], a["col0"], a["ri"], a["dyn"], a["mi"], a["n"], a["dst"], None)

    assert call(group=3) == 1  # BM % group
    assert b"ragged_tile_store" in lib.stg_last_error()
    assert call(col0=128) == 1
    assert call(dtype=11) == 2
    assert call(tiles=None) == 1
    assert call(dst=None) == 1
    assert call(mi=None) == 1
    assert call(BN=0) == 1
    assert call(n=0, tiles=None, dst=None) == 0  # nothing to do
    assert call(BM=1 << 20, BN=1 << 10) == 3  # tile too large for the launch layout


def test_window_argument_errors_and_broken_promise(stg):
    lib = stg.load_library()
    B = ctypes.byref
    m = _t([64, 64], dtype=1)
    # step below 1
    assert lib.tile_copy_windows(B(m), 8, 8, 0, 8, 0, 0, 1, 0x10, None) == 1
    assert b"step" in lib.stg_last_error()
    assert lib.tile_store_windows(0x10, 8, 8, 8, -1, 0, 0, 1, B(m), None) == 1
    # check_bounds = 0 with a grid that leaves the array: rejected on the host, nothing launched
    assert lib.tile_copy_windows(B(m), 8, 8, 8, 8, -1, 0, 0, 0x10, None) == 1  # negative origin
    assert b"promises" in lib.stg_last_error()
    assert lib.tile_copy_windows(B(_t([63, 64], dtype=1)), 8, 8, 8, 8, 0, 0, 0, 0x10, None) == 1  # last row band short
    assert lib.tile_store_windows(0x10, 8, 8, 6, 8, 0, 0, 0, B(m), None) == 1  # windows at rows 60.. overhang
    assert lib.tile_copy_windows(B(m), 8, 8, 8, 8, 0, 0, 0, None, None) == 1  # promise holds: null buffer caught
    assert b"null" in lib.stg_last_error()
    # an empty grid is a successful no-op without touching the GPU
    assert lib.tile_copy_windows(B(m), 8, 8, 8, 8, 64, 0, 1, None, None) == 0


def test_gather_backward_workspace_query_and_errors(stg):
    lib = stg.load_library()
    B = ctypes.byref
    g = _t([1024, 256], dtype=0)
    ts = _i64([64, 256])
    # row layout, each part 256-byte aligned: segment offsets int32[R + 1],
    # term ids int32[n], (row, term) pairs uint64[n], the bucket-major count
    # table int32[L1] and its scan int32[L1 + 1], scan block sums, the list
    # of long segments' pieces uint64[n / 32 + 1] and its length, per-row
    # counters int32[R], hot-bucket flags int32[buckets], the hot slices'
    # list uint64[n / 16384 + n / 16384 + 1] and its length; R = 1024 rows
    # make 512 buckets of 2 rows, n = 4096 terms one chunk, so L1 = 512
    nbytes = lib.tile_gather_backward_workspace(B(g), 4096, ts, 0)
    assert nbytes == 4352 + 16384 + 32768 + 2048 + 2304 + 256 + 1280 + 256 + 4096 + 2048 + 256 + 256
    # gather along the last axis: atomics only, no workspace
    assert lib.tile_gather_backward_workspace(B(g), 4096, _i64([1024, 64]), 1) == 0
    assert lib.tile_gather_backward_workspace(B(g), 4096, ts, 2) < 0
    # unsupported gradient dtype; a workspace too small
    bf = _t([1024, 256], dtype=1)
    assert lib.tile_gather_backward(B(bf), 0x10, 4096, ts, None, 0, B(_t([4096, 256], dtype=1)), None, 0, None) == 2
    out = _t([4096, 256], dtype=0)
    assert lib.tile_gather_backward(B(g), 0x10, 4096, ts, None, 0, B(out), 0x1000, 1024, None) == 1
    assert b"workspace" in lib.stg_last_error()
    assert lib.tile_gather_backward(B(g), 0x10, 4096, ts, None, 0, B(out), 0x1001, 1 << 20, None) == 1  # alignment


def test_gemm_scaled_argument_errors(stg):
    lib = stg.load_library()

    def call(**kw):
        a = dict(A=0x10, fa=0, lda=64, sa=0x10, lds_a=2, B=0x10, fb=0, ldb=64, sb=0x10, lds_b=2, sf=0, block=32,
                 acc=None, ldacc=0, C=0x10, ldc=8, M=8, N=8, K=64)
        a.update(kw)
        return lib.gemm_scaled(a["A"], a["fa"], a["lda"], a["sa"], a["lds_a"], a["B"], a["fb"], a["ldb"], a["sb"],
                               a["lds_b"], a["sf"], a["block"], a["acc"], a["ldacc"], a["C"], a["ldc"], a["M"], a["N"],
                               a["K"], None)

    # e4m3 scales, blocks such as 16 or 96 and fp4 x fp8 pairs are supported
    # (general path); what remains an error fails in the host checks
    assert call(fa=7) == 2  # unknown operand format
    assert call(sf=5) == 2  # unknown scale format
    assert call(block=0) == 1
    assert call(fa=2, lda=31) == 1  # fp4 rows of 64 values need 32 bytes
    assert call(K=96, block=64) == 1  # K not a multiple of the block
    assert call(lda=32) == 1  # row stride shorter than the row
    assert call(C=None) == 1
    assert call(M=-1) == 1
    assert call(M=0) == 0  # nothing to do


def test_static_scratch_size_and_oversized_rejection(stg):
    """The static scratch size is the one stg.h declares, and a call needing
    more scratch than that fails with STG_ERR_RANGE in the host checks, before
    any HIP call (fake device pointers are never touched)."""
    m = re.search(r"#define\s+STG_STATIC_SCRATCH_BYTES\s+\((\d+)ll\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == stg_pkg.STATIC_SCRATCH_BYTES
    lib = stg.load_library()
    a = _t([1 << 22, 128])
    g = _t([1 << 24, 128], data=0x2000)
    rc = lib.tile_gather_backward_static(ctypes.byref(a), ctypes.c_void_p(0x3000), 1 << 24, _i64([64, 128]), None, 0,
                                         ctypes.byref(g), None)
    assert rc == 3 and b"static array" in lib.stg_last_error()


def test_prepare_capture_is_per_thread(stg):
    """prepare() records the entry-point calls made on its own thread only: a
    call from another host thread meanwhile is made, not recorded.  The
    recording is driven directly with a library function that needs no GPU
    (stg_tile_grid), so the check runs on the host."""
    import threading
    from scatter_tile_gather_amd import _binding as b

    b.load_library()
    seen = {}

    def other():
        seen["capture"] = b._capturing()
        try:  # made, not recorded: a non-zero return is raised as an error
            b._call("stg_tile_grid", 100, 0, 10)
            seen["made"] = False
        except b.StgError:
            seen["made"] = True

    b._TLS.capture = []
    try:
        t = threading.Thread(target=other)
        t.start()
        t.join()
        b._call("stg_tile_grid", 100, 0, 10)  # recorded here
        mine = list(b._TLS.capture)
    finally:
        b._TLS.capture = None
    assert seen == {"capture": None, "made": True}
    assert [name for name, _, _ in mine] == ["stg_tile_grid"]
    assert b._capturing() is None


def test_packed_descriptor_and_array_bytes(stg):
    """The binding passes stg_tensor and int64_t[4] arguments as packed bytes:
    the packing matches the structure's fields, the C side reads it (its
    argument checks see the packed rank, dtype and shape), and the cached
    shape arrays are zero-padded copies keyed by value."""
    from scatter_tile_gather_amd import _binding as b

    raw = b._DESC.pack(0x1000, 0, 2, 16, 8, 1, 1, 8, 1, 0, 0)
    d = StgTensor.from_buffer_copy(raw)
    assert (d.data, d.dtype, d.rank) == (0x1000, 0, 2)
    assert list(d.shape) == [16, 8, 1, 1] and list(d.stride) == [8, 1, 0, 0]
    lib = stg.load_library()
    out = b._DESC.pack(0x2000, 0, 2, 8, 8, 1, 1, 8, 1, 0, 0)
    ts = b._i64arr((4, 8))
    assert ts == (4).to_bytes(8, "little") + (8).to_bytes(8, "little") + bytes(16)
    assert b._i64arr([4, 8]) is ts and b._i64arr((np.int64(4), np.int64(8))) is ts
    with pytest.raises(ValueError):
        b._i64arr((1, 2, 3, 4, 5))
    assert lib.tile_gather(raw, 0x10, 12, ts, None, 0, out, None) == 1  # out rows != 12
    assert lib.tile_gather(b._DESC.pack(0x1000, 0, 5, 16, 8, 1, 1, 8, 1, 0, 0), 0x10, 8, ts, None, 0, out, None) == 1
    assert lib.tile_gather(b._DESC.pack(0x1000, 9, 2, 16, 8, 1, 1, 8, 1, 0, 0), 0x10, 8, ts, None, 0, out, None) == 2
    assert lib.tile_gather(raw, 0x10, 8, ts, b._i64arr((1 << 50, 0)), 0, out, None) == 3  # offset range


def test_gemm_scaled_workspace_query(stg):
    """gemm_scaled_workspace: 0 where the scaled MFMA runs (e8m0 scales,
    blocks of 32 * 2^k, one operand width) or where M or N is at most 256;
    otherwise bf16 (M, ceil(K/16)*16) plus (K, ceil(N/64)*64), each rounded up
    to 256 bytes; bad arguments give minus an error code."""
    up = lambda x: (x + 255) // 256 * 256
    q = stg.gemm_scaled_workspace
    assert q("e4m3", "e4m3", "e8m0", 32, 8191, 8193, 4096) == 0
    assert q("e2m1", "e2m1", "e8m0", 64, 1000, 1000, 4096) == 0
    assert q("e4m3", "e4m3", "e4m3", 16, 256, 8193, 4096) == 0
    assert q("e4m3", "e4m3", "e4m3", 16, 8191, 256, 4096) == 0
    assert q("e4m3", "e4m3", "e4m3", 16, 300, 300, 0) == 0
    assert q("e4m3", "e4m3", "e4m3", 16, 8191, 8193, 4096) == up(8191 * 4096 * 2) + up(4096 * 8256 * 2)
    assert q("e2m1", "e4m3", "e8m0", 32, 257, 259, 99 * 32) == up(257 * 3168 * 2) + up(3168 * 320 * 2)
    assert q("e4m3", "e5m2", "e8m0", 3, 300, 301, 99) == up(300 * 112 * 2) + up(99 * 320 * 2)
    lib = stg.load_library()
    assert lib.gemm_scaled_workspace(0, 0, 1, 16, 300, 300, 48) == q("e4m3", "e4m3", "e4m3", 16, 300, 300, 48)
    assert lib.gemm_scaled_workspace(7, 0, 1, 16, 300, 300, 64) == -2  # unknown format
    assert lib.gemm_scaled_workspace(0, 0, 1, 16, 300, 300, 48) > 0
    assert lib.gemm_scaled_workspace(0, 0, 1, 16, 300, 300, 41) == -1  # K not a multiple of the block
    assert lib.gemm_scaled_workspace(0, 0, 1, 0, 300, 300, 48) == -1
    assert lib.gemm_scaled_workspace(0, 0, 1, 16, -1, 300, 32) == -1
    with pytest.raises(stg.StgError):
        q("e4m3", "e4m3", "e4m3", 16, 300, 300, 41)


def test_eager_marshalling_module_is_built(stg):
    """The C++ marshalling module of eager tile_gather calls is built into the
    package, and it rejects host tensors before any device call, as the
    ctypes form does."""
    import torch

    from scatter_tile_gather_amd import _stg_fast

    with pytest.raises(ValueError, match="GPU tensor"):
        _stg_fast.tile_gather(0, torch.zeros(8, 4), torch.zeros(4, dtype=torch.int32), torch.zeros(4, 4), (4, 4),
                              None, 0, None)
    with pytest.raises(TypeError, match="torch tensor"):
        _stg_fast.tile_gather(0, [1.0], torch.zeros(4, dtype=torch.int32), torch.zeros(4, 4), (4, 4), None, 0, None)
