"""GPU parity of gemm_scaled against the fp64 CPU oracle.

Tolerances, from the arithmetic and from a measured property of the scaled
MFMA:
 * fp4 (e2m1) operands: every product of two decoded values and two e8m0
   scales is exact in fp32, so the fp32 sum of K terms in any order is within
   gamma_K * sum|terms| (gamma_K = K u / (1 - K u), u = 2^-24) of the exact
   sum; one more rounding covers the accumulator input.
 * fp8 operands: v_mfma_scale_f32_32x32x64_f8f6f4 does not sum fp8 products
   at fp32 precision.  Over full-range random codes (64 <= K <= 2048, uniform
   and random scales) its error reached 2^-11.8 of sum|terms|, independent of
   K, i.e. it arises inside one 64-value instruction.  The bound used is
   (2^-10 + gamma_K) * sum|terms|: 4x that measurement, and still 64 times
   below the half-ulp (2^-4) that rounding an input to e4m3 costs.
 * Operands whose every partial sum is exact in 14 bits (values +-1, +-2,
   scales 2^-1 .. 2^2) must come out bit-exact in every format: that pins the
   operand layout and which scale meets which K block.
sum|terms| comes from the oracle applied to the sign-cleared codes.
"""
import numpy as np
import pytest
import torch

from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu

BITS = {"e4m3": 8, "e5m2": 8, "e2m1": 4}


def codes(rng, shape, fmt):
    """Random operand codes without NaN or infinity."""
    if fmt == "e2m1":
        return rng.integers(0, 16, shape).astype(np.uint8)
    c = rng.integers(0, 256, shape).astype(np.uint8)
    if fmt == "e4m3":
        c[(c & 0x7F) == 0x7F] = 0x38
    else:
        c[(c & 0x7C) == 0x7C] = 0x3C
    return c


def pack(c, fmt):
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4) if fmt == "e2m1" else c


def unsign(c, fmt):
    return c & (0x7 if fmt == "e2m1" else 0x7F)


def run_case(stg, orc, M, N, K, block, fa, fb, seed, with_acc=False, pad=0, scale_lo=118, scale_hi=136):
    rng = np.random.default_rng(seed)
    ca, cb = codes(rng, (M, K), fa), codes(rng, (N, K), fb)
    A, Bt = pack(ca, fa), pack(cb, fb)
    sa = rng.integers(scale_lo, scale_hi, (M, K // block)).astype(np.uint8)
    sb = rng.integers(scale_lo, scale_hi, (N, K // block)).astype(np.uint8)
    acc = rng.standard_normal((M, N)).astype(np.float32) if with_acc else None
    # padded operand rows (strides beyond the row), sentinel-filled output padding
    Ad = to_dev(np.pad(A, ((0, 0), (0, pad)), constant_values=0x5A))[:, :A.shape[1]]
    Bd = to_dev(np.pad(Bt, ((0, 0), (0, pad)), constant_values=0x5A))[:, :Bt.shape[1]]
    store = torch.full((M, N + pad), 7.0, dtype=torch.float32, device="cuda:0")
    stg.gemm_scaled(Ad, fa, to_dev(sa), Bd, fb, to_dev(sb), K, block,
                    acc=None if acc is None else to_dev(acc), out=store[:, :N])
    torch.cuda.synchronize()
    full = to_host(store)
    got = full[:, :N].astype(np.float64)
    want = orc.gemm_scaled_f64(A, fa, sa, Bt, fb, sb, K, block, acc=acc)
    mag = orc.gemm_scaled_f64(pack(unsign(ca, fa), fa), fa, sa, pack(unsign(cb, fb), fb), fb, sb, K, block)
    u = 2.0 ** -24
    gk = K * u / (1 - K * u) + (0.0 if fa == "e2m1" else 2.0 ** -10)
    tol = gk * mag + (np.abs(acc.astype(np.float64)) * u if acc is not None else 0) + 1e-30
    err = np.abs(got - want)
    assert np.all(err <= tol), (float((err - tol).max()), float(err.max()))
    if pad:
        assert np.all(full[:, N:] == 7.0)  # the output padding is never written
    return got


EXACT_CODES = {"e4m3": [0x38, 0x40, 0xB8, 0xC0], "e5m2": [0x3C, 0x40, 0xBC, 0xC0], "e2m1": [0x2, 0x4, 0xA, 0xC]}


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2"),
                                   ("e2m1", "e2m1")])
@pytest.mark.parametrize("shape,block", [((96, 96, 64), 32), ((257, 130, 1024), 32), ((33, 300, 512), 64),
                                         ((130, 70, 768), 256), ((70, 259, 256), 32), ((33, 8, 96), 32),
                                         ((260, 513, 128), 64)])
def test_scaled_exact(stg, orc, fa, fb, shape, block):
    """Values +-1, +-2 and scales 2^-1 .. 2^2: the result is exact, bit for bit.
    N = 259, 8 and 513 leave 3, 8 and 1 columns past the last whole 256-column
    tile, which go to the skinny kernel (N = 8: it alone)."""
    M, N, K = shape
    rng = np.random.default_rng(M * 7 + N + K + block)
    ca = np.array(EXACT_CODES[fa], np.uint8)[rng.integers(0, 4, (M, K))]
    cb = np.array(EXACT_CODES[fb], np.uint8)[rng.integers(0, 4, (N, K))]
    sa = rng.integers(126, 130, (M, K // block)).astype(np.uint8)
    sb = rng.integers(126, 130, (N, K // block)).astype(np.uint8)
    say("gemm_scaled exact", fa, fb, shape, "block", block)
    C = to_host(stg.gemm_scaled(to_dev(pack(ca, fa)), fa, to_dev(sa), to_dev(pack(cb, fb)), fb, to_dev(sb), K, block))
    np.testing.assert_array_equal(C.astype(np.float64),
                                  orc.gemm_scaled_f64(pack(ca, fa), fa, sa, pack(cb, fb), fb, sb, K, block))


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2"),
                                   ("e2m1", "e2m1")])
def test_scaled_formats_small(stg, orc, fa, fb):
    say("gemm_scaled formats", fa, fb, "(65, 97, 128) block 32")
    run_case(stg, orc, 65, 97, 128, 32, fa, fb, seed=1)


@pytest.mark.parametrize("shape", [(1, 1, 32), (31, 33, 64), (256, 256, 256), (257, 300, 96), (300, 257, 160),
                                   (513, 129, 384), (64, 520, 1024)])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_scaled_shapes(stg, orc, shape, fmt):
    M, N, K = shape
    say("gemm_scaled shape", shape, fmt)
    run_case(stg, orc, M, N, K, 32, fmt, fmt, seed=M + N + K)


@pytest.mark.parametrize("block", [32, 64, 128, 256])
@pytest.mark.parametrize("fmt", ["e5m2", "e2m1"])
def test_scaled_blocks_acc_and_padding(stg, orc, block, fmt):
    say("gemm_scaled block", block, fmt, "with acc and padded strides")
    run_case(stg, orc, 130, 270, 512, block, fmt, fmt, seed=block, with_acc=True, pad=7)


@pytest.mark.parametrize("fa,fb", [("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e2m1", "e2m1")])
def test_scaled_remainder_columns_random(stg, orc, fa, fb):
    """Full-range codes, accumulator input and padded strides with 5 columns
    past the last whole tile (the skinny kernel), scales per 64 values."""
    say("gemm_scaled remainder columns", fa, fb, "(131, 517, 320) block 64")
    run_case(stg, orc, 131, 517, 320, 64, fa, fb, seed=517, with_acc=True, pad=3)


def test_scaled_extreme_scales(stg, orc):
    """Scales far from 1 (2^-40 .. 2^40) on both operands."""
    say("gemm_scaled extreme scales")
    run_case(stg, orc, 96, 64, 256, 32, "e4m3", "e4m3", seed=7, scale_lo=87, scale_hi=167)


def test_scaled_k_zero_is_the_accumulator(stg, orc):
    rng = np.random.default_rng(3)
    acc = rng.standard_normal((5, 9)).astype(np.float32)
    z = torch.zeros((5, 1), dtype=torch.uint8, device="cuda:0")[:, :0]
    zb = torch.zeros((9, 1), dtype=torch.uint8, device="cuda:0")[:, :0]
    say("gemm_scaled K = 0")
    out = stg.gemm_scaled(z, "e4m3", z, zb, "e4m3", zb, 0, 32, acc=to_dev(acc))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(out), acc)


def test_scaled_large_sampled(stg, orc):
    """(4096, 4096, 4096) e4m3, block 32: sampled rows and columns, including
    the last tile rows and columns."""
    M = N = K = 4096
    rng = np.random.default_rng(11)
    ca, cb = codes(rng, (M, K), "e4m3"), codes(rng, (N, K), "e4m3")
    sa = rng.integers(120, 134, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 134, (N, K // 32)).astype(np.uint8)
    say("gemm_scaled large (4096,4096,4096) e4m3 sampled")
    C = to_host(stg.gemm_scaled(to_dev(ca), "e4m3", to_dev(sa), to_dev(cb), "e4m3", to_dev(sb), K, 32))
    rows = np.concatenate([np.arange(0, 64), np.arange(M - 64, M), rng.integers(0, M, 64)])
    cols = np.concatenate([np.arange(0, 64), np.arange(N - 64, N), rng.integers(0, N, 64)])
    want = orc.gemm_scaled_f64(ca[rows], "e4m3", sa[rows], cb[cols], "e4m3", sb[cols], K, 32)
    mag = orc.gemm_scaled_f64(ca[rows] & 0x7F, "e4m3", sa[rows], cb[cols] & 0x7F, "e4m3", sb[cols], K, 32)
    tol = (K * 2.0 ** -24 / (1 - K * 2.0 ** -24) + 2.0 ** -10) * mag + 1e-30
    err = np.abs(C[np.ix_(rows, cols)].astype(np.float64) - want)
    assert np.all(err <= tol), float((err - tol).max())


@pytest.mark.parametrize("base", [1, 3, 8, 15])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_scaled_unaligned_scale_views(stg, orc, base, fmt):
    """Scale matrices as views at every 16-byte phase with odd row strides:
    each row's bytes start at a different phase of its 16-byte aligned window.
    Operands +-1, +-2 and scales 2^-1 .. 2^2 keep the result exact."""
    M, N, K, block = 200, 150, 1024, 32
    nkb = K // block
    rng = np.random.default_rng(100 + base)
    ca = np.array(EXACT_CODES[fmt], np.uint8)[rng.integers(0, 4, (M, K))]
    cb = np.array(EXACT_CODES[fmt], np.uint8)[rng.integers(0, 4, (N, K))]
    sa_full = rng.integers(126, 130, (M, nkb + 2 * base + 1)).astype(np.uint8)
    sb_full = rng.integers(126, 130, (N, nkb + base + 3)).astype(np.uint8)
    sa, sb = sa_full[:, base:base + nkb], sb_full[:, base + 1:base + 1 + nkb]
    say("gemm_scaled unaligned scale views base", base, fmt, "strides", sa_full.shape[1], sb_full.shape[1])
    sad, sbd = to_dev(sa_full)[:, base:base + nkb], to_dev(sb_full)[:, base + 1:base + 1 + nkb]
    assert sad.data_ptr() % 16 == base % 16
    C = to_host(stg.gemm_scaled(to_dev(pack(ca, fmt)), fmt, sad, to_dev(pack(cb, fmt)), fmt, sbd, K, block))
    np.testing.assert_array_equal(C.astype(np.float64),
                                  orc.gemm_scaled_f64(pack(ca, fmt), fmt, sa, pack(cb, fmt), fmt, sb, K, block))


@pytest.mark.parametrize("K", [96, 160, 544, 640, 1056])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_scaled_packed_scales_nan_padding(stg, orc, K, fmt):
    """Scale rows 16-byte aligned (bases and row strides multiples of 16,
    32-value blocks: the packed-scale path) with every byte past K / 32 set
    to 0xFF, the e8m0 NaN: the groups of 8 (fp8) or 16 (fp4) blocks that run
    past K must not let those bytes reach the zero data there.  K = 544 and
    640 end inside a second group, 1056 inside a third.  Exact values."""
    M, N, block = 300, 600, 32
    nkb = K // block
    lds = (nkb + 15) // 16 * 16 + 16
    rng = np.random.default_rng(K + (7 if fmt == "e2m1" else 0))
    ca = np.array(EXACT_CODES[fmt], np.uint8)[rng.integers(0, 4, (M, K))]
    cb = np.array(EXACT_CODES[fmt], np.uint8)[rng.integers(0, 4, (N, K))]
    sa_full = np.full((M, lds), 0xFF, np.uint8)
    sb_full = np.full((N, lds), 0xFF, np.uint8)
    sa_full[:, :nkb] = rng.integers(126, 130, (M, nkb))
    sb_full[:, :nkb] = rng.integers(126, 130, (N, nkb))
    sad, sbd = to_dev(sa_full)[:, :nkb], to_dev(sb_full)[:, :nkb]
    assert sad.data_ptr() % 16 == 0 and sbd.data_ptr() % 16 == 0 and sad.stride(0) % 16 == 0
    say("gemm_scaled packed scales, NaN padding, K", K, fmt, "row stride", lds)
    C = to_host(stg.gemm_scaled(to_dev(pack(ca, fmt)), fmt, sad, to_dev(pack(cb, fmt)), fmt, sbd, K, block))
    np.testing.assert_array_equal(C.astype(np.float64),
                                  orc.gemm_scaled_f64(pack(ca, fmt), fmt, sa_full[:, :nkb], pack(cb, fmt), fmt,
                                                      sb_full[:, :nkb], K, block))


def test_scaled_output_may_alias_the_accumulator(stg, orc):
    M, N, K = 140, 300, 256
    rng = np.random.default_rng(77)
    ca, cb = codes(rng, (M, K), "e5m2"), codes(rng, (N, K), "e5m2")
    sa = rng.integers(124, 131, (M, K // 64)).astype(np.uint8)
    sb = rng.integers(124, 131, (N, K // 64)).astype(np.uint8)
    acc = rng.standard_normal((M, N)).astype(np.float32)
    say("gemm_scaled in place: out is acc")
    inout = to_dev(acc)
    stg.gemm_scaled(to_dev(ca), "e5m2", to_dev(sa), to_dev(cb), "e5m2", to_dev(sb), K, 64, acc=inout, out=inout)
    torch.cuda.synchronize()
    want = orc.gemm_scaled_f64(ca, "e5m2", sa, cb, "e5m2", sb, K, 64, acc=acc)
    mag = orc.gemm_scaled_f64(ca & 0x7F, "e5m2", sa, cb & 0x7F, "e5m2", sb, K, 64)
    u = 2.0 ** -24
    tol = (K * u / (1 - K * u) + 2.0 ** -10) * mag + np.abs(acc.astype(np.float64)) * u + 1e-30
    assert np.all(np.abs(to_host(inout).astype(np.float64) - want) <= tol)


@pytest.mark.parametrize("K,block", [(32, 32), (64, 32), (96, 32), (160, 32), (192, 64), (128, 128)])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_scaled_small_k_main_kernel(stg, orc, K, block, fmt):
    """K below, at and between whole stages (64 fp8 / 128 fp4 values) on a
    shape that runs the main kernel (two tile rows, three tile columns):
    partial first and last stages, windows of groups past K.  Exact values."""
    M, N = 300, 600
    rng = np.random.default_rng(K + block)
    ca = np.array(EXACT_CODES[fmt], np.uint8)[rng.integers(0, 4, (M, K))]
    cb = np.array(EXACT_CODES[fmt], np.uint8)[rng.integers(0, 4, (N, K))]
    sa = rng.integers(126, 130, (M, K // block)).astype(np.uint8)
    sb = rng.integers(126, 130, (N, K // block)).astype(np.uint8)
    say("gemm_scaled small K", K, "block", block, fmt)
    C = to_host(stg.gemm_scaled(to_dev(pack(ca, fmt)), fmt, to_dev(sa), to_dev(pack(cb, fmt)), fmt, to_dev(sb), K,
                                block))
    np.testing.assert_array_equal(C.astype(np.float64),
                                  orc.gemm_scaled_f64(pack(ca, fmt), fmt, sa, pack(cb, fmt), fmt, sb, K, block))


def test_scaled_binding_rejects_undersized_tensors(stg):
    """The C ABI cannot see allocation sizes; the binding checks that every
    tensor holds what M, N, K and block ask for before anything is launched."""
    u8 = lambda *shape: torch.zeros(shape, dtype=torch.uint8, device="cuda:0")
    A, Bt, sa, sb = u8(64, 128), u8(32, 128), u8(64, 4), u8(32, 4)
    stg.gemm_scaled(A, "e4m3", sa, Bt, "e4m3", sb, 128, 32)  # consistent: runs
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="hold K"):
        stg.gemm_scaled(A, "e4m3", sa, Bt, "e4m3", sb, 160, 32)
    with pytest.raises(ValueError, match="a_scale"):
        stg.gemm_scaled(A, "e4m3", u8(63, 4), Bt, "e4m3", sb, 128, 32)
    with pytest.raises(ValueError, match="a_scale"):
        stg.gemm_scaled(A, "e4m3", sa, Bt, "e4m3", u8(32, 3), 128, 32)
    with pytest.raises(ValueError, match="multiple of block"):
        stg.gemm_scaled(A, "e4m3", sa, Bt, "e4m3", sb, 100, 32)
    # fp4: 128 bytes hold 256 values
    stg.gemm_scaled(A, "e2m1", u8(64, 8), Bt, "e2m1", u8(32, 8), 256, 32)
    torch.cuda.synchronize()
