"""Correctly rounded tier on the GPU against the oracle, bit for bit: every op and dtype
on ragged multi-tile shapes (16-bit inputs: the 7-bit slices on the int8 and the 8-bit
slices on the bf16 matrix instructions, every pair of 7-bit slice counts, and the same
forced through the 23-bit float64 slices; f32: the 23-bit
slices), the same forced through the per-output superaccumulator path, wide exponent ranges and non-finite values (which take that path
by themselves), cancellation witnesses, permutation invariance, the column sum and f32
outputs, and sampled rows of the GPT-2 c_fc forward."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.gpu_util import assert_bits_equal, to_dev, to_host
from tests.pins import stor, vals, wide_f32

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1), (5, 37, 9), (64, 64, 64), (100, 70, 130), (130, 33, 65), (3, 300, 2)]


@pytest.fixture(autouse=True)
def _paths():
    import deterministic_invariant_gemm_det_amd as dg
    dg.det_gemm_debug_force_cr_fallback(0)
    yield
    dg.det_gemm_debug_force_cr_fallback(0)


def _gpu(op, dt, A, B, bias=None, out_dtype=None):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    a, b = to_dev(A, dt), to_dev(B, dt)
    if op == "fwd":
        y = dg.fwd(a, b, None if bias is None else to_dev(bias, dt), "cr")
    elif op == "dx":
        y = dg.dx(a, b, "cr")
    else:
        y = dg.dw(a, b, "cr", out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_host(y, "f32" if out_dtype is not None else dt)


def _operands(seed, op, dt, m, k, n, wide=False):
    sa = (m, k) if op != "dx" else (m, n)
    sb = (k, n) if op != "dw" else (m, n)
    if wide:
        A = syn.to_storage(vals(wide_f32(seed, 0, sa, -40, 40), "f32"), dt)
        B = syn.to_storage(vals(wide_f32(seed, 1, sb, -40, 40), "f32"), dt)
    else:
        A = syn.normal(seed, 0, sa, dt=dt)
        B = syn.normal(seed, 1, sb, sigma=0.5, dt=dt)
    bias = syn.normal(seed, 2, (n,), sigma=0.3, dt=dt) if op == "fwd" else None
    return A, B, bias


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["fwd", "dx", "dw"])
def test_cr_parity(op, dt):
    import deterministic_invariant_gemm_det_amd as dg
    for si, (m, k, n) in enumerate(SHAPES):
        for wide in (False, True):
            if wide and dt == "f16":
                continue   # f16's range is covered by the oracle pins; wide f32 exponents overflow it
            print(f"cr {op} {dt} {(m, k, n)} wide={wide}", flush=True)
            A, B, bias = _operands(1500 + si, op, dt, m, k, n, wide)
            want = oracle.gemm_cr(op, dt, A, B, m, k, n, bias=bias)
            got = _gpu(op, dt, A, B, bias)
            assert_bits_equal(got, want, f"cr {op} {dt} {(m, k, n)} wide={wide}")
            for path in ((1, 2) if dt != "f32" else (1,)):
                dg.det_gemm_debug_force_cr_fallback(path)
                got2 = _gpu(op, dt, A, B, bias)
                dg.det_gemm_debug_force_cr_fallback(0)
                assert_bits_equal(got2, want, f"cr path {path} {op} {dt} {(m, k, n)} wide={wide}")


def test_cr_nonfinite():
    dt, m, k, n = "f32", 70, 40, 66
    A, B, bias = _operands(1550, "fwd", dt, m, k, n)
    A = A.copy()
    A[3, 5] = np.inf
    A[10, 7] = np.nan
    B = B.copy()
    B[9, 20] = -np.inf
    want = oracle.gemm_cr("fwd", dt, A, B, m, k, n, bias=bias)
    got = _gpu("fwd", dt, A, B, bias)
    wn, gn = np.isnan(want), np.isnan(got)
    assert np.array_equal(wn, gn)
    assert_bits_equal(np.where(gn, 0, got).astype(np.float32), np.where(wn, 0, want).astype(np.float32), "non-finite")


def test_cr_cancellation_and_permutation():
    dt = "f32"
    # 2^100 + 1 - 2^100 in one reduction tile, per output row
    X = stor(np.array([[2.0 ** 100, 1.0, -(2.0 ** 100)] * 11]), dt)
    W = stor(np.ones((33, 3)), dt)
    got = _gpu("fwd", dt, X, W)
    assert np.all(got == 11.0), got
    # any permutation of the reduction index gives the same bits
    m, k, n = 40, 500, 70
    A, B, bias = _operands(1560, "fwd", "bf16", m, k, n)
    y = _gpu("fwd", "bf16", A, B, bias)
    perm = np.random.default_rng(1560).permutation(k)
    yp = _gpu("fwd", "bf16", np.ascontiguousarray(A[:, perm]), np.ascontiguousarray(B[perm, :]), bias)
    assert_bits_equal(yp, y, "permuted reduction")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_cr_column_sum_and_f32_out(dt):
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    from tests.gpu_util import torch_dtype
    for si, (m, n) in enumerate(((1, 1), (33, 70), (1000, 130), (4100, 65))):
        G = syn.normal(1570 + si, 3, (m, n), dt=dt)
        ones = syn.to_storage(np.ones((m, 1)), dt)
        for out_dt in sorted({dt, "f32"}):
            want = oracle.gemm_cr("dw", dt, ones, G, m, 1, n)[0]
            if out_dt != dt:   # the exact sum rounded to f32: round the oracle's f32-typed result
                want = oracle.gemm_cr("dw", "f32", syn.to_storage(np.ones((m, 1)), "f32"),
                                      syn.to_storage(vals(G, dt), "f32"), m, 1, n)[0]
            db = dg.db(to_dev(G, dt), "cr", out_dtype=torch_dtype(out_dt))
            torch.cuda.synchronize()
            assert_bits_equal(to_host(db, out_dt), want, f"cr db {dt}->{out_dt} {(m, n)}")
    if dt == "bf16":
        m, k, n = 300, 70, 90
        X = syn.normal(1580, 0, (m, k), dt=dt)
        G = syn.normal(1580, 3, (m, n), dt=dt)
        want = oracle.gemm_cr("dw", "f32", syn.to_storage(vals(X, dt), "f32"), syn.to_storage(vals(G, dt), "f32"),
                              m, k, n)
        assert_bits_equal(_gpu("dw", dt, X, G, out_dtype=torch.float32), want, "cr dw -> f32")


def test_cr_gpt2_c_fc_rows():
    """The GPT-2 c_fc forward (8192 x 768 -> 3072, bf16): sampled rows against the oracle."""
    import torch
    import deterministic_invariant_gemm_det_amd as dg
    dt, m, k, n = "bf16", 8192, 768, 3072
    X = syn.normal(42, syn.TID_X, (m, k), dt=dt)
    W = syn.normal(42, syn.TID_W, (k, n), sigma=0.02, dt=dt)
    b = syn.normal(42, syn.TID_B, (n,), sigma=0.1, dt=dt)
    rows = np.array([0, 1, 63, 64, 4095, 8191])
    want = oracle.gemm_cr("fwd", dt, X, W, m, k, n, bias=b, rows=rows)
    y = dg.fwd(to_dev(X, dt), to_dev(W, dt), to_dev(b, dt), "cr")
    torch.cuda.synchronize()
    assert_bits_equal(to_host(y, dt)[rows], want, "cr gpt2 c_fc rows")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_cr_two_slices(dt):
    """Rows and columns whose set bits span 24..46 positions take two slices on the sliced path
    (one tiny value per row of A and per column of B); the bits still match the oracle and the
    superaccumulator path."""
    import deterministic_invariant_gemm_det_amd as dg
    m, k, n = 130, 100, 70
    Av = vals(syn.normal(1590, 0, (m, k), dt=dt), dt)
    Bv = vals(syn.normal(1590, 1, (k, n), sigma=0.5, dt=dt), dt)
    Av[:, 7] = 1.5 * 2.0 ** -30
    Bv[11, :] = -1.25 * 2.0 ** -28
    A, B = stor(Av, dt), stor(Bv, dt)
    bias = syn.normal(1590, 2, (n,), dt=dt)
    want = oracle.gemm_cr("fwd", dt, A, B, m, k, n, bias=bias)
    assert_bits_equal(_gpu("fwd", dt, A, B, bias), want, f"two slices {dt}")
    dg.det_gemm_debug_force_cr_fallback(1)
    assert_bits_equal(_gpu("fwd", dt, A, B, bias), want, f"two slices {dt}, superaccumulator")
    dg.det_gemm_debug_force_cr_fallback(0)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_cr_eight_bit_slices(dt):
    """16-bit inputs on the 8-bit slice path: row blocks of A spanning three to five slices (one small
    value per row), columns of B spanning more (one small row of B), a reduction of several 256-index
    exact sums with the bias index, and in the same call a row block whose span exceeds five slices and
    an all-zero row block, which take the other paths; bits against the oracle and against paths 1 and 2."""
    import deterministic_invariant_gemm_det_amd as dg
    m, k, n = 270, 1100, 150
    Av = vals(syn.normal(1600, 0, (m, k), dt=dt), dt)
    Bv = vals(syn.normal(1600, 1, (k, n), sigma=0.5, dt=dt), dt)
    small = (2.0 ** -20, 2.0 ** -30, 2.0 ** -60) if dt == "bf16" else (2.0 ** -12, 2.0 ** -18, 2.0 ** -24)
    Av[0:64, 5] = 1.5 * small[0]
    Av[64:128, 9] = -1.25 * small[1]
    if dt == "bf16":
        Av[128:192, 3] = small[2]   # beyond five slices: the 23-bit path or the superaccumulator
    Av[192:256, :] = 0.0
    Bv[7, :] = -1.75 * small[0]
    A, B = stor(Av, dt), stor(Bv, dt)
    bias = syn.normal(1600, 2, (n,), sigma=0.3, dt=dt)
    want = oracle.gemm_cr("fwd", dt, A, B, m, k, n, bias=bias)
    assert_bits_equal(_gpu("fwd", dt, A, B, bias), want, f"8-bit slices {dt}")
    for path in (2, 1):
        dg.det_gemm_debug_force_cr_fallback(path)
        assert_bits_equal(_gpu("fwd", dt, A, B, bias), want, f"8-bit slices {dt}, path {path}")
        dg.det_gemm_debug_force_cr_fallback(0)
    # the weight gradient of the same operands (reduction over 270 rows, reduction-major operands)
    G = stor(vals(syn.normal(1601, 3, (m, n), dt=dt), dt), dt)
    want = oracle.gemm_cr("dw", dt, A, G, m, k, n)
    assert_bits_equal(_gpu("dw", dt, A, G), want, f"8-bit slices dw {dt}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_cr_seven_bit_slice_counts(dt):
    """16-bit inputs on the 7-bit slice (int8) path, every pair of slice counts in one call: row
    block i of A (i = 0..4) spans 7 i + 6 bit positions (small odd integers times 2^-24 and one
    value 65 * 2^(7 i - 24) per row), so it needs i + 1 slices, and column block j of B likewise
    j + 1, with a ragged sixth column block of three; then a reduction longer than one exact int32
    sum (16384 indices). Bits against the oracle and against the 23-bit path."""
    import deterministic_invariant_gemm_det_amd as dg

    def ints(seed, which, shape):
        v = vals(syn.normal(seed, which, shape, dt="f32"), "f32")
        return np.clip(np.rint(v * 40.0), -127, 127)

    m, k, n = 320, 300, 330
    ia, ib = ints(1610, 0, (m, k)), ints(1610, 1, (k, n))
    ia[:, 1] = 3.0
    ib[1, :] = -3.0
    for i in range(5):
        ia[64 * i:64 * (i + 1), 0] = 65.0 * 2.0 ** (7 * i)
    for j in range(6):
        ib[0, 64 * j:64 * (j + 1)] = -65.0 * 2.0 ** (7 * (j if j < 5 else 2))
    A, B = stor(ia * 2.0 ** -24, dt), stor(ib * 2.0 ** -24, dt)
    want = oracle.gemm_cr("fwd", dt, A, B, m, k, n)
    assert_bits_equal(_gpu("fwd", dt, A, B), want, f"7-bit slice counts {dt}")
    dg.det_gemm_debug_force_cr_fallback(2)
    assert_bits_equal(_gpu("fwd", dt, A, B), want, f"7-bit slice counts {dt}, path 2")
    dg.det_gemm_debug_force_cr_fallback(0)
    # two exact int32 sums per class: a reduction of 16384 + 200 indices, four and five slices
    m, k, n = 64, 16384 + 200, 96
    ia, ib = ints(1611, 0, (m, k)), ints(1611, 1, (k, n))
    ia[:, 1] = 1.0
    ib[1, :] = 1.0
    ia[:, 0] = 127.0 * 2.0 ** 21
    ib[0, :] = -127.0 * 2.0 ** 28
    A, B = stor(ia * 2.0 ** -24, dt), stor(ib * 2.0 ** -24, dt)
    want = oracle.gemm_cr("fwd", dt, A, B, m, k, n)
    assert_bits_equal(_gpu("fwd", dt, A, B), want, f"7-bit slices, long reduction {dt}")


def test_cr_many_tiles_mixed():
    """More than four 64 x 64 tiles per compute unit (the int8 path's workgroups then take several
    tiles each and stage a tile's first slices during the previous tile's last stage): row blocks
    of A with one to five slices, an all-zero row block, a row block past five slices and a column
    block of B with a non-finite value mixed over 33 x 33 tiles with ragged edges and a bias.
    Every output against the 23-bit path and the superaccumulator, sampled rows against the oracle."""
    import deterministic_invariant_gemm_det_amd as dg
    dt = "bf16"
    m, k, n = 64 * 32 + 37, 300, 64 * 32 + 5
    v = vals(syn.normal(1620, 0, (m, k), dt="f32"), "f32")
    ia = np.clip(np.rint(v * 40.0), -127, 127)
    ia[:, 1] = 3.0
    for i in range(m // 64 + 1):
        ia[64 * i:64 * (i + 1), 0] = 65.0 * 2.0 ** (7 * (i % 5))
    ia[64 * 7:64 * 8, :] = 0.0                  # all zero: the zero path
    ia[64 * 11:64 * 12, 2] = 2.0 ** 40          # six slices: another path
    Bv = vals(syn.normal(1620, 1, (k, n), sigma=0.5, dt=dt), dt)
    Bv[5, 64 * 9 + 3] = np.inf                  # non-finite: the superaccumulator
    A, B = stor(ia * 2.0 ** -24, dt), stor(Bv, dt)
    bias = syn.normal(1620, 2, (n,), sigma=0.3, dt=dt)
    got = _gpu("fwd", dt, A, B, bias)
    for path in (2, 1):
        dg.det_gemm_debug_force_cr_fallback(path)
        assert_bits_equal(got, _gpu("fwd", dt, A, B, bias), f"many tiles, against path {path}")
        dg.det_gemm_debug_force_cr_fallback(0)
    rows = np.array([0, 1, 63, 64, 64 * 7 + 5, 64 * 11 + 9, 64 * 16 + 31, 64 * 25 + 2, m - 1])
    want = oracle.gemm_cr("fwd", dt, A, B, m, k, n, bias=bias, rows=rows)
    # a NaN's sign and payload are not part of the result (as in test_cr_nonfinite): positions only
    def nan16(b):
        return ((b & 0x7f80) == 0x7f80) & ((b & 0x7f) != 0)
    g = got[rows]
    assert np.array_equal(nan16(g), nan16(want)) and nan16(want).any()
    assert_bits_equal(np.where(nan16(g), 0, g).astype(np.uint16), np.where(nan16(want), 0, want).astype(np.uint16),
                      "many tiles, sampled rows")


def test_cr_many_tiles_long_reduction():
    """The int8 path's persistent form with more than one exact int32 sum per class: 32 x 32 tiles of
    64 x 64 over a reduction of 16384 + 136 indices (small integers and one large value per row and
    column, five slices a side). Every output against the 23-bit path, sampled rows against the oracle."""
    import deterministic_invariant_gemm_det_amd as dg
    dt = "bf16"
    m, k, n = 64 * 32, 16384 + 136, 64 * 32
    ia = np.clip(np.rint(vals(syn.normal(1630, 0, (m, k), dt="f32"), "f32") * 40.0), -127, 127)
    ib = np.clip(np.rint(vals(syn.normal(1630, 1, (k, n), dt="f32"), "f32") * 40.0), -127, 127)
    ia[:, 1] = 1.0
    ib[1, :] = -1.0
    ia[:, 0] = 127.0 * 2.0 ** 28
    ib[0, :] = 127.0 * 2.0 ** 28
    A, B = stor(ia * 2.0 ** -24, dt), stor(ib * 2.0 ** -24, dt)
    got = _gpu("fwd", dt, A, B)
    dg.det_gemm_debug_force_cr_fallback(2)
    assert_bits_equal(got, _gpu("fwd", dt, A, B), "many tiles, long reduction, against path 2")
    dg.det_gemm_debug_force_cr_fallback(0)
    rows = np.array([0, 700, m - 1])
    want = oracle.gemm_cr("fwd", dt, A, B, m, k, n, rows=rows)
    assert_bits_equal(got[rows], want, "many tiles, long reduction, sampled rows")
