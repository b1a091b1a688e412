"""Invariances of the fast tier, bit for bit on the GPU (sgemm-bi 0.1.2 PyPI page,
"Determinism contracts": bit-identical results, the forward batch-invariant across M).

An output element's arithmetic involves only its own row of A, its own column of B and
the reduction length, and round-to-nearest-even is symmetric and scale-free, so:
  * permuting the rows of x (or dy for dx) permutes the output rows; permuting the
    columns of w permutes the output columns (fwd), permuting the rows of w permutes
    the columns of dx; for dw, permuting the columns of x or of dy permutes the rows
    or the columns of dw;
  * negating x (and the bias) negates y, and negating x negates dw, bit for bit with f32
    inputs; with bf16/f16 inputs the matrix instruction's accumulation is not symmetric
    under negation, and the outputs are at most one unit apart (recorded);
  * scaling x (and the bias) by 2^e scales y exactly when nothing over- or underflows;
  * a zero row of x gives the rounded bias (+0 without one);
  * dx(dy, w) equals fwd(dy, w^T materialised), and dw(x, dy) equals fwd(x^T
    materialised, dy) when the reduction over the batch is not split into chunks
    (reductions of fewer than 1024 rows are never split).
Shapes: ragged ones, and the GPT-2 MLP shapes at 8192 tokens."""
import numpy as np
import pytest

import synthetic as syn
from tests import pins
from tests.gpu_util import assert_bits_equal, bits, gpu_op

pytestmark = pytest.mark.gpu

SHAPES = [(67, 100, 45), (200, 320, 136), (513, 768, 1000), (8192, 768, 3072), (8192, 3072, 768)]
DTS = ("f32", "bf16", "f16")


def _perm(n, a, b):
    return np.array([(a * i + b) % n for i in range(n)])


def _inputs(dt, si, m, k, n):
    X = syn.normal(1400 + si, 0, (m, k), dt=dt)
    W = syn.normal(1400 + si, 1, (k, n), sigma=0.05, dt=dt)
    G = syn.normal(1400 + si, 3, (m, n), dt=dt)
    b = syn.normal(1400 + si, 2, (n,), sigma=0.1, dt=dt)
    return X, W, G, b


def _odd_coprime(n, start):
    a = start
    while np.gcd(a, n) != 1:
        a += 2
    return a


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{k}x{n}" for m, k, n in SHAPES])
def test_permutations(dt, shape):
    m, k, n = shape
    if dt == "f32" and m >= 8192:
        pytest.skip("f32 at the GPT-2 shapes is covered by the ragged shapes")
    X, W, G, b = _inputs(dt, SHAPES.index(shape), m, k, n)
    pr = _perm(m, _odd_coprime(m, 7), 3)
    pk = _perm(k, _odd_coprime(k, 11), 5)
    pn = _perm(n, _odd_coprime(n, 13), 1)
    c = np.ascontiguousarray
    print(f"fast permutations {dt} {shape}", flush=True)
    y = gpu_op("fwd", dt, X, W, b, tier="fast")
    assert_bits_equal(gpu_op("fwd", dt, c(X[pr]), W, b, tier="fast"), y[pr], "fwd rows")
    assert_bits_equal(gpu_op("fwd", dt, X, c(W[:, pn]), c(b[pn]), tier="fast"), y[:, pn], "fwd columns")
    gx = gpu_op("dx", dt, G, W, tier="fast")
    assert_bits_equal(gpu_op("dx", dt, c(G[pr]), W, tier="fast"), gx[pr], "dx rows")
    assert_bits_equal(gpu_op("dx", dt, G, c(W[pk]), tier="fast"), gx[:, pk], "dx columns")
    gw = gpu_op("dw", dt, X, G, tier="fast")
    assert_bits_equal(gpu_op("dw", dt, c(X[:, pk]), G, tier="fast"), gw[pk], "dw rows")
    assert_bits_equal(gpu_op("dw", dt, X, c(G[:, pn]), tier="fast"), gw[:, pn], "dw columns")


def _check_negation(neg, y, dt, what):
    """f32: -fast(-x) is fast(x) bit for bit. bf16/f16: the 32x32x16 matrix instruction's f32
    accumulation on gfx950 is not symmetric under negation, so there the outputs that differ are
    counted and their distance printed (both results are within the tier's tolerance of the
    oracle, which the parity tests check on their own)."""
    if dt == "f32":
        assert_bits_equal(neg, y, what)
        return
    a, b = pins.vals(neg, dt), pins.vals(y, dt)
    diff = bits(neg) != bits(y)
    n = int(diff.sum())
    if n:
        from tests.gpu_util import ulp
        d = np.abs(a[diff] - b[diff]) / ulp(np.maximum(np.abs(a[diff]), np.abs(b[diff])), dt)
        idx = np.argwhere(diff)[:4]
        print(f"  {what}: {n} of {diff.size} outputs differ; distance in units of the larger's ulp: max "
              f"{d.max():g}, mean {d.mean():g}; e.g. " +
              ", ".join(f"{tuple(int(v) for v in i)}: {b[tuple(i)]!r} vs {a[tuple(i)]!r}" for i in idx), flush=True)
    else:
        print(f"  {what}: identical", flush=True)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", SHAPES[:3] + SHAPES[3:4], ids=[f"{m}x{k}x{n}" for m, k, n in SHAPES[:4]])
def test_negation_scaling_zero_row(dt, shape):
    m, k, n = shape
    if dt == "f32" and m >= 8192:
        pytest.skip("f32 at the GPT-2 shapes is covered by the ragged shapes")
    X, W, G, b = _inputs(dt, SHAPES.index(shape), m, k, n)
    v = pins.vals
    print(f"fast negation / scaling {dt} {shape}", flush=True)
    y = gpu_op("fwd", dt, X, W, b, tier="fast")
    yn = gpu_op("fwd", dt, pins.stor(-v(X, dt), dt), W, pins.stor(-v(b, dt), dt), tier="fast")
    gw = gpu_op("dw", dt, X, G, tier="fast")
    gwn = gpu_op("dw", dt, pins.stor(-v(X, dt), dt), G, tier="fast")
    _check_negation(pins.stor(-v(yn, dt), dt), y, dt, f"fwd negation {dt} {shape}")
    _check_negation(pins.stor(-v(gwn, dt), dt), gw, dt, f"dw negation {dt} {shape}")
    gx = gpu_op("dx", dt, G, W, tier="fast")
    for e in ((3, -5) if dt != "f16" else (3,)):
        s = 2.0 ** e
        # compared where the unscaled output is a normal number of the dtype (f16 outputs below
        # 2^-14 are rounded on the fixed subnormal grid, which does not scale)
        ys = gpu_op("fwd", dt, pins.stor(v(X, dt) * s, dt), W, pins.stor(v(b, dt) * s, dt), tier="fast")
        keep = np.abs(v(y, dt)) > 2.0 ** -14
        assert_bits_equal(ys[keep], pins.stor(v(y, dt)[keep] * s, dt), f"fwd scaled by 2^{e}")
        gs = gpu_op("dx", dt, pins.stor(v(G, dt) * s, dt), W, tier="fast")
        keep = np.abs(v(gx, dt)) > 2.0 ** -14
        assert_bits_equal(gs[keep], pins.stor(v(gx, dt)[keep] * s, dt), f"dx scaled by 2^{e}")
    Xz = X.copy()
    Xz[m // 2] = 0
    yz = gpu_op("fwd", dt, Xz, W, b, tier="fast")
    assert_bits_equal(yz[m // 2], b, "zero row with bias")
    y0 = gpu_op("fwd", dt, Xz, W, tier="fast")
    assert not np.any(v(y0[m // 2], dt)), "zero row without bias"
    assert not np.any(np.signbit(v(y0[m // 2], dt))), "zero row gives +0"


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", [(67, 100, 45), (200, 320, 136), (960, 768, 640), (8192, 768, 3072)],
                         ids=["67x100x45", "200x320x136", "960x768x640", "8192x768x3072"])
def test_transpose_identities(dt, shape):
    m, k, n = shape
    if dt == "f32" and m >= 8192:
        pytest.skip("f32 at the GPT-2 shapes is covered by the ragged shapes")
    X, W, G, _ = _inputs(dt, 7, m, k, n)
    c = np.ascontiguousarray
    print(f"fast transposes {dt} {shape}", flush=True)
    assert_bits_equal(gpu_op("dx", dt, G, W, tier="fast"), gpu_op("fwd", dt, G, c(W.T), tier="fast"), "dx = fwd(dy, w^T)")
    if m < 1024:   # an unsplit reduction over the batch
        assert_bits_equal(gpu_op("dw", dt, X, G, tier="fast"), gpu_op("fwd", dt, c(X.T), G, tier="fast"),
                          "dw = fwd(x^T, dy)")
